"""Host-side checks of bench.py's contract that need no GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_kernel_code_hash_is_the_hash_of_the_built_code_objects():
    """The counter summaries are matched to the library by the hash of its
    GPU code: it is the SHA-256 of the configurations' gfx950 code objects,
    and the instrumented build, whose kernels differ, reports another."""
    import ctypes
    import hashlib
    sys.path.insert(0, ROOT)
    import bench
    h = bench.kernel_code_hash()
    assert h == bench.kernel_code_hash() and len(h) == 16 and int(h, 16) >= 0
    build = os.path.join(ROOT, "_build")
    sys.path.insert(0, os.path.join(ROOT, "tiled_dense_int8_amd"))
    import build as b
    cos = [os.path.join(build, f"cfg{cid}.o.co") for cid in b.config_ids()]
    if all(os.path.exists(c) for c in cos):
        d = hashlib.sha256()
        for c in cos:
            d.update(open(c, "rb").read())
        assert d.hexdigest()[:16] == h
    stamps = ctypes.CDLL(os.path.join(ROOT, "tiled_dense_int8_amd", "libtdi8_stamps.so"))
    stamps.tdi8_kernel_code_hash.restype = ctypes.c_char_p
    assert stamps.tdi8_kernel_code_hash().decode() != h
