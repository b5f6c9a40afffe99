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


def test_kernel_source_hash_is_stable_and_covers_the_kernels():
    sys.path.insert(0, ROOT)
    import bench
    h = bench.kernel_source_hash()
    assert h == bench.kernel_source_hash() and len(h) == 16
