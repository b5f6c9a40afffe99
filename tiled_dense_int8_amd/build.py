"""Build libtdi8.so (gfx950) in-tree with hipcc.

One object per tile configuration (instantiate.hip compiled with
-DTDI8_CFG=<id>), plus the host selection and the C-ABI dispatcher, linked
into tiled_dense_int8_amd/libtdi8.so.  Objects go to _build/ at the repo root.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtdi8.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions are not wanted in any kernel of this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
]


def config_ids() -> list[int]:
    text = open(os.path.join(CSRC, "configs.h")).read()
    return [int(m) for m in re.findall(r"^\s*X\((\d+),", text, flags=re.M)]


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-3:]))


def build(jobs: int | None = None, verbose: bool = False, extra_flags: list[str] | None = None,
          out: str | None = None, build_dir: str | None = None) -> str:
    """Compile every configuration and link the library (default: in-tree libtdi8.so)."""
    out = out or LIB
    bdir = build_dir or BUILD
    flags = FLAGS + list(extra_flags or [])
    os.makedirs(bdir, exist_ok=True)
    jobs = jobs or min(16, os.cpu_count() or 4)
    units = []
    for cid in config_ids():
        obj = os.path.join(bdir, f"cfg{cid}.o")
        units.append([HIPCC, *flags, f"-DTDI8_CFG={cid}", "-c",
                      os.path.join(CSRC, "instantiate.hip"), "-o", obj])
    units.append([HIPCC, *flags, "-x", "hip", "-c", os.path.join(CSRC, "abi.cpp"),
                  "-o", os.path.join(bdir, "abi.o")])
    units.append([HIPCC, *flags, "-x", "hip", "-c", os.path.join(CSRC, "selector.cpp"),
                  "-o", os.path.join(bdir, "selector.o")])
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(_run, units))
    objs = [u[u.index("-o") + 1] for u in units]
    tmp = out + ".tmp%d" % os.getpid()
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
