"""Build libtdi8.so (gfx950) in-tree with hipcc.

One object per tile configuration (instantiate.hip compiled with
-DTDI8_CFG=<id>), plus the host selection and the C-ABI dispatcher, linked
into tiled_dense_int8_amd/libtdi8.so.  Objects go to _build/ at the repo root.

Between compiling and linking, the register and LDS use of every
configuration's column-major kernel (the one the selection's occupancy is
taken on) is read from the AMDGPU metadata note of the gfx950 code object
this build just produced, and compiled into the library as a table
(_build/kernel_resources.cpp): tile_config_info reports it.  The same file
carries the SHA-256 of those code objects (tdi8_kernel_code_hash).

The library build also produces libtdi8_ceilings.so (roofline calibration
kernels) and libtdi8_stamps.so: the same sources compiled with TDI8_STAMPS,
whose kernels write per-block timelines (include/tdi8_stamps.h); its
objects go to _build/stamps/.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import re
import subprocess
import sys

import yaml

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtdi8.so")
CEILINGS_LIB = os.path.join(PKG, "libtdi8_ceilings.so")  # roofline calibration kernels (bench.py --ceilings)
STAMPS_LIB = os.path.join(PKG, "libtdi8_stamps.so")      # block timelines (bench.py --stamps)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
LLVM_BIN = "/opt/rocm/llvm/bin"
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


def config_params() -> dict[int, tuple[int, ...]]:
    """id -> (family, MF, WM, WN, WK, MT, NT, BK, ST) from configs.h."""
    text = open(os.path.join(CSRC, "configs.h")).read()
    out = {}
    for m in re.finditer(r"^\s*X\(([\d,\s]+)\)", text, flags=re.M):
        v = [int(x) for x in m.group(1).split(",")]
        out[v[0]] = tuple(v[1:])
    return out


def _run(cmd: list[str]) -> str:
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd[-3:]))
    return r.stdout


def occupancy_kernel_symbol(params: tuple[int, ...]) -> str:
    """Mangled name of a configuration's column-major-B unpredicated kernel
    (kernel_table.h: kernel[1][1]), whose resources set its occupancy."""
    fam, mf, wm, wn, wk, mt, nt, bk, st = params
    if fam == 0:
        args = "".join(f"Li{v}E" for v in (mf, wm, wn, mt, nt, bk, st)) + "Lb0ELb0ELb0E"
        return f"_ZN4tdi824gemm_rc_pipelined_kernelI{args}EEvNS_8GemmArgsE"
    args = "".join(f"Li{v}E" for v in (mt, nt, wk, bk))
    return f"_ZN4tdi822gemm_skinny_lds_kernelI{args}EEvNS_8GemmArgsE"


def code_object_path(obj: str, work: str) -> str:
    return os.path.join(work, os.path.basename(obj) + ".co")


def code_object_kernels(obj: str, work: str) -> dict[str, dict]:
    """Kernel name -> metadata (.vgpr_count, .agpr_count, ...) of the gfx950
    code object embedded in a host object built here (the code object is left
    at code_object_path(obj, work))."""
    fatbin = os.path.join(work, os.path.basename(obj) + ".fatbin")
    co = code_object_path(obj, work)
    _run([os.path.join(LLVM_BIN, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fatbin}", obj,
          os.path.join(work, os.path.basename(obj) + ".stripped")])
    _run([os.path.join(LLVM_BIN, "clang-offload-bundler"), "--unbundle", "--type=o",
          f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}", f"--input={fatbin}", f"--output={co}"])
    notes = _run([os.path.join(LLVM_BIN, "llvm-readelf"), "--notes", co])
    start = notes.index("---")
    end = notes.index("\n...", start)
    meta = yaml.safe_load(notes[start:end])
    return {k[".name"]: k for k in meta["amdhsa.kernels"]}


def write_resource_table(objs: dict[int, str], bdir: str) -> str:
    """Generate the C++ table of per-configuration kernel resources."""
    params = config_params()
    rows = []
    code = hashlib.sha256()
    for cid in sorted(params):
        kernels = code_object_kernels(objs[cid], bdir)
        sym = occupancy_kernel_symbol(params[cid])
        if sym not in kernels:
            raise RuntimeError(f"configuration {cid}: kernel {sym} not found in {objs[cid]}")
        k = kernels[sym]
        with open(code_object_path(objs[cid], bdir), "rb") as f:
            code.update(f.read())
        rows.append(f"    {{{k['.vgpr_count']}, {k['.agpr_count']}, {k['.sgpr_count']}, "
                    f"{k['.group_segment_fixed_size']}, {k['.private_segment_fixed_size']}}},  // {cid}")
    src = os.path.join(bdir, "kernel_resources.cpp")
    text = ("// Generated by tiled_dense_int8_amd/build.py from the AMDGPU metadata of the\n"
            "// gfx950 code objects of this build: resources of each configuration's\n"
            "// column-major-B unpredicated kernel.\n"
            '#include "kernel_table.h"\n\nnamespace tdi8 {\n\n'
            "const KernelResources kKernelResources[TDI8_NUM_CONFIGS] = {\n" + "\n".join(rows) +
            "\n};\n\n}  // namespace tdi8\n\n"
            "// SHA-256 of the code objects of every configuration, in id order.\n"
            'extern "C" const char *tdi8_kernel_code_hash(void) { return "' + code.hexdigest()[:16] + '"; }\n')
    with open(src, "w") as f:
        f.write(text)
    return src


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
    ceil_obj = os.path.join(bdir, "ceilings.o")
    ceil_unit = [HIPCC, *flags, "-c", os.path.join(CSRC, "ceilings.hip"), "-o", ceil_obj]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(_run, units + ([ceil_unit] if out == LIB else [])))
    objs = [u[u.index("-o") + 1] for u in units]
    res_src = write_resource_table({cid: os.path.join(bdir, f"cfg{cid}.o") for cid in config_ids()}, bdir)
    res_obj = os.path.join(bdir, "kernel_resources.o")
    _run([HIPCC, *flags, "-c", res_src, "-o", res_obj])
    objs.append(res_obj)
    tmp = out + ".tmp%d" % os.getpid()
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, out)
    if out == LIB:
        tmp = CEILINGS_LIB + ".tmp%d" % os.getpid()
        _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", ceil_obj, "-o", tmp])
        os.replace(tmp, CEILINGS_LIB)
        build(jobs, verbose, list(extra_flags or []) + ["-DTDI8_STAMPS"], STAMPS_LIB, os.path.join(bdir, "stamps"))
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
