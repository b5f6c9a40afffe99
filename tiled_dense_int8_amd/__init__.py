"""Python binding of libtdi8.so, the gfx950 tiled int8 GEMM library.

Argument marshalling only: every step of the product runs in the library's
HIP kernels (C ABI in include/tdi8.h).  The names mirror the C entry points;
``gemm`` is a convenience wrapper that takes torch tensors, whose only role
is device memory and the current stream.

There is no fallback: if libtdi8.so is missing or fails to load, importing
this package raises.  Build it with ``python tiled_dense_int8_amd/build.py``
(or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads torch's HIP runtime first, so the library binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtdi8.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with tiled_dense_int8_amd/build.py")
_lib = ctypes.CDLL(LIB_PATH)

OK = 0
ERR_INVALID_VALUE = -1
ERR_NULL_POINTER = -2
ERR_ALIASING = -3
ERR_UNSUPPORTED_DEVICE = -4
ERR_BAD_CONFIG = -5
ERR_HIP = -6

ROUTE_GENERAL, ROUTE_FALLBACK, ROUTE_SKINNY = 0, 1, 2


class TileConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "id", "family", "mfma_m", "mfma_n", "mfma_k", "waves_m", "waves_n", "waves_k",
        "m_tiles", "n_tiles", "block_m", "block_n", "block_k", "stages", "threads", "lds_bytes",
        "vgprs", "agprs", "blocks_per_cu", "reuse1_id", "excluded", "sgprs")]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


class HwInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "num_cu", "max_threads_per_block", "min_active_threads", "skinny_max_m")]


class Selection(ctypes.Structure):
    _fields_ = [("id", ctypes.c_int), ("route", ctypes.c_int), ("survivors", ctypes.c_int * 5)]


FORM_NONE, FORM_PREDICATED, FORM_PIPELINED, FORM_PIPELINED_EDGE, FORM_SPLIT, FORM_SPLIT_EDGE, \
    FORM_SKINNY_DMA, FORM_SKINNY_PREDICATED, FORM_SKINNY_ROW_GROUPS, FORM_PREDICATED_PREFETCH, \
    FORM_PERSISTENT = range(11)


class Plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "config_id", "form", "splits", "kernels", "grid_x", "grid_y", "threads")]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


_i, _p = ctypes.c_int, ctypes.c_void_p
_GEMM_ARGS = [_i, _i, _i, _p, _i, _p, _i, _p, _i, _p]
_SIGNATURES = {
    "gemm_s8s8s32": (_i, _GEMM_ARGS),
    "gemm_s8s8s32_bt": (_i, _GEMM_ARGS),
    "gemm_s8s8s32_with_config": (_i, [_i, _i] + _GEMM_ARGS),
    "gemm_s8s8s32_persistent": (_i, [_i, _i] + _GEMM_ARGS[:-1] + [_i, _GEMM_ARGS[-1]]),
    "select_tile_config": (_i, [_i, _i, _i]),
    "tile_config_count": (_i, []),
    "tile_config_info": (_i, [_i, ctypes.POINTER(TileConfig)]),
    "tile_config_split_k": (_i, [_i, _i, _i, _i, _i]),
    "gemm_plan": (_i, [_i, _i, _i, _i, _i, _p, _i, _p, _i, _p, _i, ctypes.POINTER(Plan)]),
    "select_tile_config_for": (_i, [_i, _i, _i, ctypes.POINTER(HwInfo), ctypes.POINTER(_i),
                                    ctypes.POINTER(Selection)]),
    "tdi8_validate": (_i, [_i, _i, _i, _i, _p, _i, _p, _i, _p, _i]),
    "conv2d_s8s8s32_nhwc": (_i, [_i] * 13 + [_p, _p, _p, _p]),
    "conv2d_s8s8s32_nhwc_with_config": (_i, [_i] * 14 + [_p, _p, _p, _p]),
    "conv2d_select_config": (_i, [_i] * 13),
    "conv2d_output_extent": (_i, [_i] * 5),
    "conv2d_validate": (_i, [_i] * 13 + [_p, _p, _p]),
    "tdi8_status_string": (ctypes.c_char_p, [_i]),
    "tdi8_last_hip_error": (_i, []),
    "tdi8_kernel_code_hash": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _SIGNATURES.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGNATURES)


def load_library(path: str) -> ctypes.CDLL:
    """Another build of the same C ABI (the instrumented libtdi8_stamps.so),
    loaded beside libtdi8.so with the same signatures; its functions take the
    arguments of the module-level ones of the same name."""
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


class TDI8Error(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        msg = tdi8_status_string(status)
        if status == ERR_HIP:
            msg += f" (hipError_t {tdi8_last_hip_error()})"
        super().__init__(f"tdi8 status {status}: {msg}")


INT_MAX = 2 ** 31 - 1


def _int32(**vals) -> None:
    """The C entry points take int arguments; ctypes would wrap a larger
    Python int silently (2**32 + 5 arrives as 5), so refuse it here."""
    for name, v in vals.items():
        if not -2 ** 31 <= int(v) <= INT_MAX:
            raise ValueError(f"{name} = {v} does not fit the library's int arguments (|value| < 2**31)")


# ----- the C entry points, same names and arguments -------------------------------

def gemm_s8s8s32(M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    _int32(M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=ldc)
    return _lib.gemm_s8s8s32(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_s8s8s32_bt(M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    _int32(M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=ldc)
    return _lib.gemm_s8s8s32_bt(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_s8s8s32_with_config(config_id, b_col_major, M, N, K, A, lda, B, ldb, C, ldc, stream=0) -> int:
    _int32(config_id=config_id, M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=ldc)
    return _lib.gemm_s8s8s32_with_config(config_id, 1 if b_col_major else 0, M, N, K, A, lda, B, ldb,
                                         C, ldc, stream)


def gemm_s8s8s32_persistent(config_id, b_col_major, M, N, K, A, lda, B, ldb, C, ldc, blocks=0, stream=0) -> int:
    _int32(config_id=config_id, M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=ldc, blocks=blocks)
    return _lib.gemm_s8s8s32_persistent(config_id, 1 if b_col_major else 0, M, N, K, A, lda, B, ldb,
                                        C, ldc, blocks, stream)


def gemm_plan(config_id, b_col_major, M, N, K, A, lda, B, ldb, C, ldc) -> Plan:
    """What the gemm call with these arguments would enqueue (config_id -1:
    the selected configuration); raises TDI8Error on a bad argument."""
    _int32(config_id=config_id, M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=ldc)
    out = Plan()
    st = _lib.gemm_plan(config_id, 1 if b_col_major else 0, M, N, K, A, lda, B, ldb, C, ldc,
                        ctypes.byref(out))
    if st != OK:
        raise TDI8Error(st)
    return out


def select_tile_config(M, N, K) -> int:
    _int32(M=M, N=N, K=K)
    return _lib.select_tile_config(M, N, K)


def tile_config_split_k(config_id, M, N, K, num_cu) -> int:
    _int32(config_id=config_id, M=M, N=N, K=K, num_cu=num_cu)
    return _lib.tile_config_split_k(config_id, M, N, K, num_cu)


def tile_config_count() -> int:
    return _lib.tile_config_count()


def tile_config_info(config_id: int) -> TileConfig:
    out = TileConfig()
    st = _lib.tile_config_info(config_id, ctypes.byref(out))
    if st != OK:
        raise TDI8Error(st)
    return out


def select_tile_config_for(M, N, K, hw: HwInfo, blocks_per_cu) -> Selection:
    _int32(M=M, N=N, K=K)
    arr = (ctypes.c_int * tile_config_count())(*blocks_per_cu)
    out = Selection()
    st = _lib.select_tile_config_for(M, N, K, ctypes.byref(hw), arr, ctypes.byref(out))
    if st < 0:
        raise TDI8Error(st)
    return out


def tdi8_validate(b_col_major, M, N, K, A, lda, B, ldb, C, ldc) -> int:
    _int32(M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=ldc)
    return _lib.tdi8_validate(1 if b_col_major else 0, M, N, K, A, lda, B, ldb, C, ldc)


def tdi8_status_string(status: int) -> str:
    return _lib.tdi8_status_string(status).decode()


def tdi8_last_hip_error() -> int:
    return _lib.tdi8_last_hip_error()


def tdi8_kernel_code_hash() -> str:
    return _lib.tdi8_kernel_code_hash().decode()


# ----- torch convenience -----------------------------------------------------------

def _stream_handle(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _device_of(*tensors) -> "torch.device":
    """The one GPU holding every tensor (the kernels dereference their data
    pointers as device addresses, so host tensors must never reach them)."""
    devs = {t.device for t in tensors}
    if any(d.type != "cuda" for d in devs):
        raise ValueError("tensors must be on a GPU")
    if len(devs) != 1:
        raise ValueError(f"tensors are on different devices: {sorted(str(d) for d in devs)}")
    return devs.pop()


def gemm(A: "torch.Tensor", B: "torch.Tensor", b_col_major: bool, out: "torch.Tensor | None" = None,
         config: int | None = None, stream=None, persistent_blocks: int | None = None) -> "torch.Tensor":
    """C = A x B on the GPU.

    A: int8 (M, K) with unit column stride (row stride = lda).
    B: int8 storage of the logical K x N matrix: (K, N) row-major if
       b_col_major is False, (N, K) with K contiguous if True.
    out: optional int32 (M, N) with unit column stride (row stride = ldc).
    config: run this configuration id instead of the selected one.
    persistent_blocks: run the persistent whole-tile form with this many
       blocks (0: one wave of resident blocks); needs whole tiles.
    """
    if A.dtype != torch.int8 or B.dtype != torch.int8:
        raise TypeError("A and B must be int8")
    if A.dim() != 2 or B.dim() != 2 or A.stride(1) != 1 or B.stride(1) != 1:
        raise ValueError("A and B must be 2-D with unit column stride")
    M, K = A.shape
    N = B.shape[0] if b_col_major else B.shape[1]
    if (B.shape[1] if b_col_major else B.shape[0]) != K:
        raise ValueError("inner dimensions differ")
    dev = _device_of(A, B) if out is None else _device_of(A, B, out)
    if out is None:
        out = torch.empty((M, N), dtype=torch.int32, device=dev)
    if out.dtype != torch.int32 or out.dim() != 2 or tuple(out.shape) != (M, N) or out.stride(1) != 1:
        raise ValueError("out must be int32 (M, N) with unit column stride")
    lda, ldb, ldc = max(A.stride(0), 1), max(B.stride(0), 1), max(out.stride(0), 1)
    _int32(M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=ldc)
    with torch.cuda.device(dev):
        s = _stream_handle(stream)
        if persistent_blocks is not None:
            st = gemm_s8s8s32_persistent(-1 if config is None else config, b_col_major, M, N, K, A.data_ptr(),
                                         lda, B.data_ptr(), ldb, out.data_ptr(), ldc, persistent_blocks, s)
        elif config is None:
            fn = gemm_s8s8s32_bt if b_col_major else gemm_s8s8s32
            st = fn(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, out.data_ptr(), ldc, s)
        else:
            st = gemm_s8s8s32_with_config(config, b_col_major, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                                          out.data_ptr(), ldc, s)
    if st != OK:
        raise TDI8Error(st)
    return out


# ---- convolution ---------------------------------------------------------------

def _conv_int32(N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w) -> None:
    _int32(N=N, H=H, W=W, C=C, K=K, R=R, S=S, pad_h=pad_h, pad_w=pad_w, stride_h=stride_h,
           stride_w=stride_w, dil_h=dil_h, dil_w=dil_w)


def conv2d_s8s8s32_nhwc(N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w,
                        x, w, y, stream=0) -> int:
    _conv_int32(N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w)
    return _lib.conv2d_s8s8s32_nhwc(N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w,
                                    x, w, y, stream)


def conv2d_s8s8s32_nhwc_with_config(config_id, N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w,
                                    dil_h, dil_w, x, w, y, stream=0) -> int:
    _int32(config_id=config_id)
    _conv_int32(N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w)
    return _lib.conv2d_s8s8s32_nhwc_with_config(config_id, N, H, W, C, K, R, S, pad_h, pad_w, stride_h,
                                                stride_w, dil_h, dil_w, x, w, y, stream)


def conv2d_select_config(N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w) -> int:
    _conv_int32(N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w)
    return _lib.conv2d_select_config(N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w)


def conv2d_output_extent(H, R, pad, stride, dil) -> int:
    _int32(H=H, R=R, pad=pad, stride=stride, dil=dil)
    return _lib.conv2d_output_extent(H, R, pad, stride, dil)


def conv2d_validate(N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w, x, w, y) -> int:
    _conv_int32(N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w)
    return _lib.conv2d_validate(N, H, W, C, K, R, S, pad_h, pad_w, stride_h, stride_w, dil_h, dil_w, x, w, y)


def conv2d(x, w, pad=(0, 0), stride=(1, 1), dil=(1, 1), out=None, config=None, stream=None):
    """y = conv2d(x, w) for torch tensors on the GPU: x int8 N x H x W x C,
    w int8 K x R x S x C (both contiguous), y int32 N x P x Q x K."""
    if x.dtype != torch.int8 or w.dtype != torch.int8:
        raise TypeError("x and w must be int8")
    if x.dim() != 4 or w.dim() != 4 or not x.is_contiguous() or not w.is_contiguous():
        raise ValueError("x (N, H, W, C) and w (K, R, S, C) must be contiguous 4-D tensors")
    N, H, W, C = x.shape
    K, R, S, Cw = w.shape
    if Cw != C:
        raise ValueError(f"channel counts differ: x has {C}, w has {Cw}")
    P = conv2d_output_extent(H, R, pad[0], stride[0], dil[0])
    Q = conv2d_output_extent(W, S, pad[1], stride[1], dil[1])
    if P < 0 or Q < 0:
        raise TDI8Error(min(P, Q))
    dev = _device_of(x, w) if out is None else _device_of(x, w, out)
    if out is None:
        out = torch.empty((N, P, Q, K), dtype=torch.int32, device=dev)
    if out.dtype != torch.int32 or tuple(out.shape) != (N, P, Q, K) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous int32 tensor of shape {(N, P, Q, K)}")
    with torch.cuda.device(dev):
        args = (N, H, W, C, K, R, S, pad[0], pad[1], stride[0], stride[1], dil[0], dil[1],
                x.data_ptr(), w.data_ptr(), out.data_ptr(), _stream_handle(stream))
        st = conv2d_s8s8s32_nhwc(*args) if config is None else conv2d_s8s8s32_nhwc_with_config(config, *args)
    if st != OK:
        raise TDI8Error(st)
    return out
