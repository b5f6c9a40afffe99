"""Helpers for the GPU parity tests: place seeded host matrices on the device
with chosen leading dimensions, byte offsets and sentinel padding, run one
entry point of the C-ABI library, and bring C back with its padding."""
from __future__ import annotations

import sys

import numpy as np

import synthetic

SENT_A, SENT_B, SENT_C = 99, -77, -123456789
CANARY = 64  # int32 elements of sentinel after C's last row


def note(msg: str) -> None:
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


class DeviceCase:
    """Device copies of logical A (M x K), B (K x N) and a sentinel-filled C."""

    def __init__(self, A_log, B_log, b_col_major, lda=None, ldb=None, ldc=None, offsets=(0, 0, 0)):
        import torch
        self.M, self.K = A_log.shape
        self.N = B_log.shape[1]
        self.bcm = bool(b_col_major)
        M, N, K = self.M, self.N, self.K
        self.lda = lda if lda is not None else max(K, 1)
        b_rows, b_cols = (N, K) if self.bcm else (K, N)
        self.ldb = ldb if ldb is not None else max(b_cols, 1)
        self.ldc = ldc if ldc is not None else max(N, 1)
        oa, ob, oc = offsets
        # host storage with sentinel padding
        self.A_store = np.full((M, self.lda), SENT_A, np.int8)
        self.A_store[:, :K] = A_log
        self.B_store = np.full((b_rows, self.ldb), SENT_B, np.int8)
        self.B_store[:, :b_cols] = synthetic.store_b(B_log, self.bcm)
        dev = "cuda"
        self.a_buf = torch.empty(oa + self.A_store.size + 16, dtype=torch.int8, device=dev)
        self.a_buf[oa:oa + self.A_store.size].copy_(torch.from_numpy(self.A_store.reshape(-1)))
        self.b_buf = torch.empty(ob + self.B_store.size + 16, dtype=torch.int8, device=dev)
        self.b_buf[ob:ob + self.B_store.size].copy_(torch.from_numpy(self.B_store.reshape(-1)))
        self.c_elems = M * self.ldc
        self.c_buf = torch.full((oc + self.c_elems + CANARY,), SENT_C, dtype=torch.int32, device=dev)
        self.A_ptr = self.a_buf.data_ptr() + oa
        self.B_ptr = self.b_buf.data_ptr() + ob
        self.C_ptr = self.c_buf.data_ptr() + 4 * oc
        self.oc = oc

    def run(self, entry, config=None, stream=0, persistent=None):
        import tiled_dense_int8_amd as t
        if persistent is not None:
            return t.gemm_s8s8s32_persistent(-1 if config is None else config, self.bcm, self.M, self.N, self.K,
                                             self.A_ptr, self.lda, self.B_ptr, self.ldb, self.C_ptr, self.ldc,
                                             persistent, stream)
        args = (self.M, self.N, self.K, self.A_ptr, self.lda, self.B_ptr, self.ldb, self.C_ptr, self.ldc, stream)
        if config is not None:
            return t.gemm_s8s8s32_with_config(config, self.bcm, *args)
        fn = t.gemm_s8s8s32_bt if self.bcm else t.gemm_s8s8s32
        return fn(*args)

    def result(self):
        """(C window as (M, N) int32, everything else of the buffer)."""
        import torch
        torch.cuda.synchronize()
        flat = self.c_buf.cpu().numpy()
        win = flat[self.oc:self.oc + self.c_elems].reshape(self.M, self.ldc)
        C = win[:, :self.N].copy()
        rest = np.concatenate([flat[:self.oc], win[:, self.N:].reshape(-1), flat[self.oc + self.c_elems:]])
        return C, rest

    def oracle(self):
        import oracle
        return oracle.gemm(self.A_store, self.B_store, self.bcm, M=self.M, N=self.N, K=self.K)


def check_case(case: DeviceCase, entry_desc: str, config=None, expect=None, persistent=None):
    import tiled_dense_int8_amd as t
    note(f"[case] {entry_desc} M={case.M} N={case.N} K={case.K} bcm={case.bcm} lda={case.lda} "
         f"ldb={case.ldb} ldc={case.ldc} config={config} persistent={persistent}")
    st = case.run(None, config=config, persistent=persistent)
    assert st == t.OK, t.tdi8_status_string(st)
    C, rest = case.result()
    want = expect if expect is not None else case.oracle()
    if not np.array_equal(C, want):
        bad = np.argwhere(C != want)
        i, j = bad[0]
        raise AssertionError(f"{entry_desc}: {len(bad)} mismatches, first at ({i},{j}): got {C[i, j]} "
                             f"want {want[i, j]}")
    assert (rest == SENT_C).all(), f"{entry_desc}: wrote outside the C window"
    return C
