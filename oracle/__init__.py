"""CPU oracle for the matrix-product dispatch and the expert-ID matmul.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It shares no
code with the GPU library (``gemv_expert_id_amd``) and neither imports the
other; the seeded input generators in ``workloads`` serve both.

The arithmetic lives in ``mm_oracle.c`` (plain C, fp64 accumulation, triple
loops in ascending contraction order). This module builds that file with gcc,
loads it with ctypes and marshals numpy arrays; the one exception is the
output epilogue ``gemm_axpby`` (alpha * product + beta * C_old), two float64
numpy operations written out here.

Parity of every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (worked examples printed on the pages, closed
forms, exact rational brute force, library routines for the rounding).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, F16, BF16 = 0, 1, 2
_ELT = {F32: 4, F16: 2, BF16: 2}
_STORE = {F32: np.float32, F16: np.uint16, BF16: np.uint16}

_lib = None


def build(force: bool = True) -> str:
    """Compile mm_oracle.c into liboracle.so with gcc and OpenMP."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-shared", "-fPIC", "-std=c11", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    i64, u64, u32, i32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int
    vp = ctypes.c_void_p
    lib.orc_round.argtypes = [i32, vp, vp, i64]
    lib.orc_decode.argtypes = [i32, vp, vp, i64]
    lib.orc_gemm.argtypes = [i32, i64, i64, i64, i64, i32, i32, i64, i64, i64, i64, u64, u64,
                             vp, vp, vp, i32]
    lib.orc_gemm_at.argtypes = [i32, i64, i32, i32, i64, i64, i64, i64, u64, u64, vp, vp, i64,
                                vp, vp, vp, vp, i32]
    lib.orc_id.argtypes = [i32, u32, u32, u32, u32, u32, u64, i32, vp, vp, vp, vp, i32]
    lib.orc_id_rows.argtypes = [i32, u32, u32, u32, u32, u32, u64, i32, vp, vp, vp, i64, vp,
                                vp, i32]
    lib.orc_id_map.argtypes = [u32, u32, u32, vp, vp, vp, vp]
    lib.orc_max_threads.argtypes = []
    lib.orc_half_to_double.argtypes = [ctypes.c_uint16]
    lib.orc_half_to_double.restype = ctypes.c_double
    lib.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_to_double.restype = ctypes.c_double
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc < 0:
        raise ValueError(f"oracle {what}: bad argument (code {rc})")


def max_threads() -> int:
    return int(_load().orc_max_threads())


def round_to(dtype: int, x) -> np.ndarray:
    """Round float64 values to `dtype` (nearest, ties to even); returns stored bits."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=_STORE[dtype])
    _check(_load().orc_round(dtype, _ptr(x), _ptr(out), x.size), "round")
    return out


def decode(dtype: int, bits) -> np.ndarray:
    """Exact float64 values of stored `dtype` elements."""
    bits = np.ascontiguousarray(bits, dtype=_STORE[dtype])
    out = np.empty(bits.shape, dtype=np.float64)
    _check(_load().orc_decode(dtype, _ptr(bits), _ptr(out), bits.size), "decode")
    return out


def gemm(dtype: int, batch: int, m: int, n: int, k: int, trans_a: bool, trans_b: bool,
         lda: int, ldb: int, stride_a: int, stride_b: int, off_a: int, off_b: int,
         A: np.ndarray, B: np.ndarray, nthreads: int = 0) -> np.ndarray:
    """C[b] = op(A[b]).op(B[b]) as dense float64 [batch, m, n] (unrounded).

    A and B are flat buffers of stored bits; lda/ldb and the batch strides are
    in elements, off_a/off_b in bytes.
    """
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    C = np.empty((batch, m, n), dtype=np.float64)
    rc = _load().orc_gemm(dtype, batch, m, n, k, int(trans_a), int(trans_b), lda, ldb,
                          stride_a, stride_b, off_a, off_b, _ptr(A), _ptr(B), _ptr(C), nthreads)
    _check(rc, "gemm")
    return C


def gemm_axpby(alpha: float, beta: float, product, c_old) -> np.ndarray:
    """Output epilogue (tract-metal mlx_gemm/mod.rs, `dispatch_metal_mlx_gemm`:
    function constants `do_axpby` and `use_out_source`): alpha * product +
    beta * C_old in float64, unrounded. `product` is a result of gemm() or
    gemm_at(); `c_old` the decoded old outputs at the same positions. With
    beta == 0 the old values take no part (a NaN there does not propagate)."""
    out = float(alpha) * np.asarray(product, dtype=np.float64)
    if beta != 0:
        out = out + float(beta) * np.asarray(c_old, dtype=np.float64)
    return out


def gemm_at(dtype: int, k: int, trans_a: bool, trans_b: bool, lda: int, ldb: int,
            stride_a: int, stride_b: int, off_a: int, off_b: int, A: np.ndarray,
            B: np.ndarray, bs, is_, js, nthreads: int = 0) -> np.ndarray:
    """The same product evaluated only at output positions (bs[s], is_[s], js[s])."""
    bs = np.ascontiguousarray(bs, dtype=np.int64)
    is_ = np.ascontiguousarray(is_, dtype=np.int64)
    js = np.ascontiguousarray(js, dtype=np.int64)
    out = np.empty(bs.shape, dtype=np.float64)
    rc = _load().orc_gemm_at(dtype, k, int(trans_a), int(trans_b), lda, ldb, stride_a, stride_b,
                             off_a, off_b, _ptr(np.ascontiguousarray(A)),
                             _ptr(np.ascontiguousarray(B)), bs.size, _ptr(bs), _ptr(is_),
                             _ptr(js), _ptr(out), nthreads)
    _check(rc, "gemm_at")
    return out


def matmul_id(wdtype: int, m: int, n: int, k: int, top_k: int, n_experts: int,
              expert_stride_bytes: int, layout: int, W: np.ndarray, X: np.ndarray,
              ids: np.ndarray, nthreads: int = 0) -> np.ndarray:
    """Expert-ID matmul as dense float64 [m*top_k, n] (unrounded; +0.0 rows for bad ids)."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.uint32)
    out = np.empty((m * top_k, n), dtype=np.float64)
    rc = _load().orc_id(wdtype, m, n, k, top_k, n_experts, expert_stride_bytes, layout,
                        _ptr(np.ascontiguousarray(W)), _ptr(X), _ptr(ids), _ptr(out), nthreads)
    _check(rc, "matmul_id")
    return out


def matmul_id_rows(wdtype: int, m: int, n: int, k: int, top_k: int, n_experts: int,
                   expert_stride_bytes: int, layout: int, W: np.ndarray, X: np.ndarray,
                   ids: np.ndarray, rows, nthreads: int = 0) -> np.ndarray:
    """The expert-ID matmul for selected routed rows only: float64 [len(rows), n]."""
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    X = np.ascontiguousarray(X, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.uint32)
    out = np.empty((rows.size, n), dtype=np.float64)
    rc = _load().orc_id_rows(wdtype, m, n, k, top_k, n_experts, expert_stride_bytes, layout,
                             _ptr(np.ascontiguousarray(W)), _ptr(X), _ptr(ids), rows.size,
                             _ptr(rows), _ptr(out), nthreads)
    _check(rc, "matmul_id_rows")
    return out


def matmul_id_map(m: int, top_k: int, n_experts: int, ids: np.ndarray, fill: int = 0xFFFFFFFF):
    """Map pass: (counts[E], routed_rows[E, m], zero_row[m*top_k], promise_broken).

    routed_rows entries past counts[e] keep `fill`.
    """
    ids = np.ascontiguousarray(ids, dtype=np.uint32)
    counts = np.zeros(n_experts, dtype=np.uint32)
    routed = np.full((n_experts, m), fill, dtype=np.uint32)
    zero_row = np.zeros(m * top_k, dtype=np.uint8)
    rc = _load().orc_id_map(m, top_k, n_experts, _ptr(ids), _ptr(counts), _ptr(routed),
                            _ptr(zero_row))
    _check(rc, "matmul_id_map")
    return counts, routed, zero_row.astype(bool), bool(rc == 1)
