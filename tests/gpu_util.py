"""Helpers for the GPU parity tests: device buffers from the seeded inputs,
calls through the C ABI, and the comparison against the oracle.

Tolerance (floating point): max |gpu - oracle_f64| <= tol * sqrt(K) *
max|A| * max|B| with tol = 1e-6 when every input is f32 and 4e-3 when any
input is f16 or bf16; maxima over the whole operands passed. Integer outputs
(counts, routed rows) and ramp / identity inputs are compared bit for bit.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import gemv_expert_id_amd as mm
import oracle
import workloads as wl

DEV = "cuda:0"
TOL = {wl.F32: 1e-6, wl.F16: 4e-3, wl.BF16: 4e-3}


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """Stored bits -> device tensor holding the same bytes."""
    bits = np.ascontiguousarray(bits)
    if bits.dtype == np.float32:
        t = torch.from_numpy(bits)
    elif bits.dtype == np.uint16:
        t = torch.from_numpy(bits.view(np.int16))
    elif bits.dtype == np.uint32:
        t = torch.from_numpy(bits.view(np.int32))
    else:
        raise TypeError(bits.dtype)
    return t.to(DEV)


def from_dev(t: torch.Tensor, np_dtype) -> np.ndarray:
    return t.cpu().numpy().view(np_dtype)


def empty_like_bits(n: int, dtype: int, fill_nan: bool = True) -> torch.Tensor:
    host = np.full(n, wl.nan_bits(dtype) if fill_nan else 0, dtype=wl.NP_STORE[dtype])
    return to_dev(host)


def finite_absmax(bits: np.ndarray, dtype: int) -> float:
    v = wl.storage_to_float(bits, dtype)
    v = v[np.isfinite(v)]
    return float(np.abs(v).max()) if v.size else 0.0


def bound(dtype: int, k: int, amax: float, bmax: float) -> float:
    return TOL[dtype] * math.sqrt(k) * amax * bmax


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: int, k: int, amax: float,
                 bmax: float, what: str = ""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    lim = bound(dtype, k, amax, bmax)
    assert err <= lim, f"{what}: max |err| {err:.3e} > {lim:.3e}"
    return err


# ---------------------------------------------------------------------------
# GEMM / GEMV
# ---------------------------------------------------------------------------

class GemmRun:
    """A GemmCase on the device, run through mm_gemm (or mm_gemv)."""

    def __init__(self, case: wl.GemmCase, c_extra: int = 7):
        self.case = case
        self.a = to_dev(case.A)
        self.b = to_dev(case.B)
        self.c_elems = case.c_elems + c_extra
        self.c = empty_like_bits(self.c_elems, case.dtype)
        e = wl.ELT[case.dtype]
        self.desc = mm.gemm_desc(case.dtype, case.m, case.n, case.k, batch=case.batch,
                                 trans_a=case.trans_a, trans_b=case.trans_b, lda=case.lda,
                                 ldb=case.ldb, ldc=case.ldc, stride_a=case.stride_a,
                                 stride_b=case.stride_b, stride_c=case.stride_c,
                                 offset_a=case.off_a, offset_b=case.off_b, offset_c=case.off_c)
        self.bufs = (mm.buf(self.a), mm.buf(self.b), mm.buf(self.c))
        self.elt = e

    def run(self, entry=None, stream=None):
        entry = entry or mm.mm_gemm
        return entry(self.desc, *self.bufs, stream=stream or torch.cuda.current_stream())

    def c_bits(self) -> np.ndarray:
        torch.cuda.synchronize()
        return from_dev(self.c, wl.NP_STORE[self.case.dtype])

    def logical_c(self, bits: np.ndarray):
        """(values [batch, m, n] in f64, mask of C elements that belong to the output)."""
        c = self.case
        base = c.off_c // self.elt
        b, i, j = np.meshgrid(np.arange(c.batch), np.arange(c.m), np.arange(c.n), indexing="ij")
        idx = base + b * c.stride_c + i * c.ldc + j
        vals = oracle.decode(c.dtype, bits[idx])
        mask = np.zeros(bits.size, dtype=bool)
        mask[idx.reshape(-1)] = True
        return vals, mask

    def check_untouched(self, bits: np.ndarray, mask: np.ndarray):
        """Every C element outside the output must still hold the NaN sentinel."""
        outside = bits[~mask]
        sentinel = wl.nan_bits(self.case.dtype)
        if self.case.dtype == wl.F32:
            assert np.all(np.isnan(outside)), "kernel wrote outside the output"
        else:
            assert np.all(outside == sentinel), "kernel wrote outside the output"

    def oracle_full(self, nthreads=0):
        c = self.case
        return oracle.gemm(c.dtype, c.batch, c.m, c.n, c.k, c.trans_a, c.trans_b, c.lda, c.ldb,
                           c.stride_a, c.stride_b, c.off_a, c.off_b, c.A, c.B, nthreads)

    def operand_absmax(self):
        return finite_absmax(self.case.A, self.case.dtype), finite_absmax(self.case.B,
                                                                          self.case.dtype)


def skinny_rounds_rule(batch: int, nx: int, nw: int, row_bytes: int) -> bool:
    """mm.h's rounds rule for the skinny route: its blocks (batch x
    ceil(nw / 16); 768, 512 or 256 resident at once for nx up to 16, 32 or
    64) in one round; else rows of at least 512 bytes (two rounds) or 1024
    (more) for nx <= 32, and at most three rounds for nx in 33..64."""
    nxf = (nx + 15) // 16
    cap = 256 * (3 if nxf == 1 else 2 if nxf == 2 else 1)
    rounds = -(-(batch * -(-nw // 16)) // cap)
    if rounds <= 1:
        return True
    if nxf <= 2:
        return row_bytes >= (512 if rounds <= 2 else 1024)
    return rounds <= 3


def expected_gemm_route(case: wl.GemmCase) -> int:
    """The route mm_gemm documents for this case (mm.h, dispatch): skinny when
    A and B keep rows along k, one side has 2..64 rows, the other >= 2, the
    16-byte layout holds (device buffers are 256-byte aligned, so only the
    offsets matter) and the rounds rule allows it; GEMV when m == 1 or
    n == 1; GEMM otherwise."""
    c = case
    ch = 16 // wl.ELT[c.dtype]
    x_is_a = 2 <= c.m <= 64 and c.n >= 2
    skinny = (not c.trans_a and c.trans_b
              and (x_is_a or (2 <= c.n <= 64 and c.m >= 2))
              and c.k % ch == 0 and c.lda % ch == 0 and c.ldb % ch == 0
              and c.stride_a % ch == 0 and c.stride_b % ch == 0
              and c.off_a % 16 == 0 and c.off_b % 16 == 0)
    if skinny:
        nx, nw = (c.m, c.n) if x_is_a else (c.n, c.m)
        skinny = skinny_rounds_rule(c.batch, nx, nw, c.k * wl.ELT[c.dtype])
    if skinny:
        return mm.MM_ROUTE_GEMV_WIDE
    if c.m == 1 or c.n == 1:
        return mm.MM_ROUTE_GEMV
    return mm.MM_ROUTE_GEMM


def check_gemm(case: wl.GemmCase, entry=None, exact: bool = False, what: str = ""):
    """Run on the GPU, compare with the full oracle; returns the receipt."""
    run = GemmRun(case)
    rec = run.run(entry)
    bits = run.c_bits()
    got, mask = run.logical_c(bits)
    run.check_untouched(bits, mask)
    ref = run.oracle_full()
    if exact:
        ref_bits = oracle.round_to(case.dtype, ref)
        got_bits = bits[np.nonzero(mask)[0]]
        # compare through decode to keep the (batch, m, n) order
        np.testing.assert_array_equal(got, oracle.decode(case.dtype, ref_bits), err_msg=what)
    else:
        amax, bmax = run.operand_absmax()
        assert_close(got, ref, case.dtype, case.k, amax, bmax, what)
    return rec


# ---------------------------------------------------------------------------
# Expert-ID matmul
# ---------------------------------------------------------------------------

class IdRun:
    def __init__(self, case: wl.IdCase, route: int, multiplicity: int = None):
        self.case = case
        c = case
        if multiplicity is None:
            multiplicity = 0 if route == 1 else 1
        self.params = mm.id_params(c.m, c.n, c.k, c.top_k, c.n_experts, c.expert_stride_bytes,
                                   c.layout, multiplicity, route)
        self.cap = mm.mm_id_query(c.wdtype, self.params)
        self.w = to_dev(c.W)
        self.x = to_dev(c.X.reshape(-1))
        self.ids = to_dev(c.ids.reshape(-1))
        self.out = empty_like_bits(c.m * c.top_k * c.n, wl.F32)
        if route == 1:
            self.counts = to_dev(np.full(c.n_experts, 0xDEADBEEF, dtype=np.uint32))
            self.routed = to_dev(np.full(c.n_experts * c.m, 0xFFFFFFFF, dtype=np.uint32))
        else:
            self.counts = self.routed = None

    def run(self, stream=None):
        s = stream or torch.cuda.current_stream()
        return mm.mm_id(self.params, self.case.wdtype, mm.buf(self.w), mm.buf(self.x),
                        mm.buf(self.ids), mm.buf(self.out), mm.buf(self.counts),
                        mm.buf(self.routed), stream=s)

    def out_f64(self) -> np.ndarray:
        torch.cuda.synchronize()
        return from_dev(self.out, np.float32).astype(np.float64).reshape(
            self.case.m * self.case.top_k, self.case.n)

    def scratch(self):
        torch.cuda.synchronize()
        return (from_dev(self.counts, np.uint32),
                from_dev(self.routed, np.uint32).reshape(self.case.n_experts, self.case.m))

    def oracle(self, rows=None):
        c = self.case
        if rows is None:
            return oracle.matmul_id(c.wdtype, c.m, c.n, c.k, c.top_k, c.n_experts,
                                    c.expert_stride_bytes, c.layout, c.W, c.X, c.ids)
        return oracle.matmul_id_rows(c.wdtype, c.m, c.n, c.k, c.top_k, c.n_experts,
                                     c.expert_stride_bytes, c.layout, c.W, c.X, c.ids, rows)

    def absmax(self):
        return finite_absmax(self.case.W, self.case.wdtype), float(np.abs(self.case.X).max())

    def tol_dtype(self):
        return self.case.wdtype  # f32 weights and f32 input: 1e-6; else 4e-3
