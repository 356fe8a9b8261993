"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module only draws random numbers and lays them out in memory as stored
bits (f32 values, or IEEE binary16 / bfloat16 bit patterns as uint16). It
holds none of the matrix-product arithmetic: no products, sums, or output
rounding. Both the GPU library and the oracle receive exactly these bytes.

Draws use ``numpy.random.default_rng(seed)`` (PCG64), float64 draws in the
order listed for each workload, rounded to float32 (nearest even) and then
to the storage type (nearest even).

The five named workloads are the synthetic stand-ins for the shapes the
pages' layers run at: a 128^3 f32 GEMM, an f16 decode GEMV against an
[11008, 4096] weight, a batched strided f16 GEMM, an 8192^3 f16 GEMM and a
64-expert bf16 expert-ID matmul (prefill plus decode).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

F32, F16, BF16 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16"}
ELT = {F32: 4, F16: 2, BF16: 2}
NP_STORE = {F32: np.float32, F16: np.uint16, BF16: np.uint16}


# --------------------------------------------------------------------------
# Storage conversion of generated values (input preparation only).
# --------------------------------------------------------------------------

def _f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def to_storage(x, dtype: int) -> np.ndarray:
    """Generated float values -> stored bits (float32 or uint16 patterns)."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == F32:
        return x32
    if dtype == F16:
        return x32.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        return _f32_to_bf16_bits(x32)
    raise ValueError(f"unknown dtype {dtype}")


def storage_to_float(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Stored bits -> float64 values (for building fixtures and checks)."""
    bits = np.asarray(bits)
    if dtype == F32:
        return bits.astype(np.float32).astype(np.float64)
    if dtype == F16:
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    u = bits.astype(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def nan_bits(dtype: int):
    """A quiet-NaN stored value, used to fill padding no kernel may read."""
    if dtype == F32:
        return np.float32(np.nan)
    return np.uint16(0x7E00 if dtype == F16 else 0x7FC0)


def ramp(n: int, seed: int) -> np.ndarray:
    """The integer-ramp test input of tract-metal's gemv_wide tests:
    value i is ((7i + 13*seed) mod 29 - 14) / 64, exact in f16, bf16 and f32."""
    i = np.arange(n, dtype=np.int64)
    return (((i * 7 + seed * 13) % 29) - 14).astype(np.float64) / 64.0


# --------------------------------------------------------------------------
# GEMM / GEMV operand layout.
# --------------------------------------------------------------------------

@dataclasses.dataclass
class GemmCase:
    """One C = op(A).op(B) problem laid out in flat buffers.

    Stored shapes: A is [m,k] (or [k,m] when trans_a), B is [k,n] (or [n,k]
    when trans_b), per batch. ld*, stride_* are in elements (stride 0 =
    one matrix broadcast to every batch); off_* are byte offsets.
    """
    dtype: int
    batch: int
    m: int
    n: int
    k: int
    trans_a: bool
    trans_b: bool
    lda: int
    ldb: int
    ldc: int
    stride_a: int
    stride_b: int
    stride_c: int
    off_a: int
    off_b: int
    off_c: int
    A: np.ndarray          # flat stored bits
    B: np.ndarray          # flat stored bits
    c_elems: int           # elements the C buffer needs (offset included)

    @property
    def flops(self) -> int:
        return 2 * self.batch * self.m * self.n * self.k


def _place(values: np.ndarray, dtype: int, ld: int, stride: int, off_elems: int,
           extra: int = 0) -> np.ndarray:
    """Lay [batch, rows, cols] values into a flat buffer with leading dim `ld`,
    batch stride `stride` (0: store only the first matrix) and an element
    offset; everything else holds NaN."""
    bt, rows, cols = values.shape
    nb = 1 if stride == 0 else bt
    span = off_elems + (nb - 1) * stride + (rows - 1) * ld + cols + extra
    buf = np.full(span, nan_bits(dtype), dtype=NP_STORE[dtype])
    bits = to_storage(values, dtype)
    for b in range(nb):
        base = off_elems + b * stride
        for r in range(rows):
            buf[base + r * ld: base + r * ld + cols] = bits[b, r]
    return buf


def make_gemm_case(dtype: int, a_vals: np.ndarray, b_vals: np.ndarray, trans_a: bool,
                   trans_b: bool, *, lda: int = 0, ldb: int = 0, ldc: int = 0,
                   stride_a: Optional[int] = None, stride_b: Optional[int] = None,
                   stride_c: int = 0, off_a: int = 0, off_b: int = 0, off_c: int = 0,
                   broadcast_a: bool = False, broadcast_b: bool = False) -> GemmCase:
    """Build a GemmCase from stored-orientation values.

    a_vals: [batch, m, k] (or [batch, k, m] if trans_a); b_vals likewise.
    With broadcast_*, only the first matrix is stored and its stride is 0.
    Offsets are in elements here and stored as bytes in the case.
    """
    a_vals = np.asarray(a_vals, dtype=np.float64)
    b_vals = np.asarray(b_vals, dtype=np.float64)
    batch = max(a_vals.shape[0], b_vals.shape[0])
    if trans_a:
        k, m = a_vals.shape[1:]
    else:
        m, k = a_vals.shape[1:]
    if trans_b:
        n, kb = b_vals.shape[1:]
    else:
        kb, n = b_vals.shape[1:]
    assert kb == k, (a_vals.shape, b_vals.shape)
    a_rows, a_cols = a_vals.shape[1:]
    b_rows, b_cols = b_vals.shape[1:]
    lda = lda or a_cols
    ldb = ldb or b_cols
    ldc = ldc or n
    if broadcast_a:
        stride_a = 0
    elif stride_a is None:
        stride_a = (a_rows - 1) * lda + a_cols
    if broadcast_b:
        stride_b = 0
    elif stride_b is None:
        stride_b = (b_rows - 1) * ldb + b_cols
    if not stride_c:
        stride_c = m * ldc
    A = _place(a_vals[:1] if broadcast_a else a_vals, dtype, lda, stride_a, off_a)
    B = _place(b_vals[:1] if broadcast_b else b_vals, dtype, ldb, stride_b, off_b)
    c_elems = off_c + (batch - 1) * stride_c + (m - 1) * ldc + n
    e = ELT[dtype]
    return GemmCase(dtype, batch, m, n, k, trans_a, trans_b, lda, ldb, ldc, stride_a,
                    stride_b, stride_c, off_a * e, off_b * e, off_c * e, A, B, c_elems)


def random_gemm_case(seed: int, dtype: int, batch: int, m: int, n: int, k: int,
                     trans_a: bool, trans_b: bool, dist: str = "normal", **layout) -> GemmCase:
    """Random operands: A then B drawn from one generator ("normal": N(0,1)/sqrt(k)
    scaled to unit-ish outputs; "uniform": U[-1, 1])."""
    rng = np.random.default_rng(seed)
    a_shape = (batch, k, m) if trans_a else (batch, m, k)
    b_shape = (batch, n, k) if trans_b else (batch, k, n)
    if dist == "uniform":
        a = rng.uniform(-1.0, 1.0, a_shape)
        b = rng.uniform(-1.0, 1.0, b_shape)
    else:
        a = rng.standard_normal(a_shape)
        b = rng.standard_normal(b_shape) / math.sqrt(k)
    return make_gemm_case(dtype, a, b, trans_a, trans_b, **layout)


# --------------------------------------------------------------------------
# Expert-ID matmul inputs.
# --------------------------------------------------------------------------

@dataclasses.dataclass
class IdCase:
    """One expert-ID matmul problem: weights [E, n, k] (row-major per expert,
    `expert_stride_bytes` apart), f32 activations, u32 ids [m, top_k]."""
    wdtype: int
    m: int
    n: int
    k: int
    top_k: int
    n_experts: int
    expert_stride_bytes: int
    layout: int                 # 0 shared per token, 1 slotted
    W: np.ndarray               # flat stored bits
    X: np.ndarray               # float32 [m or m*top_k, k]
    ids: np.ndarray             # uint32 [m, top_k]

    @property
    def flops(self) -> int:
        valid = int((self.ids < self.n_experts).sum())
        return 2 * valid * self.n * self.k


def make_id_case(wdtype: int, w_vals: np.ndarray, x_vals: np.ndarray, ids: np.ndarray,
                 layout: int = 0, stride_pad_elems: int = 0) -> IdCase:
    """w_vals [E, n, k]; x_vals [m, k] (shared) or [m*top_k, k] (slotted); ids [m, top_k].
    stride_pad_elems adds NaN-filled elements between experts."""
    w_vals = np.asarray(w_vals, dtype=np.float64)
    E, n, k = w_vals.shape
    ids = np.ascontiguousarray(ids, dtype=np.uint32)
    m, top_k = ids.shape
    stride = n * k + stride_pad_elems
    W = np.full(E * stride, nan_bits(wdtype), dtype=NP_STORE[wdtype])
    bits = to_storage(w_vals, wdtype).reshape(E, n * k)
    for e in range(E):
        W[e * stride: e * stride + n * k] = bits[e]
    X = to_storage(x_vals, F32)
    return IdCase(wdtype, m, n, k, top_k, E, stride * ELT[wdtype], layout, W, X, ids)


def distinct_ids(rng: np.random.Generator, m: int, top_k: int, n_experts: int) -> np.ndarray:
    """Per token, the first top_k entries of a fresh permutation of the experts."""
    ids = np.empty((m, top_k), dtype=np.uint32)
    for t in range(m):
        ids[t] = rng.permutation(n_experts)[:top_k]
    return ids


def random_id_case(seed: int, wdtype: int, m: int, n: int, k: int, top_k: int,
                   n_experts: int, layout: int = 0, distinct: bool = True,
                   w_scale: float = 0.02, stride_pad_elems: int = 0) -> IdCase:
    rng = np.random.default_rng(seed)
    w = w_scale * rng.standard_normal((n_experts, n, k))
    rows = m if layout == 0 else m * top_k
    x = rng.standard_normal((rows, k))
    if distinct:
        ids = distinct_ids(rng, m, top_k, n_experts)
    else:
        ids = rng.integers(0, n_experts, (m, top_k)).astype(np.uint32)
    return make_id_case(wdtype, w, x, ids, layout, stride_pad_elems)


# --------------------------------------------------------------------------
# The five named workloads.
# --------------------------------------------------------------------------

def gemm_f32_128() -> GemmCase:
    """f32 GEMM, batch 1, M=N=K=128, A and B row-major (no transposes),
    entries U[-1, 1] from seed 0 (A drawn first)."""
    rng = np.random.default_rng(0)
    a = rng.uniform(-1.0, 1.0, (1, 128, 128))
    b = rng.uniform(-1.0, 1.0, (1, 128, 128))
    return make_gemm_case(F32, a, b, False, False)


def gemv_f16_decode() -> GemmCase:
    """f16 decode GEMV: x [1, 4096] ~ N(0,1), W [11008, 4096] ~ 0.02 N(0,1)
    stored [N, K] and used transposed (trans_b), seed 1 (x drawn first)."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, 1, 4096))
    w = 0.02 * rng.standard_normal((1, 11008, 4096))
    return make_gemm_case(F16, x, w, False, True)


def gemv_f16_skinny() -> GemmCase:
    """Skinny f16 product (a short batch of decode tokens): x [8, 4096] ~ N(0,1),
    W [11008, 4096] ~ 0.02 N(0,1) stored [N, K] and used transposed (trans_b),
    seed 5 (x drawn first). Not one of the five named workloads: it measures
    the skinny route at the decode GEMV's weight shape."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 8, 4096))
    w = 0.02 * rng.standard_normal((1, 11008, 4096))
    return make_gemm_case(F16, x, w, False, True)


def gemm_f16_batched() -> GemmCase:
    """Batched strided f16 GEMM C = A.B^T: batch 32, A and B [32, 512, 128],
    entries N(0,1)/sqrt(128), contiguous batch strides, seed 2."""
    rng = np.random.default_rng(2)
    a = rng.standard_normal((32, 512, 128)) / math.sqrt(128.0)
    b = rng.standard_normal((32, 512, 128)) / math.sqrt(128.0)
    return make_gemm_case(F16, a, b, False, True)


def gemm_f16_large() -> GemmCase:
    """f16 GEMM M=N=K=8192, A row-major, B stored [N, K] (trans_b), entries
    U[-0.5, 0.5], seed 3 (A drawn first)."""
    rng = np.random.default_rng(3)
    a = rng.uniform(-0.5, 0.5, (8192, 8192)).astype(np.float32)
    a_bits = a.astype(np.float16).view(np.uint16)
    del a
    b = rng.uniform(-0.5, 0.5, (8192, 8192)).astype(np.float32)
    b_bits = b.astype(np.float16).view(np.uint16)
    del b
    n = 8192
    return GemmCase(F16, 1, n, n, n, False, True, n, n, n, n * n, n * n, n * n, 0, 0, 0,
                    a_bits.reshape(-1), b_bits.reshape(-1), n * n)


@dataclasses.dataclass
class MoeWorkload:
    prefill: IdCase
    decode: IdCase


def moe_bf16() -> MoeWorkload:
    """64 experts, bf16 weight stack [64, 1408, 2048] ~ 0.02 N(0,1) (drawn
    expert by expert); f32 activations [512, 2048] ~ N(0,1) shared per token;
    top_k = 8 distinct ids per token (a prefix of a fresh permutation), seed 4.
    Then a decode pass: x [1, 2048] ~ N(0,1), 8 ids drawn with repeats allowed
    and slot 7 forced equal to slot 0."""
    rng = np.random.default_rng(4)
    E, n, k, m, top_k = 64, 1408, 2048, 512, 8
    W = np.empty(E * n * k, dtype=np.uint16)
    for e in range(E):
        W[e * n * k:(e + 1) * n * k] = to_storage(0.02 * rng.standard_normal((n, k)),
                                                  BF16).reshape(-1)
    X = to_storage(rng.standard_normal((m, k)), F32)
    ids = distinct_ids(rng, m, top_k, E)
    xd = to_storage(rng.standard_normal((1, k)), F32)
    idd = rng.integers(0, E, top_k).astype(np.uint32)
    idd[7] = idd[0]
    stride = n * k * 2
    prefill = IdCase(BF16, m, n, k, top_k, E, stride, 0, W, X, ids)
    decode = IdCase(BF16, 1, n, k, top_k, E, stride, 0, W, xd, idd.reshape(1, top_k))
    return MoeWorkload(prefill, decode)


def moe_bf16_slotted_decode(moe: MoeWorkload) -> IdCase:
    """The decode pass of `moe_bf16` with the slotted activation layout: one
    f32 row per (token, slot), x [8, 2048] ~ N(0,1) from seed 5, same weights
    and ids (slot 7 repeats slot 0's expert with its own activations)."""
    d = moe.decode
    rng = np.random.default_rng(5)
    xs = to_storage(rng.standard_normal((d.m * d.top_k, d.k)), F32)
    return IdCase(d.wdtype, d.m, d.n, d.k, d.top_k, d.n_experts, d.expert_stride_bytes, 1,
                  d.W, xs, d.ids)
