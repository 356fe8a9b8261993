"""The five named workloads at full size, through the same calls the benchmark times.

Every output is compared with the oracle in full, except the f16 8192^3 GEMM
(5.5e11 multiply-adds, minutes of oracle time): there the oracle evaluates
seeded output positions one by one, three inside every 256 x 256 output tile
(the tile of the kernel that runs it) plus the corners, and every element is
checked to have been written. The map pass is compared in full, bit for bit.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import gemv_expert_id_amd as mm
import oracle
import workloads as wl
from gpu_util import GemmRun, IdRun, assert_close, finite_absmax

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_gemm_f32_128():
    _say("workload: f32 GEMM 128^3 NN")
    case = wl.gemm_f32_128()
    run = GemmRun(case)
    rec = run.run()
    assert rec.route == mm.MM_ROUTE_GEMM
    got, _ = run.logical_c(run.c_bits())
    amax, bmax = run.operand_absmax()
    err = assert_close(got, run.oracle_full(), case.dtype, case.k, amax, bmax, "f32 128")
    _say(f"  max err {err:.3e}")


def test_gemv_f16_decode():
    _say("workload: f16 decode GEMV [1,4096] x [11008,4096]^T")
    case = wl.gemv_f16_decode()
    run = GemmRun(case)
    rec = run.run()
    assert rec.route == mm.MM_ROUTE_GEMV
    got, mask = run.logical_c(run.c_bits())
    amax, bmax = run.operand_absmax()
    err = assert_close(got, run.oracle_full(), case.dtype, case.k, amax, bmax, "gemv decode")
    _say(f"  max err {err:.3e}")


def test_gemm_f16_batched():
    _say("workload: batched f16 NT 32 x [512,128] x [512,128]^T (full compare)")
    case = wl.gemm_f16_batched()
    run = GemmRun(case)
    rec = run.run()
    assert rec.route == mm.MM_ROUTE_GEMM and rec.kernel == mm.MM_KERNEL_GEMM_PANEL, rec.kernel
    # 128-row panels, each panel's 8 B tiles split over 2 blocks (256 blocks).
    assert (rec.variant & 0xff, rec.variant >> 8) == (2, 128), rec.variant
    bits = run.c_bits()
    got, mask = run.logical_c(bits)
    run.check_untouched(bits, mask)
    amax, bmax = run.operand_absmax()
    err = assert_close(got, run.oracle_full(), case.dtype, case.k, amax, bmax, "batched")
    _say(f"  max err {err:.3e} over {got.size} outputs")


def _per_tile_positions(m: int, n: int, tile: int, per_tile: int, seed: int):
    """`per_tile` seeded positions inside every tile x tile block of an m x n
    output, plus its four corners."""
    rng = np.random.default_rng(seed)
    ti, tj = np.meshgrid(np.arange(m // tile), np.arange(n // tile), indexing="ij")
    ti = np.repeat(ti.reshape(-1), per_tile)
    tj = np.repeat(tj.reshape(-1), per_tile)
    is_ = ti * tile + rng.integers(0, tile, ti.size)
    js = tj * tile + rng.integers(0, tile, tj.size)
    is_ = np.concatenate([is_, [0, 0, m - 1, m - 1]])
    js = np.concatenate([js, [0, n - 1, 0, n - 1]])
    return is_, js


def test_gemm_f16_large():
    _say("workload: f16 GEMM 8192^3 NT (three samples in every 256 x 256 tile)")
    case = wl.gemm_f16_large()
    run = GemmRun(case)
    rec = run.run()
    assert rec.route == mm.MM_ROUTE_GEMM and rec.kernel == mm.MM_KERNEL_GEMM_LARGE
    bits = run.c_bits()
    is_, js = _per_tile_positions(case.m, case.n, 256, 3, 2)
    bs = np.zeros_like(is_)
    ref = oracle.gemm_at(case.dtype, case.k, case.trans_a, case.trans_b, case.lda, case.ldb,
                         case.stride_a, case.stride_b, case.off_a, case.off_b, case.A, case.B,
                         bs, is_, js)
    got = oracle.decode(case.dtype, bits[is_ * case.ldc + js])
    amax, bmax = run.operand_absmax()
    err = assert_close(got, ref, case.dtype, case.k, amax, bmax, "8192^3 per-tile samples")
    vals, mask = run.logical_c(bits)
    assert np.all(np.isfinite(vals)), "an output element was not written"
    _say(f"  max err {err:.3e} over {is_.size} positions")


@pytest.fixture(scope="module")
def moe():
    return wl.moe_bf16()


def test_moe_prefill(moe):
    _say("workload: expert-ID prefill 64 x bf16 [1408,2048], X [512,2048], top_k 8")
    case = moe.prefill
    run = IdRun(case, route=1)
    rec = run.run()
    assert rec.dispatch_count == 2
    counts, routed = run.scratch()
    rc, rr, _, _ = oracle.matmul_id_map(case.m, case.top_k, case.n_experts, case.ids)
    np.testing.assert_array_equal(counts, rc)
    assert int(counts.sum()) == case.m * case.top_k
    for e in range(case.n_experts):
        np.testing.assert_array_equal(routed[e, :counts[e]], rr[e, :rc[e]])
    # 352-wide tiles: 8 waves of 3 sixteen-output fragment slots (3 + 256 * 8).
    assert rec.kernel == mm.MM_KERNEL_ID_GROUPED_MFMA and rec.variant == 3 | (8 << 8), \
        (rec.kernel, rec.variant)
    got = run.out_f64()
    ref = run.oracle()
    wmax, xmax = run.absmax()
    err = assert_close(got, ref, case.wdtype, case.k, wmax, xmax, "prefill")
    _say(f"  max err {err:.3e} over all {got.shape[0]} routed rows")


def test_moe_decode(moe):
    _say("workload: expert-ID decode m=1 top_k=8 with a repeated id (direct route)")
    case = moe.decode
    assert case.ids[0, 7] == case.ids[0, 0]
    run = IdRun(case, route=0, multiplicity=1)
    rec = run.run()
    assert rec.route == mm.MM_ROUTE_ID_DIRECT
    got = run.out_f64()
    ref = run.oracle()
    wmax, xmax = finite_absmax(case.W, case.wdtype), float(np.abs(case.X).max())
    err = assert_close(got, ref, case.wdtype, case.k, wmax, xmax, "decode")
    np.testing.assert_array_equal(got[0], got[7])
    _say(f"  max err {err:.3e}")


def test_moe_decode_slotted(moe):
    """The decode pass with one activation row per slot (slotted layout): the
    repeated expert is computed for each of its slots with that slot's row."""
    _say("workload: expert-ID decode, slotted activations [8,2048], direct route")
    case = wl.moe_bf16_slotted_decode(moe)
    run = IdRun(case, route=0, multiplicity=1)
    rec = run.run()
    assert rec.route == mm.MM_ROUTE_ID_DIRECT
    assert rec.kernel == mm.MM_KERNEL_ID_DIRECT_FAST and rec.variant == 2, (rec.kernel, rec.variant)
    got = run.out_f64()
    ref = run.oracle()
    wmax, xmax = finite_absmax(case.W, case.wdtype), float(np.abs(case.X).max())
    err = assert_close(got, ref, case.wdtype, case.k, wmax, xmax, "decode slotted")
    assert not np.array_equal(got[0], got[7])  # same expert, different activation rows
    _say(f"  max err {err:.3e}")
