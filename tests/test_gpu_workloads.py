"""The five named workloads at full size, through the same calls the benchmark times.

Where the oracle cannot finish the whole output in seconds, it evaluates a
seeded sample of output positions one by one (GEMM) or whole routed rows
(expert-ID); the map pass is always compared in full, bit for bit.
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


def _sampled_gemm(case: wl.GemmCase, n_samples: int, seed: int):
    run = GemmRun(case)
    rec = run.run()
    bits = run.c_bits()
    rng = np.random.default_rng(seed)
    bs = rng.integers(0, case.batch, n_samples)
    is_ = rng.integers(0, case.m, n_samples)
    js = rng.integers(0, case.n, n_samples)
    # always include the four corners of the first and last batch
    bs = np.concatenate([bs, [0, 0, 0, 0, case.batch - 1, case.batch - 1]])
    is_ = np.concatenate([is_, [0, 0, case.m - 1, case.m - 1, 0, case.m - 1]])
    js = np.concatenate([js, [0, case.n - 1, 0, case.n - 1, 0, case.n - 1]])
    ref = oracle.gemm_at(case.dtype, case.k, case.trans_a, case.trans_b, case.lda, case.ldb,
                         case.stride_a, case.stride_b, case.off_a, case.off_b, case.A, case.B,
                         bs, is_, js)
    idx = case.off_c // wl.ELT[case.dtype] + bs * case.stride_c + is_ * case.ldc + js
    got = oracle.decode(case.dtype, bits[idx])
    amax, bmax = run.operand_absmax()
    err = assert_close(got, ref, case.dtype, case.k, amax, bmax, "sampled")
    # every output element must have been written (no NaN sentinel left inside C)
    vals, mask = run.logical_c(bits)
    assert np.all(np.isfinite(vals))
    return rec, err


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
    _say("workload: batched f16 NT 32 x [512,128] x [512,128]^T")
    rec, err = _sampled_gemm(wl.gemm_f16_batched(), 8192, 1)
    assert rec.route == mm.MM_ROUTE_GEMM
    _say(f"  max err {err:.3e}")


def test_gemm_f16_large():
    _say("workload: f16 GEMM 8192^3 NT")
    rec, err = _sampled_gemm(wl.gemm_f16_large(), 2048, 2)
    assert rec.route == mm.MM_ROUTE_GEMM
    _say(f"  max err {err:.3e}")


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
    got = run.out_f64()
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(5)
    rows = np.concatenate([rng.choice(case.m * case.top_k, 40, replace=False),
                           [0, case.m * case.top_k - 1]])
    # also the first and last routed row of a few experts
    for e in (0, 17, 63):
        rows = np.concatenate([rows, [rr[e, 0], rr[e, rc[e] - 1]]])
    ref = run.oracle(rows)
    wmax, xmax = run.absmax()
    err = assert_close(got[rows], ref, case.wdtype, case.k, wmax, xmax, "prefill rows")
    _say(f"  max err {err:.3e} over {rows.size} rows")


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
    got = run.out_f64()
    ref = run.oracle()
    wmax, xmax = finite_absmax(case.W, case.wdtype), float(np.abs(case.X).max())
    err = assert_close(got, ref, case.wdtype, case.k, wmax, xmax, "decode slotted")
    assert not np.array_equal(got[0], got[7])  # same expert, different activation rows
    _say(f"  max err {err:.3e}")
