"""GPU parity of the expert-ID matmul (direct route; map + grouped route).

Shapes follow mlx-native dense_matmul_id.rs (its test uses m=9, n=7, k=35,
top_k=2, E=4) plus ragged multi-tile shapes, both activation layouts, every
weight dtype, padded expert strides, out-of-range ids (including -1 passed
as u32) and repeated ids on the direct route. Map outputs are bit-exact.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import gemv_expert_id_amd as mm
import oracle
import workloads as wl
from gpu_util import IdRun, assert_close, from_dev, to_dev

pytestmark = pytest.mark.gpu

DTYPES = [wl.F32, wl.F16, wl.BF16]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check_all_rows(run: IdRun, what: str):
    got = run.out_f64()
    ref = run.oracle()
    wmax, xmax = run.absmax()
    assert_close(got, ref, run.case.wdtype, run.case.k, wmax, xmax, what)
    bad = (run.case.ids.reshape(-1) >= run.case.n_experts)
    if bad.any():
        assert np.all(got[bad] == 0.0) and not np.any(np.signbit(got[bad])), "bad-id rows not +0"


def _check_map(run: IdRun):
    counts, routed = run.scratch()
    rc, rr, zero_row, broken = oracle.matmul_id_map(run.case.m, run.case.top_k,
                                                    run.case.n_experts, run.case.ids)
    assert not broken
    np.testing.assert_array_equal(counts, rc)
    for e in range(run.case.n_experts):
        np.testing.assert_array_equal(routed[e, :counts[e]], rr[e, :rc[e]], err_msg=f"expert {e}")


def _with_bad_ids(case: wl.IdCase):
    ids = case.ids.reshape(-1)
    if ids.size >= 3:
        ids[1] = case.n_experts + 2
        ids[-1] = 0xFFFFFFFF
    return case


@pytest.mark.parametrize("wdt", DTYPES)
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("shape", [(9, 7, 35, 2, 4), (5, 130, 260, 3, 6), (3, 1408, 2048, 8, 64),
                                   (17, 33, 64, 4, 9),
                                   # many repeats per token on the one-group fast form
                                   # (k = 2048 for 2-byte weights, 1024 for f32)
                                   (3, 40, 2048, 16, 4), (4, 24, 1024, 8, 3),
                                   # several K groups, and K past 8192
                                   (2, 24, 4096, 3, 5), (1, 8, 12288, 2, 3),
                                   # top_k above the wave width: element-loop form
                                   (2, 70, 2048, 70, 8)])
def test_direct(wdt, layout, shape):
    m, n, k, top_k, E = shape
    _say(f"direct wdt={wl.DTYPE_NAMES[wdt]} layout={layout} shape={shape}")
    case = _with_bad_ids(wl.random_id_case(40 + m, wdt, m, n, k, top_k, E, layout=layout,
                                           distinct=False))
    run = IdRun(case, route=0)
    rec = run.run()
    assert rec.route == mm.MM_ROUTE_ID_DIRECT and rec.dispatch_count == 1
    _check_all_rows(run, "direct")


@pytest.mark.parametrize("wdt", DTYPES)
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("shape", [(9, 7, 35, 2, 4), (5, 130, 260, 3, 6), (40, 300, 520, 8, 16),
                                   (300, 65, 96, 2, 3), (1, 17, 40, 4, 1024),
                                   # k % 256 == 0: the pipelined bf16 form (k = 256 is one round)
                                   (33, 200, 512, 4, 8), (17, 96, 256, 2, 5),
                                   # more than 128 rows per expert: several row tiles
                                   (300, 64, 512, 2, 3)])
def test_prefill_map_grouped(wdt, layout, shape):
    m, n, k, top_k, E = shape
    _say(f"prefill wdt={wl.DTYPE_NAMES[wdt]} layout={layout} shape={shape}")
    case = _with_bad_ids(wl.random_id_case(50 + m, wdt, m, n, k, top_k, E, layout=layout,
                                           stride_pad_elems=8))
    run = IdRun(case, route=1)
    rec = run.run()
    assert rec.route == mm.MM_ROUTE_ID_PREFILL and rec.dispatch_count == 2
    _check_map(run)
    _check_all_rows(run, "grouped")


@pytest.mark.parametrize("wdt", DTYPES)
def test_map_then_grouped_separately(wdt):
    m, n, k, top_k, E = 33, 150, 136, 4, 12
    _say(f"map+grouped separate wdt={wl.DTYPE_NAMES[wdt]}")
    case = _with_bad_ids(wl.random_id_case(60, wdt, m, n, k, top_k, E))
    run = IdRun(case, route=1)
    s = torch.cuda.current_stream()
    r1 = mm.mm_id_map(run.params, mm.buf(run.ids), mm.buf(run.counts), mm.buf(run.routed),
                      mm.buf(run.out), stream=s)
    r2 = mm.mm_id_grouped(run.params, wdt, mm.buf(run.w), mm.buf(run.x), mm.buf(run.counts),
                          mm.buf(run.routed), mm.buf(run.out), stream=s)
    assert r1.route == mm.MM_ROUTE_ID_MAP and r2.route == mm.MM_ROUTE_ID_GROUPED
    _check_map(run)
    _check_all_rows(run, "separate")


@pytest.mark.parametrize("route", [0, 1])
@pytest.mark.parametrize("wdt", DTYPES)
def test_ramp_bit_exact(route, wdt):
    """Ramp weights and activations (exact in bf16): both routes reproduce the
    rounded oracle bit for bit, including the bf16 hi/lo split."""
    m, n, k, top_k, E = 20, 72, 200, 3, 7
    rng = np.random.default_rng(70)
    w = wl.ramp(E * n * k, 2).reshape(E, n, k)
    x = wl.ramp(m * k, 1).reshape(m, k)
    ids = wl.distinct_ids(rng, m, top_k, E)
    case = wl.make_id_case(wdt, w, x, ids)
    _say(f"ramp id route={route} wdt={wl.DTYPE_NAMES[wdt]}")
    run = IdRun(case, route=route)
    run.run()
    got = from_dev(run.out, np.float32).reshape(m * top_k, n)
    ref = oracle.round_to(wl.F32, run.oracle())
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("wdt", DTYPES)
def test_ramp_bit_exact_pipelined_grouped(wdt):
    """k = 512 takes the pipelined MFMA grouped kernel for every weight dtype
    (bf16 as stored, f16 split exactly into bf16 halves, f32 on 16x16x4 f32
    MFMA; activations into bf16 hi + lo for the first two); on ramp inputs
    every term is exact, so the output matches the rounded oracle bit for
    bit. More than 128 rows land on one expert, so full 128-row tiles (eight
    row groups) are covered too."""
    m, n, k, top_k, E = 150, 72, 512, 2, 2
    rng = np.random.default_rng(71)
    w = wl.ramp(E * n * k, 3).reshape(E, n, k)
    x = wl.ramp(m * k, 4).reshape(m, k)
    ids = wl.distinct_ids(rng, m, top_k, E)
    case = wl.make_id_case(wdt, w, x, ids)
    _say(f"ramp pipelined grouped wdt={wl.DTYPE_NAMES[wdt]}")
    run = IdRun(case, route=1)
    rec = run.run()
    assert rec.kernel == mm.MM_KERNEL_ID_GROUPED_MFMA, rec.kernel
    got = from_dev(run.out, np.float32).reshape(m * top_k, n)
    ref = oracle.round_to(wl.F32, run.oracle())
    np.testing.assert_array_equal(got, ref)


# Fragment slots per wave of the pipelined grouped kernel. The host sizes the
# output tile so that (experts in use) x (output tiles) reaches the CU count,
# then takes the fewest of 2, 4 or 6 slots of 16 outputs per wave that cover
# the tile (f32 weights: at most 4). With 64 experts in use:
#   n = 120  -> 64-wide tiles            -> 2 slots
#   n = 1000 -> 256-wide tiles           -> 4 slots
#   n = 1408 -> 352-wide tiles (2-byte)  -> 6 slots; f32: 240-wide -> 4 slots
#   n = 1040 -> 272-wide tiles (2-byte)  -> 6 slots; f32: 208-wide -> 4 slots
# bf16 and f16 tiles that need 6 slots on 4 waves run on 8 waves with 3 slots each.
# (wdt, (m, n, k, top_k, E), slots on 4 waves)
FRAG_CASES = [
    (wl.BF16, (64, 120, 256, 4, 64), 2), (wl.F16, (64, 120, 256, 4, 64), 2),
    (wl.F32, (64, 120, 256, 4, 64), 2),
    (wl.BF16, (64, 1000, 256, 4, 64), 4), (wl.F16, (64, 1000, 256, 4, 64), 4),
    (wl.F32, (64, 1000, 256, 4, 64), 4),
    (wl.BF16, (64, 1408, 256, 4, 64), 6), (wl.F16, (64, 1408, 256, 4, 64), 6),
    (wl.F32, (64, 1408, 256, 4, 64), 4),
]


def grouped_variant(wdt, slots):
    """Receipt variant of the pipelined grouped kernel for a tile that needs
    `slots` 16-output fragments per wave on 4 waves: bf16 and f16 tiles
    needing 6 run on 8 waves with 3 slots each (3 + 256 * 8), every other
    case reports its slot count."""
    return 3 | (8 << 8) if wdt in (wl.BF16, wl.F16) and slots == 6 else slots


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("wdt,shape,slots", FRAG_CASES)
def test_grouped_fragment_slots(wdt, shape, slots, layout):
    """Every fragment-slot instance of the pipelined grouped kernel, every
    weight dtype, both activation layouts, ragged tile edges (n not a
    multiple of the tile width), out-of-range ids: all routed rows against
    the oracle; the receipt names the instance that ran."""
    m, n, k, top_k, E = shape
    _say(f"grouped slots={slots} wdt={wl.DTYPE_NAMES[wdt]} layout={layout} shape={shape}")
    case = _with_bad_ids(wl.random_id_case(100 + n, wdt, m, n, k, top_k, E, layout=layout))
    run = IdRun(case, route=1)
    rec = run.run()
    assert rec.kernel == mm.MM_KERNEL_ID_GROUPED_MFMA, rec.kernel
    assert rec.variant == grouped_variant(wdt, slots), f"variant {rec.variant}, slots {slots}"
    _check_map(run)
    _check_all_rows(run, f"grouped slots={slots}")


@pytest.mark.parametrize("wdt", DTYPES)
@pytest.mark.parametrize("layout", [0, 1])
def test_grouped_max_experts_pipelined(wdt, layout):
    """The expert limit (1024) on the pipelined grouped kernel: 512 routed
    rows over 1024 experts, 272-wide tiles (2-byte weights: the 8-wave
    instance, whose 512 threads rebuild the tile schedule from 1024 counts at
    two experts each; f32: 4 waves), out-of-range ids, every routed row
    against the oracle."""
    m, n, k, top_k, E = 64, 272, 128, 8, 1024
    _say(f"grouped max experts wdt={wl.DTYPE_NAMES[wdt]} layout={layout} E={E}")
    case = _with_bad_ids(wl.random_id_case(90, wdt, m, n, k, top_k, E, layout=layout))
    run = IdRun(case, route=1)
    rec = run.run()
    assert rec.kernel == mm.MM_KERNEL_ID_GROUPED_MFMA, rec.kernel
    if wdt != wl.F32:
        assert rec.variant == 3 | (8 << 8), rec.variant
    _check_map(run)
    _check_all_rows(run, "grouped max experts")


@pytest.mark.parametrize("wdt,slots", [(wl.BF16, 6), (wl.F16, 6), (wl.F32, 4)])
def test_grouped_wide_tiles_full_row_tiles_ramp_exact(wdt, slots):
    """The widest tile of each weight dtype with more than 128 routed rows per
    expert (full 128-row tiles, several row tiles per expert, a ragged last
    one): ramp inputs make every partial sum exact, so the output equals the
    rounded oracle bit for bit."""
    m, n, k, top_k, E = 1024, 1040, 256, 8, 64
    _say(f"grouped ramp exact slots={slots} wdt={wl.DTYPE_NAMES[wdt]} m={m} n={n} k={k}")
    rng = np.random.default_rng(72)
    w = wl.ramp(E * n * k, 5).reshape(E, n, k)
    x = wl.ramp(m * k, 6).reshape(m, k)
    ids = wl.distinct_ids(rng, m, top_k, E)
    case = wl.make_id_case(wdt, w, x, ids)
    run = IdRun(case, route=1)
    rec = run.run()
    assert rec.kernel == mm.MM_KERNEL_ID_GROUPED_MFMA and rec.variant == grouped_variant(wdt, slots), \
        (rec.kernel, rec.variant)
    counts, _ = run.scratch()
    assert counts.max() > 128
    got = from_dev(run.out, np.float32).reshape(m * top_k, n)
    ref = oracle.round_to(wl.F32, run.oracle())
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("wdt", DTYPES)
@pytest.mark.parametrize("layout", [0, 1])
def test_direct_staged_instances_ramp_exact(wdt, layout):
    """The direct route's staged kernel: activation row in LDS (variant 1), and
    with the slotted layout and one weight group per row (k = 2048 for 2-byte
    weights, 1024 for f32) the first slot naming an expert also computes the
    later slots naming it (variant 2). Many repeats per token, an
    out-of-range id; ramp inputs make the output exact, compared bit for bit."""
    m, n, top_k, E = 3, 40, 12, 3
    k = 1024 if wdt == wl.F32 else 2048
    rng = np.random.default_rng(73)
    w = wl.ramp(E * n * k, 7).reshape(E, n, k)
    rows = m if layout == 0 else m * top_k
    x = wl.ramp(rows * k, 8).reshape(rows, k)
    ids = rng.integers(0, E, (m, top_k)).astype(np.uint32)
    ids[1, 5] = E + 1
    case = wl.make_id_case(wdt, w, x, ids, layout=layout)
    _say(f"direct staged wdt={wl.DTYPE_NAMES[wdt]} layout={layout}")
    run = IdRun(case, route=0)
    rec = run.run()
    assert rec.kernel == mm.MM_KERNEL_ID_DIRECT_FAST, rec.kernel
    assert rec.variant == (2 if layout == 1 else 1), rec.variant
    got = from_dev(run.out, np.float32).reshape(m * top_k, n)
    ref = oracle.round_to(wl.F32, run.oracle())
    np.testing.assert_array_equal(got, ref)


def test_direct_repeats_and_dedup_rows_identical():
    m, n, k, top_k, E = 2, 300, 512, 8, 5
    _say("direct repeats")
    rng = np.random.default_rng(80)
    case = wl.random_id_case(81, wl.BF16, m, n, k, top_k, E, distinct=False)
    case.ids[:] = np.array([[3, 1, 3, 3, 0, 1, 4, 3], [2, 2, 2, 2, 2, 2, 2, 2]], dtype=np.uint32)
    run = IdRun(case, route=0)
    run.run()
    got = run.out_f64().reshape(m, top_k, n)
    assert np.array_equal(got[0, 0], got[0, 2]) and np.array_equal(got[0, 0], got[0, 7])
    assert all(np.array_equal(got[1, 0], got[1, s]) for s in range(top_k))
    _check_all_rows(run, "repeats")


def test_grouped_scratch_reuse_smaller_second_call():
    """A second prefill on the same scratch with fewer tokens sees only its own lists."""
    _say("scratch reuse")
    big = wl.random_id_case(90, wl.BF16, 64, 96, 128, 4, 8)
    run = IdRun(big, route=1)
    run.run()
    _check_all_rows(run, "first")
    small = wl.random_id_case(91, wl.BF16, 10, 96, 128, 4, 8)
    p = mm.id_params(small.m, small.n, small.k, small.top_k, small.n_experts,
                     small.expert_stride_bytes, 0, 0, 1)
    w, x, ids = to_dev(small.W), to_dev(small.X.reshape(-1)), to_dev(small.ids.reshape(-1))
    out = to_dev(np.full(small.m * small.top_k * small.n, np.nan, dtype=np.float32))
    mm.mm_id(p, wl.BF16, mm.buf(w), mm.buf(x), mm.buf(ids), mm.buf(out), mm.buf(run.counts),
             mm.buf(run.routed), stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    got = from_dev(out, np.float32).astype(np.float64).reshape(-1, small.n)
    ref = oracle.matmul_id(small.wdtype, small.m, small.n, small.k, small.top_k, small.n_experts,
                           small.expert_stride_bytes, 0, small.W, small.X, small.ids)
    assert_close(got, ref, wl.BF16, small.k, float(np.abs(wl.storage_to_float(small.W, wl.BF16)).max()),
                 float(np.abs(small.X).max()), "second call")


def test_all_ids_invalid():
    _say("all ids invalid")
    case = wl.random_id_case(95, wl.BF16, 6, 40, 64, 2, 4)
    case.ids[:] = 9
    for route in (0, 1):
        run = IdRun(case, route=route)
        run.run()
        got = run.out_f64()
        assert np.all(got == 0.0) and not np.any(np.signbit(got))
        if route == 1:
            counts, _ = run.scratch()
            assert np.all(counts == 0)
