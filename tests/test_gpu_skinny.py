"""GPU parity of the skinny route (a few rows on one side of C = A . B^T)
against the oracle.

Shapes follow the pages' skinny tests (tract-metal mlx_gemm/mod.rs,
`gemv_wide_tests`: m = 2..15 at n = 128, k = 256 in f16, m in {2, 5, 8, 15}
in f32, and the tail-row cases) on the same ramp inputs, which keep every
partial sum exact so the comparison is bit for bit; random operands add
m = 16 to 64 (one activation fragment per 16 rows), the mirrored case (n
small, m large), contraction tails, batches,
broadcast operands, padded leading dimensions and byte offsets. Layouts the
route does not take (misaligned offsets, k not a whole number of 16-byte
chunks) must fall through to the other routes and stay correct.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import gemv_expert_id_amd as mm
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

DTYPES = [wl.F32, wl.F16, wl.BF16]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield


from gpu_util import GemmRun, check_gemm, expected_gemm_route  # noqa: E402


def _ramp_case(dt, m, n, k, **layout):
    """The pages' skinny-test operands: a = ramp([m, k], 1), b = ramp([n, k], 2)."""
    a = wl.ramp(m * k, 1).reshape(1, m, k)
    b = wl.ramp(n * k, 2).reshape(1, n, k)
    return wl.make_gemm_case(dt, a, b, False, True, **layout)


def _run(case, exact, what):
    rec = check_gemm(case, exact=exact, what=what)
    assert rec.route == expected_gemm_route(case), (what, rec.route)
    if rec.route == mm.MM_ROUTE_GEMV_WIDE:
        assert rec.kernel == mm.MM_KERNEL_GEMV_WIDE and rec.dispatch_count == 1
    return rec


@pytest.mark.parametrize("dt", [wl.F16, wl.BF16])
@pytest.mark.parametrize("m", list(range(2, 17)))
def test_page_skinny_ramp_exact(dt, m):
    _say(f"skinny ramp {wl.DTYPE_NAMES[dt]} m={m} n=128 k=256")
    rec = _run(_ramp_case(dt, m, 128, 256), True, f"m={m}")
    assert rec.route == mm.MM_ROUTE_GEMV_WIDE


@pytest.mark.parametrize("m", [2, 5, 8, 15, 16])
def test_page_skinny_f32_ramp_exact(m):
    _say(f"skinny ramp f32 m={m} n=128 k=256")
    rec = _run(_ramp_case(wl.F32, m, 128, 256), True, f"m={m}")
    assert rec.route == mm.MM_ROUTE_GEMV_WIDE


@pytest.mark.parametrize("dt,m,n,k", [(wl.F16, 3, 130, 260), (wl.F16, 7, 63, 2048),
                                      (wl.F32, 4, 2, 512), (wl.BF16, 9, 17, 72),
                                      (wl.F32, 16, 33, 4), (wl.F16, 2, 2, 8)])
def test_page_skinny_tails_ramp_exact(dt, m, n, k):
    """The pages' tail-row cases (ragged n, k a few chunks past a step) plus
    the smallest shapes: one 16-byte chunk of contraction, two outputs."""
    _say(f"skinny tails {wl.DTYPE_NAMES[dt]} m={m} n={n} k={k}")
    _run(_ramp_case(dt, m, n, k), True, f"{m}x{n}x{k}")


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("m", [17, 24, 32, 33, 45, 48, 49, 63, 64])
def test_skinny_fragments_ramp_exact(dt, m):
    """17 to 64 rows: one activation fragment per 16 rows (receipt variant
    2, 3 or 4), ragged n and k tails, bit for bit on ramp inputs."""
    _say(f"skinny fragments {wl.DTYPE_NAMES[dt]} m={m}")
    rec = _run(_ramp_case(dt, m, 130, 264), True, f"{m}x130x264")
    assert rec.route == mm.MM_ROUTE_GEMV_WIDE and rec.variant == (m + 15) // 16, (rec.route, rec.variant)


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("m,n,k", [(16, 1000, 1024), (5, 4099, 264), (2, 64, 4096),
                                   (300, 5, 256), (4097, 16, 136), (12, 12, 40),
                                   (32, 1000, 1024), (20, 4099, 264), (300, 29, 256),
                                   (18, 24, 40), (64, 1000, 1024), (40, 4099, 264),
                                   (300, 57, 256)])
def test_skinny_random(dt, m, n, k):
    """Random operands, both roles: few rows in A (m <= 64) or in B (n <= 64)."""
    _say(f"skinny random {wl.DTYPE_NAMES[dt]} m={m} n={n} k={k}")
    case = wl.random_gemm_case(31, dt, 1, m, n, k, False, True)
    rec = _run(case, False, f"{m}x{n}x{k}")
    assert rec.route == mm.MM_ROUTE_GEMV_WIDE


@pytest.mark.parametrize("dt", DTYPES)
def test_skinny_batched_padded_offsets(dt):
    """Batch strides, padded lda/ldb/ldc, 16-byte offsets and a C stride."""
    ch = 16 // wl.ELT[dt]
    _say(f"skinny batched padded {wl.DTYPE_NAMES[dt]}")
    rng = np.random.default_rng(32)
    a = rng.standard_normal((3, 6, 96))
    b = rng.standard_normal((3, 211, 96)) / np.sqrt(96)
    case = wl.make_gemm_case(dt, a, b, False, True, lda=96 + 2 * ch, ldb=96 + ch, ldc=230,
                             off_a=ch, off_b=3 * ch, off_c=5, stride_c=6 * 230 + 17)
    rec = _run(case, False, "batched padded")
    assert rec.route == mm.MM_ROUTE_GEMV_WIDE


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("which", ["a", "b"])
def test_skinny_broadcast(dt, which):
    """One operand shared by every batch (batch stride 0)."""
    _say(f"skinny broadcast {which} {wl.DTYPE_NAMES[dt]}")
    rng = np.random.default_rng(33)
    a = rng.standard_normal((4, 8, 64)) if which == "b" else rng.standard_normal((1, 8, 64))
    b = rng.standard_normal((1, 100, 64)) if which == "b" else rng.standard_normal((4, 100, 64))
    case = wl.make_gemm_case(dt, a, b / 8.0, False, True, broadcast_a=(which == "a"),
                             broadcast_b=(which == "b"))
    rec = _run(case, False, f"broadcast {which}")
    assert rec.route == mm.MM_ROUTE_GEMV_WIDE


@pytest.mark.parametrize("dt,batch,m,n,k", [
    (wl.F16, 32, 64, 512, 64), (wl.F16, 32, 4, 512, 256), (wl.F16, 32, 4, 512, 128),
    (wl.BF16, 3, 40, 4096, 64), (wl.BF16, 4, 40, 4096, 64),
    (wl.F32, 16, 20, 2048, 256), (wl.F32, 16, 20, 2048, 128)])
def test_skinny_rounds_rule_both_sides(dt, batch, m, n, k):
    """Batched shapes on both sides of the skinny route's rounds rule (its
    blocks in more than one round: kept for long rows or few rounds, else
    the tiled GEMM): the receipt names the route the rule picks, and every
    output matches the oracle."""
    _say(f"skinny rounds rule {wl.DTYPE_NAMES[dt]} batch={batch} m={m} n={n} k={k}")
    case = wl.random_gemm_case(39 + k, dt, batch, m, n, k, False, True)
    _run(case, False, f"rounds {batch}x{m}x{n}x{k}")


@pytest.mark.parametrize("dt", [wl.F16, wl.BF16])
def test_layouts_the_route_declines(dt):
    """Not a whole number of 16-byte chunks (k = 36), an offset off the
    16-byte grid, or another transpose layout: the GEMM route takes them."""
    _say(f"skinny declined layouts {wl.DTYPE_NAMES[dt]}")
    rng = np.random.default_rng(34)
    cases = [
        wl.random_gemm_case(35, dt, 1, 4, 300, 36, False, True),
        wl.make_gemm_case(dt, rng.standard_normal((1, 4, 64)), rng.standard_normal((1, 300, 64)) / 8,
                          False, True, off_b=1),
        wl.random_gemm_case(36, dt, 1, 4, 300, 64, False, False),
        wl.random_gemm_case(37, dt, 1, 4, 300, 64, True, True),
    ]
    for i, case in enumerate(cases):
        rec = _run(case, False, f"declined {i}")
        assert rec.route == mm.MM_ROUTE_GEMM, i


def test_skinny_decode_shape_sampled():
    """x[8, 4096] . W[11008, 4096]^T in f16, the launch the benchmark times:
    every row at 512 sampled output columns (plus both ends) against the
    oracle, all outputs written, and the NaN sentinel around C untouched."""
    from gpu_util import assert_close
    _say("skinny f16 8 x 4096 . 11008 x 4096^T sampled")
    case = wl.gemv_f16_skinny()
    run = GemmRun(case)
    rec = run.run()
    assert rec.route == mm.MM_ROUTE_GEMV_WIDE and rec.kernel == mm.MM_KERNEL_GEMV_WIDE
    bits = run.c_bits()
    vals, mask = run.logical_c(bits)
    run.check_untouched(bits, mask)
    assert np.all(np.isfinite(vals)), "an output element was not written"
    rng = np.random.default_rng(38)
    cols = np.concatenate([[0, case.n - 1], rng.choice(case.n, 512, replace=False)])
    is_ = np.repeat(np.arange(case.m), cols.size)
    js = np.tile(cols, case.m)
    bs = np.zeros_like(is_)
    ref = oracle.gemm_at(case.dtype, case.k, case.trans_a, case.trans_b, case.lda, case.ldb,
                         case.stride_a, case.stride_b, case.off_a, case.off_b, case.A, case.B,
                         bs, is_, js)
    amax, bmax = run.operand_absmax()
    assert_close(vals[0, is_, js], ref, case.dtype, case.k, amax, bmax, "skinny decode shape")
