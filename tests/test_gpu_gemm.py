"""GPU parity of the matrix-product dispatch (GEMV and GEMM routes) against the oracle.

Shapes follow the pages' tests (tract-metal mlx_gemm/mod.rs `test_mat_vec`,
`test_mat_mul`, `gemv_wide_tests`) plus ragged multi-tile cases, every
transpose layout, padded leading dimensions, byte offsets, batch strides and
broadcast operands. Floating-point results meet the normalised tolerance;
ramp and permutation inputs are compared bit for bit.
"""
from __future__ import annotations

import itertools
import sys

import numpy as np
import pytest

import gemv_expert_id_amd as mm
import workloads as wl

pytestmark = pytest.mark.gpu

DTYPES = [wl.F32, wl.F16, wl.BF16]
LAYOUTS = list(itertools.product([False, True], [False, True]))


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    caps = mm.mm_capabilities(0)
    _say(f"device {caps.arch.decode()} cus={caps.cu_count} clock={caps.max_clock_mhz}MHz")
    yield


from gpu_util import check_gemm, expected_gemm_route  # noqa: E402


# (batch, m, n, k) tuples, both readings of the pages' (b, m, k, n)-or-(b, m, n, k) order.
PAGE_SHAPES = [
    ((1, 4, 4, 1), False, False), ((10, 1, 4, 4), False, False), ((5, 1, 15, 7), False, True),
    ((1, 3, 5, 4), False, False), ((1, 2, 5, 10), False, True), ((1, 4, 4, 4), False, True),
    ((1, 4, 4, 200), False, True), ((1, 25, 1280, 32000), False, True),
]


@pytest.mark.parametrize("shape,ta,tb", PAGE_SHAPES)
@pytest.mark.parametrize("order", ["bmkn", "bmnk"])
def test_page_shapes_f32(shape, ta, tb, order):
    b, m, x, y = shape
    k, n = (x, y) if order == "bmkn" else (y, x)
    _say(f"page shape {shape} order={order} -> b={b} m={m} n={n} k={k} ta={ta} tb={tb}")
    case = wl.random_gemm_case(7, wl.F32, b, m, n, k, ta, tb)
    rec = check_gemm(case, what=f"{shape}")
    assert rec.route == expected_gemm_route(case)
    assert rec.dispatch_count == 1


def test_lm_head_shape_f32():
    """(1, 25, 1280, 32000) + tB read as m=25, k=1280, n=32000 (LM-head shape)."""
    _say("lm head f32 m=25 k=1280 n=32000")
    case = wl.random_gemm_case(8, wl.F32, 1, 25, 32000, 1280, False, True)
    check_gemm(case, what="lm-head")


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", [(1, 17, 33, 1), (3, 100, 70, 77), (1, 128, 128, 128),
                                   (2, 5, 513, 3), (1, 512, 512, 4)])
def test_f32_small_kernel(ta, tb, shape):
    """f32 with k <= 128 and at most 1024 tiles of 16 x 16: one wave per tile on
    f32 MFMA; ragged m, n, k (including k = 1 and k % 4 != 0), padded leading
    dimensions and offsets; random operands to the tolerance, ramp bit for bit."""
    b, m, n, k = shape
    _say(f"f32 small kernel ta={ta} tb={tb} shape={shape}")
    case = wl.random_gemm_case(90, wl.F32, b, m, n, k, ta, tb, dist="uniform",
                               lda=(m if ta else k) + 3, ldb=(k if tb else n) + 5, off_a=2, off_b=1)
    rec = check_gemm(case, what=f"{shape}")
    assert rec.kernel == mm.MM_KERNEL_GEMM_F32_SMALL, rec.kernel
    a_shape = (b, k, m) if ta else (b, m, k)
    b_shape = (b, n, k) if tb else (b, k, n)
    ramp = wl.make_gemm_case(wl.F32, wl.ramp(int(np.prod(a_shape)), 1).reshape(a_shape),
                             wl.ramp(int(np.prod(b_shape)), 2).reshape(b_shape), ta, tb)
    check_gemm(ramp, exact=True, what=f"ramp {shape}")


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_f32_wide_tiles_ragged(ta, tb):
    """Enough 64 x 64 tiles for the wide f32 form (smaller problems use 32 x 32),
    ragged in m, n and k."""
    _say(f"f32 wide tiles m=1030 n=1100 k=70 ta={ta} tb={tb}")
    case = wl.random_gemm_case(12, wl.F32, 1, 1030, 1100, 70, ta, tb)
    rec = check_gemm(case, what="f32 wide")
    assert rec.kernel == mm.MM_KERNEL_GEMM_F32


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", [(1, 130, 260, 70), (3, 257, 129, 95), (2, 64, 48, 300),
                                   (1, 2, 256, 128), (1, 15, 256, 128), (2, 200, 3, 17)])
def test_gemm_layouts_ragged(dt, ta, tb, shape):
    b, m, n, k = shape
    _say(f"gemm dt={wl.DTYPE_NAMES[dt]} ta={ta} tb={tb} b={b} m={m} n={n} k={k}")
    case = wl.random_gemm_case(11 + m, dt, b, m, n, k, ta, tb)
    check_gemm(case, what=f"{dt} {ta} {tb} {shape}")


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_gemm_padded_offsets_strides(dt, ta, tb):
    rng = np.random.default_rng(3)
    b, m, n, k = 3, 70, 90, 45
    a = rng.standard_normal((b, k, m) if ta else (b, m, k))
    bb = rng.standard_normal((b, n, k) if tb else (b, k, n)) / np.sqrt(k)
    case = wl.make_gemm_case(dt, a, bb, ta, tb, lda=a.shape[2] + 5, ldb=bb.shape[2] + 3,
                             ldc=n + 6, off_a=3, off_b=5, off_c=1,
                             stride_a=a.shape[1] * (a.shape[2] + 5) + 11,
                             stride_c=m * (n + 6) + 9)
    _say(f"gemm padded dt={wl.DTYPE_NAMES[dt]} ta={ta} tb={tb}")
    check_gemm(case, what="padded")


@pytest.mark.parametrize("dt", DTYPES)
def test_gemm_broadcast_operands(dt):
    rng = np.random.default_rng(4)
    b, m, n, k = 4, 33, 65, 40
    a = rng.standard_normal((1, m, k))
    bb = rng.standard_normal((b, n, k)) / np.sqrt(k)
    case = wl.make_gemm_case(dt, np.broadcast_to(a, (b, m, k)), bb, False, True, broadcast_a=True)
    _say(f"gemm broadcast A dt={wl.DTYPE_NAMES[dt]}")
    check_gemm(case, what="broadcast A")
    bb1 = rng.standard_normal((1, k, n)) / np.sqrt(k)
    a4 = rng.standard_normal((b, m, k))
    case = wl.make_gemm_case(dt, a4, np.broadcast_to(bb1, (b, k, n)), False, False,
                             broadcast_b=True)
    _say(f"gemm broadcast B dt={wl.DTYPE_NAMES[dt]}")
    check_gemm(case, what="broadcast B")


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", [(2, 1, 300, 129), (3, 257, 1, 64), (1, 1, 1, 77),
                                   (1, 1, 4099, 520), (2, 1030, 1, 33)])
def test_gemv_route(dt, ta, tb, shape):
    b, m, n, k = shape
    _say(f"gemv dt={wl.DTYPE_NAMES[dt]} ta={ta} tb={tb} b={b} m={m} n={n} k={k}")
    case = wl.random_gemm_case(21 + n, dt, b, m, n, k, ta, tb)
    rec = check_gemm(case, entry=mm.mm_gemv, what="gemv")
    assert rec.route == mm.MM_ROUTE_GEMV


@pytest.mark.parametrize("dt", DTYPES)
def test_gemv_padded_strided(dt):
    rng = np.random.default_rng(5)
    # m == 1, A stored transposed [k, 1] with lda > 1: a strided vector.
    b, m, n, k = 2, 1, 301, 200
    a = rng.standard_normal((b, k, m))
    bb = rng.standard_normal((b, n, k)) / np.sqrt(k)
    case = wl.make_gemm_case(dt, a, bb, True, True, lda=3, ldb=k + 8, off_a=1, off_b=2, off_c=3)
    _say(f"gemv strided vector dt={wl.DTYPE_NAMES[dt]}")
    check_gemm(case, what="strided vector")
    # n == 1: output stride ldc > 1.
    b, m, n, k = 2, 150, 1, 130
    a = rng.standard_normal((b, m, k))
    bb = rng.standard_normal((b, k, n)) / np.sqrt(k)
    case = wl.make_gemm_case(dt, a, bb, False, False, ldc=5, ldb=2)
    _say(f"gemv strided output dt={wl.DTYPE_NAMES[dt]}")
    check_gemm(case, what="strided output")


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", [(1, 3, 130, 260), (1, 7, 63, 2048), (2, 4, 2, 512),
                                   (1, 1, 1000, 4096), (1, 1000, 1, 4096), (2, 129, 131, 257)])
def test_ramp_bit_exact(dt, ta, tb, shape):
    """Ramp inputs (tract-metal gemv_wide tests): all partial sums are exact in
    f32, so every route must reproduce the rounded oracle bit for bit."""
    b, m, n, k = shape
    a = wl.ramp(b * m * k, 1).reshape((b, k, m) if ta else (b, m, k))
    bb = wl.ramp(b * n * k, 2).reshape((b, n, k) if tb else (b, k, n))
    case = wl.make_gemm_case(dt, a, bb, ta, tb)
    _say(f"ramp dt={wl.DTYPE_NAMES[dt]} ta={ta} tb={tb} shape={shape}")
    check_gemm(case, exact=True, what="ramp")


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_permutation_bit_exact(dt, ta, tb):
    rng = np.random.default_rng(6)
    b, m, k = 2, 70, 96
    n = k
    a_log = rng.standard_normal((b, m, k))
    p = np.zeros((b, k, n))
    for i in range(b):
        p[i, rng.permutation(k), np.arange(n)] = 1.0
    case = wl.make_gemm_case(dt, a_log.transpose(0, 2, 1) if ta else a_log,
                             p.transpose(0, 2, 1) if tb else p, ta, tb)
    _say(f"permutation dt={wl.DTYPE_NAMES[dt]} ta={ta} tb={tb}")
    check_gemm(case, exact=True, what="permutation")


def test_all_ones_page_example():
    """(10, 32, 32, 16) all ones -> 16 everywhere (tract-metal `test_mlx_gemm`)."""
    for dt in DTYPES:
        case = wl.make_gemm_case(dt, np.ones((10, 32, 16)), np.ones((10, 16, 32)), False, False)
        _say(f"all ones dt={wl.DTYPE_NAMES[dt]}")
        check_gemm(case, exact=True, what="all ones")


def test_worked_example_page():
    """Ramp 0.. (2, 2, 4, 3) -> the 16 values printed in tract-metal `test_mlx_gemm`."""
    a = np.arange(12, dtype=np.float64).reshape(2, 2, 3)
    b = np.arange(24, dtype=np.float64).reshape(2, 3, 4)
    for dt in DTYPES:
        case = wl.make_gemm_case(dt, a, b, False, False)
        _say(f"worked example dt={wl.DTYPE_NAMES[dt]}")
        check_gemm(case, exact=True, what="worked example")


def test_large_k_many_tiles_f16():
    _say("f16 NT m=300 n=520 k=4100")
    case = wl.random_gemm_case(31, wl.F16, 1, 300, 520, 4100, False, True)
    check_gemm(case, what="large k")


def _sampled_check(case, n_samples, seed, exact=False, kernel=None, variant=None):
    from gpu_util import GemmRun, assert_close
    import oracle
    run = GemmRun(case)
    rec = run.run()
    if kernel is not None:
        assert rec.kernel == kernel, f"kernel {rec.kernel}, expected {kernel}"
    if variant is not None:
        # (the large kernel's low bit names its paired-stage form)
        got = rec.variant & ~1 if rec.kernel == mm.MM_KERNEL_GEMM_LARGE else rec.variant
        assert got == variant, f"variant {rec.variant}, expected {variant}"
    bits = run.c_bits()
    rng = np.random.default_rng(seed)
    bs = rng.integers(0, case.batch, n_samples)
    is_ = np.concatenate([rng.integers(0, case.m, n_samples), [0, case.m - 1]])
    js = np.concatenate([rng.integers(0, case.n, n_samples), [case.n - 1, 0]])
    bs = np.concatenate([bs, [0, case.batch - 1]])
    ref = oracle.gemm_at(case.dtype, case.k, case.trans_a, case.trans_b, case.lda, case.ldb,
                         case.stride_a, case.stride_b, case.off_a, case.off_b, case.A, case.B,
                         bs, is_, js)
    idx = case.off_c // wl.ELT[case.dtype] + bs * case.stride_c + is_ * case.ldc + js
    got = oracle.decode(case.dtype, bits[idx])
    if exact:
        np.testing.assert_array_equal(got, oracle.decode(case.dtype, oracle.round_to(case.dtype, ref)))
    else:
        amax, bmax = run.operand_absmax()
        assert_close(got, ref, case.dtype, case.k, amax, bmax, "sampled")
    vals, _ = run.logical_c(bits)
    assert np.all(np.isfinite(vals)), "an output element was not written"


@pytest.mark.parametrize("dt", [wl.F16, wl.BF16])
@pytest.mark.parametrize("k", [256, 640])
def test_large_tile_route(dt, k):
    """m, n multiples of 256 with >= 128 tiles, k % 128 == 0, k >= 256: the
    256 x 256 MFMA kernel (k = 256: first and last rounds only; k = 640: the
    steady loop runs too)."""
    _say(f"large-tile NT dt={wl.DTYPE_NAMES[dt]} m=4096 n=8192 k={k}")
    case = wl.random_gemm_case(41, dt, 1, 4096, 8192, k, False, True)
    _sampled_check(case, 4096, 3, kernel=mm.MM_KERNEL_GEMM_LARGE, variant=256)


def test_large_tile_route_ramp_exact():
    _say("large-tile NT ramp exact m=8192 n=4096 k=384")
    m, n, k = 8192, 4096, 384
    a = wl.ramp(m * k, 1).reshape(1, m, k)
    b = wl.ramp(n * k, 2).reshape(1, n, k)
    case = wl.make_gemm_case(wl.F16, a, b, False, True)
    _sampled_check(case, 4096, 4, exact=True, kernel=mm.MM_KERNEL_GEMM_LARGE, variant=256)


@pytest.mark.parametrize("dt,b,m,n,k,kernel,variant", [
    (wl.F16, 1, 3072, 4096, 256, mm.MM_KERNEL_GEMM_LARGE, 256),  # 192 tiles of 256 x 256
    (wl.F16, 1, 2048, 4096, 256, mm.MM_KERNEL_GEMM_LARGE, 128),  # 128 of them: 128 x 128 tiles
    (wl.BF16, 2, 2048, 2048, 384, mm.MM_KERNEL_GEMM_LARGE, 128),  # 64 per batch item
    (wl.F16, 1, 1024, 2048, 512, mm.MM_KERNEL_GEMM_LARGE, 128),
    (wl.BF16, 3, 384, 640, 256, mm.MM_KERNEL_GEMM_LARGE, 128),   # 15 tiles per batch item
    (wl.F16, 1, 128, 128, 1024, mm.MM_KERNEL_GEMM_LARGE, 128),   # a single tile
    (wl.F16, 1, 1000, 2048, 512, mm.MM_KERNEL_GEMM_LARGE, 128),  # m not a multiple of 128
    (wl.F16, 1, 1000, 2048, 320, mm.MM_KERNEL_GEMM_TILED, 0),    # k not a multiple of 128
])
def test_large_tile_threshold(dt, b, m, n, k, kernel, variant):
    """The pipelined kernel takes NT products with k a multiple of 128 and
    k >= 256: 256 x 256 tiles when at least 192 of them cover the batch, else
    128 x 128 tiles; other k go to the 128 x 128 register-staged kernel.
    Every output against the oracle; the receipt names the tile edge."""
    _say(f"large-tile threshold dt={wl.DTYPE_NAMES[dt]} b={b} m={m} n={n} k={k}")
    case = wl.random_gemm_case(46 + k, dt, b, m, n, k, False, True)
    rec = check_gemm(case, what=f"threshold {b}x{m}x{n}x{k}")
    got = rec.variant & ~1 if rec.kernel == mm.MM_KERNEL_GEMM_LARGE else rec.variant
    assert (rec.kernel, got) == (kernel, variant), (rec.kernel, rec.variant)


@pytest.mark.parametrize("dt,ta,tb,b,m,n,k", [
    (wl.F16, False, True, 1, 2304, 2048, 256),   # NT, 288 tiles of 128 x 128
    (wl.BF16, False, True, 1, 2300, 2052, 384),  # NT, ragged m and n, 306 tiles
    (wl.F16, False, True, 4, 1152, 1024, 256),   # NT, 72 tiles per batch item, 288 in all
    (wl.BF16, False, True, 1, 2432, 2304, 512),  # NT, the steady loop runs (k / 128 = 4 rounds)
    (wl.F16, False, False, 1, 2304, 2048, 512),  # NN: B K-strided
    (wl.BF16, True, True, 2, 1152, 2304, 256),   # TT: A K-strided, 162 tiles per item, 324 in all
])
def test_pair_kernel_128_tiles(dt, ta, tb, b, m, n, k):
    """Products with more 128 x 128 tiles than CUs take the paired-stage
    form of the pipelined kernel (two k-stages per LDS region, 128-byte
    pieces of K-contiguous operands; NT, and NN / TT when not ragged).
    Every output against the oracle."""
    _say(f"pair 128 dt={wl.DTYPE_NAMES[dt]} ta={int(ta)} tb={int(tb)} b={b} {m}x{n}x{k}")
    case = wl.random_gemm_case(90 + k % 7, dt, b, m, n, k, ta, tb)
    rec = check_gemm(case, what=f"pair {b}x{m}x{n}x{k}")
    assert (rec.kernel, rec.variant) == (mm.MM_KERNEL_GEMM_LARGE, 129), (rec.kernel, rec.variant)


@pytest.mark.parametrize("dt", [wl.F16, wl.BF16])
def test_pair_kernel_ramp_exact(dt):
    """The paired-stage form at 128 x 128 tiles, ramp inputs, bit for bit."""
    m, n, k = 2304, 2048, 256
    _say(f"pair 128 ramp exact dt={wl.DTYPE_NAMES[dt]} {m}x{n}x{k}")
    a = wl.ramp(m * k, 1).reshape(1, m, k)
    b = wl.ramp(n * k, 2).reshape(1, n, k)
    rec = check_gemm(wl.make_gemm_case(dt, a, b, False, True), exact=True, what="pair ramp")
    assert (rec.kernel, rec.variant) == (mm.MM_KERNEL_GEMM_LARGE, 129), (rec.kernel, rec.variant)


def test_pair_kernel_batched_padded_offsets():
    """The paired-stage form with padded leading dimensions, gapped batch
    strides and element offsets on every operand (270 tiles); every output."""
    _say("pair 128 batched padded bf16")
    rng = np.random.default_rng(14)
    b_, m, n, k = 3, 1280, 1152, 256
    a = rng.standard_normal((b_, m, k))
    bb = rng.standard_normal((b_, n, k)) / np.sqrt(k)
    case = wl.make_gemm_case(wl.BF16, a, bb, False, True, lda=k + 64, ldb=k + 8, ldc=n + 4,
                             off_a=8, off_b=16, off_c=4, stride_a=m * (k + 64) + 64,
                             stride_b=n * (k + 8) + 8, stride_c=m * (n + 4) + 12)
    rec = check_gemm(case, what="pair batched padded")
    assert (rec.kernel, rec.variant) == (mm.MM_KERNEL_GEMM_LARGE, 129), (rec.kernel, rec.variant)


@pytest.mark.parametrize("ta,tb,b,m,n,k,variant", [
    (False, True, 1, 3072, 4096, 256, 257),   # NT, 256 x 256 tiles: paired
    (False, True, 1, 2048, 4096, 256, 129),   # NT, 128 tiles of 256 (< 192): 512 of 128 x 128, paired
    (False, True, 1, 1024, 2048, 256, 128),   # NT, 128 tiles of 128 x 128: four stages
    (False, True, 1, 2304, 2048, 256, 129),   # NT, 288 tiles of 128 x 128: paired
    (False, True, 1, 4000, 3000, 256, 257),   # NT ragged: paired
    (False, False, 1, 3072, 4096, 256, 257),  # NN: paired
    (False, False, 1, 4000, 3000, 256, 256),  # NN ragged: four stages
    (True, True, 2, 1152, 2304, 256, 129),    # TT, 324 tiles of 128 x 128: paired
    (True, True, 2, 1152, 1280, 256, 128),    # TT, 180 tiles of 128 x 128: four stages
    (True, True, 1, 1000, 2304, 256, 128),    # TT ragged: four stages
    (True, False, 1, 3072, 4096, 256, 256),   # TN: four stages
    (False, True, 1, 1024, 2048, 512, 129),   # NT, 128 tiles, k % 256 == 0, k >= 512: four regions
    (False, False, 1, 1024, 2048, 512, 129),  # NN, the same
    (False, False, 1, 1000, 2048, 512, 128),  # NN ragged: four stages
    (True, False, 1, 1024, 2048, 512, 128),   # TN: four stages
    (False, True, 1, 1024, 2048, 384, 128),   # k not a multiple of 256: four stages
])
def test_pipelined_form_rule(ta, tb, b, m, n, k, variant):
    """The receipt names the pipelined kernel's tile edge and, in its low bit,
    the paired-stage form: NT with 256 x 256 tiles or more than 256 tiles of
    128 x 128, or (four regions) at most 256 of them with k a multiple of 256
    and at least 512; NN and TT the same unless ragged; TN never."""
    import torch
    from gpu_util import GemmRun
    _say(f"pipelined form rule ta={int(ta)} tb={int(tb)} b={b} {m}x{n}x{k}")
    case = wl.random_gemm_case(98, wl.F16, b, m, n, k, ta, tb)
    run = GemmRun(case)
    rec = run.run()
    torch.cuda.synchronize()
    assert (rec.kernel, rec.variant) == (mm.MM_KERNEL_GEMM_LARGE, variant), (rec.kernel, rec.variant)


@pytest.mark.parametrize("dt,ta,tb,b,m,n,k", [
    (wl.F16, False, True, 1, 512, 1024, 1024),   # NT, 32 tiles; the steady loop runs twice
    (wl.BF16, False, False, 1, 384, 640, 512),   # NN, first and last rounds only
    (wl.F16, True, True, 2, 256, 384, 1536),     # TT
    (wl.F16, False, True, 1, 200, 300, 512),     # NT ragged
    (wl.BF16, False, True, 3, 256, 128, 768),    # NT batched, one steady round
])
def test_pair_kernel_four_regions(dt, ta, tb, b, m, n, k):
    """At most one 128 x 128 tile per CU and k a multiple of 256 (>= 512):
    the paired-stage form with four LDS regions. Every output against the
    oracle."""
    _say(f"pair4 dt={wl.DTYPE_NAMES[dt]} ta={int(ta)} tb={int(tb)} b={b} {m}x{n}x{k}")
    case = wl.random_gemm_case(97 + k % 5, dt, b, m, n, k, ta, tb)
    rec = check_gemm(case, what=f"pair4 {b}x{m}x{n}x{k}")
    assert (rec.kernel, rec.variant) == (mm.MM_KERNEL_GEMM_LARGE, 129), (rec.kernel, rec.variant)


@pytest.mark.parametrize("dt", [wl.F16, wl.BF16])
def test_mid_tile_ramp_exact(dt):
    """128 x 128 tiles of the pipelined kernel (k = 1024: the steady loop
    runs), ramp inputs, every output bit for bit."""
    m, n, k = 384, 512, 1024
    _say(f"mid-tile NT ramp exact dt={wl.DTYPE_NAMES[dt]} m={m} n={n} k={k}")
    a = wl.ramp(m * k, 1).reshape(1, m, k)
    b = wl.ramp(n * k, 2).reshape(1, n, k)
    rec = check_gemm(wl.make_gemm_case(dt, a, b, False, True), exact=True, what="mid ramp")
    assert (rec.kernel, rec.variant & ~1) == (mm.MM_KERNEL_GEMM_LARGE, 128), (rec.kernel, rec.variant)


@pytest.mark.parametrize("dt", [wl.F16, wl.BF16])
def test_mid_tile_batched_padded_offsets(dt):
    """128 x 128 tiles with padded leading dimensions, batch strides with
    gaps and element offsets on every operand; every output."""
    _say(f"mid-tile NT batched padded dt={wl.DTYPE_NAMES[dt]}")
    rng = np.random.default_rng(12)
    b_, m, n, k = 3, 256, 640, 384
    a = rng.standard_normal((b_, m, k))
    bb = rng.standard_normal((b_, n, k)) / np.sqrt(k)
    case = wl.make_gemm_case(dt, a, bb, False, True, lda=k + 64, ldb=k + 8, ldc=n + 4,
                             off_a=8, off_b=16, off_c=4, stride_a=m * (k + 64) + 64,
                             stride_b=n * (k + 8) + 8, stride_c=m * (n + 4) + 12)
    rec = check_gemm(case, what="mid batched padded")
    assert (rec.kernel, rec.variant & ~1) == (mm.MM_KERNEL_GEMM_LARGE, 128), (rec.kernel, rec.variant)


def test_mid_tile_broadcast_b():
    """128 x 128 tiles, one B for a batch of four (batch stride 0)."""
    _say("mid-tile NT B broadcast f16 b=4 m=512 n=256 k=512")
    rng = np.random.default_rng(13)
    b_, m, n, k = 4, 512, 256, 512
    a = rng.uniform(-1, 1, (b_, m, k))
    b1 = rng.uniform(-1, 1, (1, n, k)) / np.sqrt(k)
    case = wl.make_gemm_case(wl.F16, a, np.broadcast_to(b1, (b_, n, k)), False, True,
                             broadcast_b=True)
    assert case.stride_b == 0
    rec = check_gemm(case, what="mid broadcast")
    assert (rec.kernel, rec.variant & ~1) == (mm.MM_KERNEL_GEMM_LARGE, 128), (rec.kernel, rec.variant)


LAYOUTS = [(False, True), (False, False), (True, True), (True, False)]  # (trans_a, trans_b)


@pytest.mark.parametrize("dt", [wl.F16, wl.BF16])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_pipelined_layouts_128_tiles(dt, ta, tb):
    """Every transpose layout on the pipelined kernel's 128 x 128 tiles: a
    K-strided operand (A stored [k, m], B stored [k, n]) lands k-major in
    LDS and reaches the MFMA through transposing LDS reads. Every output
    against the oracle; then ramp inputs bit for bit."""
    m, n, k = 384, 640, 512
    _say(f"pipelined 128 layouts dt={wl.DTYPE_NAMES[dt]} ta={int(ta)} tb={int(tb)} {m}x{n}x{k}")
    case = wl.random_gemm_case(60 + 2 * ta + tb, dt, 1, m, n, k, ta, tb)
    rec = check_gemm(case, what=f"layout {int(ta)}{int(tb)}")
    assert (rec.kernel, rec.variant & ~1) == (mm.MM_KERNEL_GEMM_LARGE, 128), (rec.kernel, rec.variant)
    a = wl.ramp(m * k, 1).reshape((1, k, m) if ta else (1, m, k))
    b = wl.ramp(n * k, 2).reshape((1, n, k) if tb else (1, k, n))
    rec = check_gemm(wl.make_gemm_case(dt, a, b, ta, tb), exact=True, what="layout ramp")
    assert (rec.kernel, rec.variant & ~1) == (mm.MM_KERNEL_GEMM_LARGE, 128), (rec.kernel, rec.variant)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_pipelined_layouts_batched_padded(ta, tb):
    """Every layout on 128 x 128 tiles with padded leading dimensions, batch
    strides with gaps and element offsets on every operand."""
    _say(f"pipelined layouts batched padded ta={int(ta)} tb={int(tb)}")
    rng = np.random.default_rng(14)
    b_, m, n, k = 3, 256, 384, 384
    a = rng.standard_normal((b_, k, m) if ta else (b_, m, k))
    bb = rng.standard_normal((b_, n, k) if tb else (b_, k, n)) / np.sqrt(k)
    lda = (m if ta else k) + 24
    ldb = (k if tb else n) + 40
    rows_a = k if ta else m
    rows_b = n if tb else k
    case = wl.make_gemm_case(wl.BF16, a, bb, ta, tb, lda=lda, ldb=ldb, ldc=n + 4, off_a=8,
                             off_b=16, off_c=4, stride_a=rows_a * lda + 64,
                             stride_b=rows_b * ldb + 8, stride_c=m * (n + 4) + 12)
    rec = check_gemm(case, what="layouts batched padded")
    assert (rec.kernel, rec.variant & ~1) == (mm.MM_KERNEL_GEMM_LARGE, 128), (rec.kernel, rec.variant)


@pytest.mark.parametrize("dt", [wl.F16, wl.BF16])
@pytest.mark.parametrize("ta,tb", LAYOUTS[1:])
@pytest.mark.parametrize("k", [256, 512])
def test_pipelined_layouts_256_tiles(dt, ta, tb, k):
    """NN, TN and TT products large enough for 256 x 256 tiles (192 of them),
    sampled against the oracle (NN and TT on the paired-stage form; k = 512
    runs its steady loop)."""
    m, n = 3072, 4096
    _say(f"pipelined 256 layouts dt={wl.DTYPE_NAMES[dt]} ta={int(ta)} tb={int(tb)} {m}x{n}x{k}")
    case = wl.random_gemm_case(64 + 2 * ta + tb, dt, 1, m, n, k, ta, tb)
    _sampled_check(case, 4096, 15, kernel=mm.MM_KERNEL_GEMM_LARGE, variant=256)


@pytest.mark.parametrize("dt,ta,tb,b,m,n,k,variant", [
    (wl.F16, False, True, 1, 1000, 3000, 512, 128),
    (wl.BF16, False, False, 1, 777, 1000, 256, 128),
    (wl.F16, True, False, 2, 304, 520, 384, 128),
    (wl.BF16, True, True, 1, 136, 200, 256, 128),
    (wl.F16, False, False, 1, 100, 704, 256, 128),    # fewer rows than one tile
    (wl.BF16, False, True, 3, 200, 72, 256, 128),     # fewer columns than one tile
])
def test_pipelined_ragged_edges(dt, ta, tb, b, m, n, k, variant):
    """m and n not multiples of the tile edge on the pipelined kernel: edge
    tiles read through buffer resources cut at each operand's extent and
    store only inside C. (A K-strided operand's rows must still be whole
    16-byte chunks, so its m or n is a multiple of 8.) Every output against
    the oracle, and the NaN sentinel around C untouched (check_gemm)."""
    _say(f"pipelined ragged dt={wl.DTYPE_NAMES[dt]} ta={int(ta)} tb={int(tb)} b={b} {m}x{n}x{k}")
    case = wl.random_gemm_case(70 + m % 7 + n % 5, dt, b, m, n, k, ta, tb)
    rec = check_gemm(case, what=f"ragged {b}x{m}x{n}x{k}")
    assert (rec.kernel, rec.variant & ~1) == (mm.MM_KERNEL_GEMM_LARGE, variant), (rec.kernel, rec.variant)


def test_pipelined_ragged_ramp_exact():
    """A ragged NT product on the pipelined kernel, ramp inputs, bit for bit."""
    m, n, k = 200, 136, 512
    _say(f"pipelined ragged ramp {m}x{n}x{k}")
    a = wl.ramp(m * k, 1).reshape(1, m, k)
    b = wl.ramp(n * k, 2).reshape(1, n, k)
    rec = check_gemm(wl.make_gemm_case(wl.F16, a, b, False, True), exact=True, what="ragged ramp")
    assert (rec.kernel, rec.variant & ~1) == (mm.MM_KERNEL_GEMM_LARGE, 128), (rec.kernel, rec.variant)


@pytest.mark.parametrize("ta,tb", [(False, True), (False, False)])
def test_pipelined_ragged_256_tiles(ta, tb):
    """A ragged product large enough for 256 x 256 tiles (16 x 12 = 192 of
    them), sampled against the oracle plus both ends of every row."""
    m, n, k = 4000, 3000, 256
    _say(f"pipelined ragged 256 ta={int(ta)} tb={int(tb)} {m}x{n}x{k}")
    case = wl.random_gemm_case(75 + tb, wl.F16, 1, m, n, k, ta, tb)
    _sampled_check(case, 4096, 16, kernel=mm.MM_KERNEL_GEMM_LARGE, variant=256)


def test_large_tile_route_batched_padded():
    _say("large-tile NT batched, padded ld, bf16 m=4096 n=4096 k=256 batch 2")
    rng = np.random.default_rng(9)
    b_, m, n, k = 2, 4096, 4096, 256
    a = rng.standard_normal((b_, m, k))
    bb = rng.standard_normal((b_, n, k)) / np.sqrt(k)
    case = wl.make_gemm_case(wl.BF16, a, bb, False, True, lda=k + 64, ldb=k + 8, ldc=n + 4)
    _sampled_check(case, 4096, 5, kernel=mm.MM_KERNEL_GEMM_LARGE, variant=256)


def test_large_tile_route_broadcast_b():
    """Batch of two with one B for both (batch stride 0) and element offsets on
    every operand, on the 256 x 256 kernel."""
    _say("large-tile NT batched, B broadcast, offsets, f16 m=4096 n=4096 k=256 batch 2")
    rng = np.random.default_rng(11)
    b_, m, n, k = 2, 4096, 4096, 256
    a = rng.uniform(-1, 1, (b_, m, k))
    b1 = rng.uniform(-1, 1, (1, n, k)) / np.sqrt(k)
    case = wl.make_gemm_case(wl.F16, a, np.broadcast_to(b1, (b_, n, k)), False, True,
                             broadcast_b=True, off_a=8, off_b=16, off_c=4)
    assert case.stride_b == 0
    _sampled_check(case, 4096, 7, kernel=mm.MM_KERNEL_GEMM_LARGE, variant=256)


@pytest.mark.parametrize("dt,seed", [(wl.F16, 44), (wl.BF16, 45)])
def test_large_tile_route_full_compare(dt, seed):
    """The 256 x 256 kernel at its smallest admissible size (512 tiles,
    k = 256) with every output compared against the oracle."""
    from gpu_util import GemmRun, assert_close
    _say(f"large-tile NT full compare dt={wl.DTYPE_NAMES[dt]} m=4096 n=8192 k=256")
    case = wl.random_gemm_case(seed, dt, 1, 4096, 8192, 256, False, True, dist="uniform")
    run = GemmRun(case)
    rec = run.run()
    assert rec.kernel == mm.MM_KERNEL_GEMM_LARGE and rec.variant & ~1 == 256, (rec.kernel, rec.variant)
    bits = run.c_bits()
    got, mask = run.logical_c(bits)
    run.check_untouched(bits, mask)
    amax, bmax = run.operand_absmax()
    err = assert_close(got, run.oracle_full(), case.dtype, case.k, amax, bmax, "large full")
    _say(f"  max err {err:.3e}")


def panel_variant(b, m, n, k):
    """(split, panel rows) the panel kernel takes: 128-row panels for k = 64
    or 128 when m % 128 == 0 and (m / 128) * b * most128 reaches 256 blocks,
    split to reach 256 blocks, where most128 is min(4, tiles) for up to 8
    tiles of 64 columns and min(16, tiles / 2) beyond; else 64-row panels
    split to reach 512 blocks, at most min(32, tiles) ways."""
    tiles = n // 64
    most128 = min(4, tiles) if tiles <= 8 else min(16, tiles // 2)
    tall = k >= 64 and m % 128 == 0 and (m // 128) * b * most128 >= 256
    pm = 128 if tall else 64
    items = (m // pm) * b
    want = 256 if tall else 512
    most = most128 if tall else min(32, tiles)
    return min(most, -(-want // items)), pm


def panel_taken(b, m, n, k):
    """Whether the panel kernel takes an aligned NT short-K product: at least
    128 panels of 64 rows, or few enough that up to min(32, n / 64) blocks
    each still reach 512."""
    items = (m // 64) * b
    return (k in (32, 64, 128) and m % 64 == 0 and n % 64 == 0
            and (items >= 128 or items * min(32, n // 64) >= 512))


def check_panel_variant(rec, b, m, n, k):
    assert rec.kernel == mm.MM_KERNEL_GEMM_PANEL, rec.kernel
    got = (rec.variant & 0xff, rec.variant >> 8)
    assert got == panel_variant(b, m, n, k), f"(split, panel rows) {got}"
    return got


@pytest.mark.parametrize("dt", [wl.F16, wl.BF16])
@pytest.mark.parametrize("k", [32, 64, 128])
@pytest.mark.parametrize("n", [128, 192, 384, 640, 1536])
def test_panel_kernel(dt, k, n):
    """Batched short-K NT products on the panel kernel (A panel resident in
    LDS, B tiles of 64 rows streamed through three stages (64-row panels) or
    four (128-row panels), output stores written through, a panel's tiles
    split over several blocks): every admissible k, 64-row panels (n =
    128, 192, and every n at k = 32) and 128-row panels (n >= 384 at k = 64
    and 128), 1 to 6 tiles per block (every pipeline depth), all outputs
    against the oracle; the receipt names the split and the panel height."""
    b, m = 16, 512
    _say(f"panel NT dt={wl.DTYPE_NAMES[dt]} b={b} m={m} n={n} k={k}")
    case = wl.random_gemm_case(47 + k + n, dt, b, m, n, k, False, True)
    rec = check_gemm(case, what=f"panel k={k} n={n}")
    split, pm = check_panel_variant(rec, b, m, n, k)
    assert pm == (128 if k >= 64 and n >= 384 else 64), pm
    assert split == {128: 2, 192: 3}.get(n, 4), split


@pytest.mark.parametrize("dt,b,m,n,k", [
    (wl.F16, 96, 64, 512, 64), (wl.BF16, 8, 960, 512, 64), (wl.F16, 8, 192, 2048, 128),
    (wl.BF16, 4, 512, 4096, 128), (wl.F16, 16, 128, 1024, 64), (wl.F16, 64, 64, 1024, 32),
    (wl.BF16, 2, 512, 8192, 128), (wl.F16, 16, 128, 128, 64)])
def test_panel_kernel_few_panels(dt, b, m, n, k):
    """Fewer than 128 panels of 64 rows: each panel's B tiles split over up
    to 32 blocks (64-row panels) or 16 blocks of two tiles or more (128-row
    panels) so that the GPU still fills; shapes too small for that stay on
    the tiled kernel. All outputs against the oracle; the receipt names the
    kernel and, on the panel kernel, the split and the panel height."""
    _say(f"panel NT few panels dt={wl.DTYPE_NAMES[dt]} b={b} m={m} n={n} k={k}")
    case = wl.random_gemm_case(50 + k + b, dt, b, m, n, k, False, True)
    rec = check_gemm(case, what=f"few panels {b}x{m}x{n}x{k}")
    if panel_taken(b, m, n, k):
        check_panel_variant(rec, b, m, n, k)
    else:
        assert rec.kernel == mm.MM_KERNEL_GEMM_TILED, rec.kernel


@pytest.mark.parametrize("k", [64, 128])
def test_panel_kernel_unsplit_long_rows(k):
    """Enough 128-row panels that no split is needed: each block walks all 8
    B tiles, so its four B stages are reused twice."""
    b, m, n = 64, 512, 512
    _say(f"panel NT unsplit bf16 b=64 m=512 n=512 k={k}")
    case = wl.random_gemm_case(48 + k, wl.BF16, b, m, n, k, False, True)
    rec = check_gemm(case, what="panel unsplit")
    assert check_panel_variant(rec, b, m, n, k) == (1, 128)


def test_panel_kernel_unsplit_64_row_panels():
    """k = 32 keeps 64-row panels; enough of them that no split is needed."""
    b, m, n, k = 64, 512, 512, 32
    _say("panel NT unsplit f16 b=64 m=512 n=512 k=32")
    case = wl.random_gemm_case(49, wl.F16, b, m, n, k, False, True)
    rec = check_gemm(case, what="panel unsplit k=32")
    assert check_panel_variant(rec, b, m, n, k) == (1, 64)


@pytest.mark.parametrize("dt", [wl.F16, wl.BF16])
def test_panel_kernel_padded_offsets_ramp_exact(dt):
    """The panel kernel with padded leading dimensions, batch strides with gaps
    and 16-byte element offsets on every operand; ramp inputs, bit for bit."""
    b, m, n, k = 4, 2048, 384, 128
    _say(f"panel NT padded ramp dt={wl.DTYPE_NAMES[dt]}")
    a = wl.ramp(b * m * k, 1).reshape(b, m, k)
    bb = wl.ramp(b * n * k, 2).reshape(b, n, k)
    case = wl.make_gemm_case(dt, a, bb, False, True, lda=k + 8, ldb=k + 24, ldc=n + 8,
                             off_a=8, off_b=16, off_c=8, stride_a=m * (k + 8) + 64,
                             stride_b=n * (k + 24) + 8, stride_c=m * (n + 8) + 16)
    rec = check_gemm(case, exact=True, what="panel padded ramp")
    assert check_panel_variant(rec, b, m, n, k) == (4, 128)


@pytest.mark.parametrize("k", [128, 192, 320])
def test_large_shape_other_k(k):
    """k below 256 or not a multiple of 128, so not the 256 x 256 kernel: at
    k = 128 the panel kernel (32 panels of 128 rows, each split over 8
    blocks), at 192 and 320 the 128 x 128 kernel; same results."""
    _say(f"NT f16 m=4096 n=8192 k={k}")
    case = wl.random_gemm_case(43, wl.F16, 1, 4096, 8192, k, False, True)
    want = mm.MM_KERNEL_GEMM_PANEL if panel_taken(1, 4096, 8192, k) else mm.MM_KERNEL_GEMM_TILED
    assert (want == mm.MM_KERNEL_GEMM_PANEL) == (k == 128)
    _sampled_check(case, 2048, 6, kernel=want)


@pytest.mark.parametrize("dt", DTYPES)
def test_forced_routes_agree_bit_exact(dt):
    """mm_gemm_route: the skinny, tiled-GEMM and (m GEMVs sharing W) GEMV routes
    of one 8-row product give the rounded oracle's bits on ramp inputs."""
    import torch
    from gpu_util import GemmRun
    import oracle
    m, n, k = 8, 300, 256
    _say(f"forced routes dt={wl.DTYPE_NAMES[dt]} m={m} n={n} k={k}")
    a = wl.ramp(m * k, 1).reshape(1, m, k)
    bb = wl.ramp(n * k, 2).reshape(1, n, k)
    case = wl.make_gemm_case(dt, a, bb, False, True)
    ref_bits = oracle.round_to(dt, GemmRun(case).oracle_full()).reshape(m, n)
    for route in (mm.MM_ROUTE_GEMV_WIDE, mm.MM_ROUTE_GEMM, mm.MM_ROUTE_GEMV):
        run = GemmRun(case, c_extra=0)
        desc = run.desc
        if route == mm.MM_ROUTE_GEMV:  # m GEMVs in one launch, W shared
            desc = mm.gemm_desc(dt, 1, n, k, batch=m, trans_b=True, stride_a=k, stride_b=0,
                                stride_c=n)
        rec = mm.mm_gemm_route(desc, route, *run.bufs, stream=torch.cuda.current_stream())
        assert rec.route == route
        got = run.c_bits()[: m * n].reshape(m, n)
        np.testing.assert_array_equal(got, ref_bits, err_msg=f"route {route}")
