"""GPU parity of the output epilogue C = alpha * op(A) op(B) + beta * C_old
(mm_gemm_ex; tract-metal mlx_gemm/mod.rs `dispatch_metal_mlx_gemm` function
constants do_axpby and use_out_source) on every route and kernel family:
GEMV (row and column forms), skinny, tiled, short-K, large and f32 tiles.

Reference: the oracle's product combined by oracle.gemm_axpby with the old
values as stored. Tolerance: |alpha| times the product bound of gpu_util plus
two units of the output format's rounding at the largest reference value
(the beta * C_old term can dominate the result). With beta == 0 the old C
(NaN-filled) must not matter; alpha = 0, beta = 1 must leave C bit for bit;
ramp inputs with power-of-two alpha and beta are compared bit for bit.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import gemv_expert_id_amd as mm
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

EPS = {wl.F32: 2.0 ** -24, wl.F16: 2.0 ** -11, wl.BF16: 2.0 ** -8}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield


from gpu_util import GemmRun, bound, finite_absmax, from_dev, to_dev  # noqa: E402


def _positions(run):
    c = run.case
    base = c.off_c // run.elt
    b, i, j = np.meshgrid(np.arange(c.batch), np.arange(c.m), np.arange(c.n), indexing="ij")
    return base + b * c.stride_c + i * c.ldc + j


def _run(case, alpha, beta, c_old=None, exact=False, what=""):
    """c_old: logical [batch, m, n] values stored into C before the call (None:
    C keeps its NaN fill)."""
    run = GemmRun(case)
    idx = _positions(run)
    old_vals = np.zeros(idx.shape)
    if c_old is not None:
        host = from_dev(run.c, wl.NP_STORE[case.dtype]).copy()
        host[idx] = wl.to_storage(c_old, case.dtype)
        run.c = to_dev(host)
        run.bufs = (run.bufs[0], run.bufs[1], mm.buf(run.c))
        old_vals = oracle.decode(case.dtype, host[idx])
    rec = mm.mm_gemm_ex(run.desc, alpha, beta, *run.bufs, stream=torch.cuda.current_stream())
    bits = run.c_bits()
    got, mask = run.logical_c(bits)
    run.check_untouched(bits, mask)
    ref = oracle.gemm_axpby(alpha, beta, run.oracle_full(), old_vals)
    if exact:
        np.testing.assert_array_equal(got, oracle.decode(case.dtype, oracle.round_to(case.dtype, ref)),
                                      err_msg=what)
    else:
        assert np.all(np.isfinite(got)), f"{what}: non-finite output"
        amax, bmax = run.operand_absmax()
        lim = abs(alpha) * bound(case.dtype, case.k, amax, bmax) + 2 * EPS[case.dtype] * np.abs(ref).max()
        err = float(np.abs(got - ref).max())
        assert err <= lim, f"{what}: max |err| {err:.3e} > {lim:.3e}"
    return rec


ROUTE_CASES = [
    # (batch, m, n, k, ta, tb, route, kernel)
    (1, 1, 300, 264, False, True, mm.MM_ROUTE_GEMV, mm.MM_KERNEL_GEMV_ROWS),
    (2, 1, 300, 77, False, False, mm.MM_ROUTE_GEMV, mm.MM_KERNEL_GEMV_COLS),
    (2, 5, 300, 256, False, True, mm.MM_ROUTE_GEMV_WIDE, mm.MM_KERNEL_GEMV_WIDE),
    (1, 300, 200, 300, False, False, mm.MM_ROUTE_GEMM, None),
    (2, 256, 256, 96, False, True, mm.MM_ROUTE_GEMM, None),
    # batched short-K NT: the panel kernel when beta == 0, else the tiled one
    (64, 128, 256, 64, False, True, mm.MM_ROUTE_GEMM, None),
]


@pytest.mark.parametrize("dt", [wl.F32, wl.F16, wl.BF16])
@pytest.mark.parametrize("shape", ROUTE_CASES)
@pytest.mark.parametrize("alpha,beta", [(0.75, -1.25), (-2.0, 0.0), (1.0, 1.0)])
def test_axpby_every_route(dt, shape, alpha, beta):
    b, m, n, k, ta, tb, route, kernel = shape
    _say(f"axpby {wl.DTYPE_NAMES[dt]} alpha={alpha} beta={beta} shape={shape[:6]}")
    case = wl.random_gemm_case(80 + m, dt, b, m, n, k, ta, tb)
    rng = np.random.default_rng(81)
    c_old = rng.standard_normal((b, m, n)) if beta != 0 else None
    rec = _run(case, alpha, beta, c_old, what=str(shape))
    assert rec.route == route, rec.route
    if kernel is not None:
        assert rec.kernel == kernel, rec.kernel
    if dt == wl.F32 and route == mm.MM_ROUTE_GEMM:
        small = k <= 128 and ((m + 15) // 16) * ((n + 15) // 16) <= 1024
        assert rec.kernel == (mm.MM_KERNEL_GEMM_F32_SMALL if small else mm.MM_KERNEL_GEMM_F32)
    if dt != wl.F32 and (b, m, n, k) == (64, 128, 256, 64):
        assert rec.kernel == (mm.MM_KERNEL_GEMM_PANEL if beta == 0 else mm.MM_KERNEL_GEMM_TILED)


@pytest.mark.parametrize("dt", [wl.F16, wl.BF16])
def test_axpby_large_tile_sampled(dt):
    """The 256 x 256 kernel's epilogue, sampled against the oracle."""
    m, n, k = 4096, 8192, 256
    _say(f"axpby large {wl.DTYPE_NAMES[dt]} {m}x{n}x{k}")
    case = wl.random_gemm_case(82, dt, 1, m, n, k, False, True)
    run = GemmRun(case)
    rng = np.random.default_rng(83)
    c_old = rng.standard_normal((m, n)).astype(np.float32)
    host = from_dev(run.c, wl.NP_STORE[dt]).copy()
    host[: m * n] = wl.to_storage(c_old, dt).reshape(-1)
    run.c = to_dev(host)
    rec = mm.mm_gemm_ex(run.desc, 0.5, -0.75, run.bufs[0], run.bufs[1], mm.buf(run.c),
                        stream=torch.cuda.current_stream())
    assert rec.kernel == mm.MM_KERNEL_GEMM_LARGE
    bits = run.c_bits()
    is_ = rng.integers(0, m, 3000)
    js = rng.integers(0, n, 3000)
    prod = oracle.gemm_at(dt, k, False, True, case.lda, case.ldb, case.stride_a, case.stride_b,
                          case.off_a, case.off_b, case.A, case.B, np.zeros_like(is_), is_, js)
    old = oracle.decode(dt, host[is_ * n + js])
    ref = oracle.gemm_axpby(0.5, -0.75, prod, old)
    got = oracle.decode(dt, bits[is_ * n + js])
    amax, bmax = run.operand_absmax()
    lim = 0.5 * bound(dt, k, amax, bmax) + 2 * EPS[dt] * np.abs(ref).max()
    assert float(np.abs(got - ref).max()) <= lim


@pytest.mark.parametrize("dt", [wl.F32, wl.F16, wl.BF16])
def test_beta_zero_never_reads_c(dt):
    """C is NaN-filled; beta = 0 must give finite alpha * A.B on every route."""
    for (b, m, n, k, ta, tb, _, _) in ROUTE_CASES:
        case = wl.random_gemm_case(84, dt, b, m, n, k, ta, tb)
        _run(case, 1.5, 0.0, None, what=f"beta0 {(b, m, n, k)}")


@pytest.mark.parametrize("dt", [wl.F32, wl.F16, wl.BF16])
def test_alpha_zero_beta_one_keeps_c(dt):
    for (b, m, n, k, ta, tb, _, _) in ROUTE_CASES:
        case = wl.random_gemm_case(85, dt, b, m, n, k, ta, tb)
        c_old = np.random.default_rng(86).standard_normal((b, m, n))
        _run(case, 0.0, 1.0, c_old, exact=True, what=f"keep {(b, m, n, k)}")


@pytest.mark.parametrize("dt", [wl.F32, wl.F16, wl.BF16])
def test_axpby_ramp_bit_exact(dt):
    """Ramp operands and old values, alpha = 2, beta = 0.5: every term is exact,
    so each route matches the rounded reference bit for bit."""
    for (b, m, n, k, ta, tb, _, _) in ROUTE_CASES:
        a_shape = (b, k, m) if ta else (b, m, k)
        b_shape = (b, n, k) if tb else (b, k, n)
        a = wl.ramp(int(np.prod(a_shape)), 1).reshape(a_shape)
        bv = wl.ramp(int(np.prod(b_shape)), 2).reshape(b_shape)
        case = wl.make_gemm_case(dt, a, bv, ta, tb)
        c_old = wl.ramp(b * m * n, 3).reshape(b, m, n)
        _run(case, 2.0, 0.5, c_old, exact=True, what=f"ramp {(b, m, n, k)}")


# The pipelined kernel (128 x 128 tiles here) in every transpose layout with
# m and n off the tile edge: ragged edge tiles take the per-element epilogue;
# the last three cases run its paired-stage forms.
PIPELINED_CASES = [
    # (batch, m, n, k, ta, tb)
    (1, 200, 132, 256, False, True),
    (1, 100, 136, 256, False, False),
    (2, 136, 76, 384, True, True),
    (1, 136, 200, 256, True, False),
    (1, 1000, 516, 512, False, True),   # paired stages, four regions, ragged
    (1, 256, 384, 1024, False, False),  # paired stages, four regions, NN
    (1, 2304, 2052, 256, False, True),  # paired stages, two regions (306 tiles), ragged
]


@pytest.mark.parametrize("dt", [wl.F16, wl.BF16])
@pytest.mark.parametrize("shape", PIPELINED_CASES)
@pytest.mark.parametrize("alpha,beta", [(0.75, -1.25), (1.0, 1.0)])
def test_axpby_pipelined_ragged_layouts(dt, shape, alpha, beta):
    b, m, n, k, ta, tb = shape
    _say(f"axpby pipelined {wl.DTYPE_NAMES[dt]} alpha={alpha} beta={beta} shape={shape}")
    case = wl.random_gemm_case(87 + m % 5, dt, b, m, n, k, ta, tb)
    c_old = np.random.default_rng(88).standard_normal((b, m, n))
    rec = _run(case, alpha, beta, c_old, what=str(shape))
    assert (rec.kernel, rec.variant & ~1) == (mm.MM_KERNEL_GEMM_LARGE, 128), (rec.kernel, rec.variant)


def test_axpby_pipelined_ramp_bit_exact():
    """Ramp operands and old values on the ragged pipelined kernel, alpha = 2,
    beta = 0.5, bit for bit."""
    b, m, n, k, ta, tb = PIPELINED_CASES[0]
    a = wl.ramp(b * m * k, 1).reshape(b, m, k)
    bv = wl.ramp(b * n * k, 2).reshape(b, n, k)
    case = wl.make_gemm_case(wl.BF16, a, bv, ta, tb)
    c_old = wl.ramp(b * m * n, 3).reshape(b, m, n)
    rec = _run(case, 2.0, 0.5, c_old, exact=True, what="pipelined ramp")
    assert rec.kernel == mm.MM_KERNEL_GEMM_LARGE, rec.kernel
