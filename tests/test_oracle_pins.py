"""Pins for the CPU oracle, checked against things other than the oracle itself.

Every pin here is independent of the oracle's code: values printed on the
pages, closed forms, exact rational arithmetic over the stored bits, and
library conversions (numpy) for the rounding and decoding helpers. Together
they fail on a dropped term, a wrong sign, a swapped index, a transposed
operand, a wrong batch stride or offset, a wrong expert stride or activation
row, and a wrong rounding direction.
"""
from __future__ import annotations

import itertools
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DTYPES = [wl.F32, wl.F16, wl.BF16]
LAYOUTS = list(itertools.product([False, True], [False, True]))


def _read_golden(name):
    header, values = None, []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if header is None:
                header = dict(kv.split("=") for kv in line.split())
            else:
                values += [float(v) for v in line.split()]
    return {k: int(v) for k, v in header.items()}, np.array(values)


def _gemm(case: wl.GemmCase, nthreads=0):
    return oracle.gemm(case.dtype, case.batch, case.m, case.n, case.k, case.trans_a,
                       case.trans_b, case.lda, case.ldb, case.stride_a, case.stride_b,
                       case.off_a, case.off_b, case.A, case.B, nthreads)


# ----------------------------------------------------------------------------
# Worked examples printed on the tract-metal page.
# ----------------------------------------------------------------------------

def test_worked_example_ramp_batched():
    h, expected = _read_golden("tract_mlx_gemm_ramp_example.txt")
    b, m, n, k = h["batch"], h["m"], h["n"], h["k"]
    a = np.arange(b * m * k, dtype=np.float64).reshape(b, m, k)
    bb = np.arange(b * k * n, dtype=np.float64).reshape(b, k, n)
    for dt in DTYPES:   # every value and every partial sum is an exact small integer
        c = _gemm(wl.make_gemm_case(dt, a, bb, False, False))
        np.testing.assert_array_equal(c.reshape(-1), expected)


def test_all_ones():
    h, expected = _read_golden("tract_mlx_gemm_all_ones.txt")
    b, m, n, k = h["batch"], h["m"], h["n"], h["k"]
    for dt in DTYPES:
        c = _gemm(wl.make_gemm_case(dt, np.ones((b, m, k)), np.ones((b, k, n)), False, False))
        assert c.shape == (b, m, n)
        assert np.all(c == expected[0])
    # C = K in general, and it is exact after rounding to f16 for K <= 2048.
    c = _gemm(wl.make_gemm_case(wl.F16, np.ones((1, 3, 2048)), np.ones((1, 5, 2048)),
                                False, True))
    assert np.all(c == 2048.0)
    assert np.all(oracle.decode(wl.F16, oracle.round_to(wl.F16, c)) == 2048.0)


# ----------------------------------------------------------------------------
# Identity / permutation: a single nonzero term per output, in every layout.
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_permutation_every_layout(dt, ta, tb):
    rng = np.random.default_rng(11)
    batch, m, k = 3, 5, 6
    n = k
    a_log = np.round(rng.uniform(-4, 4, (batch, m, k)) * 8) / 8     # exact in every dtype
    perms = [rng.permutation(k) for _ in range(batch)]
    p_log = np.zeros((batch, k, n))
    for b in range(batch):
        p_log[b, perms[b], np.arange(n)] = 1.0                    # P[p, j] = 1 iff p = perm[j]
    a_st = a_log.transpose(0, 2, 1) if ta else a_log
    b_st = p_log.transpose(0, 2, 1) if tb else p_log
    case = wl.make_gemm_case(dt, a_st, b_st, ta, tb, lda=a_st.shape[2] + 3,
                             ldb=b_st.shape[2] + 2, off_a=5, off_b=7)
    c = _gemm(case)
    for b in range(batch):
        np.testing.assert_array_equal(c[b], a_log[b][:, perms[b]])
    # Identity on the left returns B (in its logical orientation).
    eye = np.broadcast_to(np.eye(m)[None], (batch, m, m))
    b_log = np.round(rng.uniform(-4, 4, (batch, m, 4)) * 8) / 8
    case = wl.make_gemm_case(dt, eye.transpose(0, 2, 1) if ta else eye,
                             b_log.transpose(0, 2, 1) if tb else b_log, ta, tb)
    np.testing.assert_array_equal(_gemm(case), b_log)


def test_broadcast_stride_zero():
    rng = np.random.default_rng(12)
    a = np.round(rng.uniform(-2, 2, (1, 4, 3)) * 4) / 4
    b = np.round(rng.uniform(-2, 2, (5, 3, 6)) * 4) / 4
    case = wl.make_gemm_case(wl.F32, np.broadcast_to(a, (5, 4, 3)), b, False, False,
                             broadcast_a=True)
    assert case.stride_a == 0
    c = _gemm(case)
    for i in range(5):
        np.testing.assert_array_equal(c[i], a[0] @ b[i])   # small dyadic values: exact


# ----------------------------------------------------------------------------
# Rank-1 closed forms, including ragged K.
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("k", [1, 7, 33, 130])
def test_rank1_closed_form(dt, k):
    rng = np.random.default_rng(k)
    m, n = 6, 9
    u = rng.integers(-8, 9, m) / 4.0
    v = rng.integers(-8, 9, n) / 8.0
    a = np.repeat(u[:, None], k, axis=1)[None]         # A[i, p] = u_i
    b = np.repeat(v[None, :], k, axis=0)[None]         # B[p, j] = v_j
    c = _gemm(wl.make_gemm_case(dt, a, b, False, False))
    np.testing.assert_array_equal(c[0], k * np.outer(u, v))


# ----------------------------------------------------------------------------
# Output epilogue alpha * A.B + beta * C_old (tract-metal `dispatch_metal_mlx_gemm`
# do_axpby / use_out_source): identity and rank-1 products give closed forms.
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("alpha,beta", [(2.0, -0.5), (-1.25, 3.0), (0.0, 1.0), (1.0, 0.0)])
def test_axpby_closed_forms(alpha, beta):
    """I.B scaled by alpha plus C_old scaled by beta, elementwise, and a rank-1
    product k u v^T: catches a swapped alpha/beta, a dropped term or a sign."""
    rng = np.random.default_rng(13)
    m, n = 5, 7
    b_log = np.round(rng.uniform(-4, 4, (1, m, n)) * 8) / 8
    c_old = np.round(rng.uniform(-4, 4, (1, m, n)) * 8) / 8
    prod = _gemm(wl.make_gemm_case(wl.F32, np.eye(m)[None], b_log, False, False))
    np.testing.assert_array_equal(oracle.gemm_axpby(alpha, beta, prod, c_old),
                                  alpha * b_log + beta * c_old)
    u = rng.integers(-8, 9, m) / 4.0
    v = rng.integers(-8, 9, n) / 8.0
    k = 9
    prod = _gemm(wl.make_gemm_case(wl.F32, np.repeat(u[:, None], k, 1)[None],
                                   np.repeat(v[None, :], k, 0)[None], False, False))
    np.testing.assert_array_equal(oracle.gemm_axpby(alpha, beta, prod, c_old),
                                  alpha * k * np.outer(u, v)[None] + beta * c_old)


def test_axpby_beta_zero_ignores_old_values():
    prod = np.arange(6.0).reshape(1, 2, 3)
    got = oracle.gemm_axpby(1.5, 0.0, prod, np.full((1, 2, 3), np.nan))
    np.testing.assert_array_equal(got, 1.5 * prod)


@pytest.mark.parametrize("dt,k", [(wl.F32, 1000), (wl.F16, 300), (wl.BF16, 200)])
def test_arithmetic_series(dt, k):
    """A = 1, B[p, j] = p (B stored [n, k]): every output is k(k-1)/2."""
    a = np.ones((1, 2, k))
    b = np.tile(np.arange(k, dtype=np.float64), (3, 1))[None]
    c = _gemm(wl.make_gemm_case(dt, a, b, False, True))
    assert np.all(c == k * (k - 1) / 2)


# ----------------------------------------------------------------------------
# Exact rational brute force over the stored bits.
# ----------------------------------------------------------------------------

def _exact_values(bits, dt):
    """Decode stored bits with numpy (independent of the oracle's decoders)."""
    return wl.storage_to_float(bits, dt)


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", [(2, 4, 4, 4), (1, 3, 5, 7)])
def test_fraction_bruteforce(dt, ta, tb, shape):
    batch, m, n, k = shape
    # Padded leading dimensions and element offsets exercise every index term.
    case = wl.random_gemm_case(100 + m, dt, batch, m, n, k, ta, tb,
                               lda=(m if ta else k) + 2, ldb=(k if tb else n) + 1,
                               off_a=3, off_b=1)
    c = _gemm(case)
    A = _exact_values(case.A, dt)
    B = _exact_values(case.B, dt)
    e = wl.ELT[dt]
    a0, b0 = case.off_a // e, case.off_b // e
    for b in range(batch):
        for i in range(m):
            for j in range(n):
                terms = []
                for p in range(k):
                    ai = a0 + b * case.stride_a + (p * case.lda + i if ta else i * case.lda + p)
                    bi = b0 + b * case.stride_b + (j * case.ldb + p if tb else p * case.ldb + j)
                    terms.append(Fraction(A[ai]) * Fraction(B[bi]))
                exact = sum(terms, Fraction(0))
                bound = k * 2.0 ** -52 * float(sum(abs(t) for t in terms))
                assert abs(Fraction(c[b, i, j]) - exact) <= Fraction(bound), (b, i, j)


def test_sampled_entries_match_full():
    case = wl.random_gemm_case(5, wl.F16, 3, 17, 19, 37, True, False, lda=20, ldb=25)
    full = _gemm(case)
    rng = np.random.default_rng(0)
    bs = rng.integers(0, 3, 50)
    is_ = rng.integers(0, 17, 50)
    js = rng.integers(0, 19, 50)
    got = oracle.gemm_at(case.dtype, case.k, case.trans_a, case.trans_b, case.lda, case.ldb,
                         case.stride_a, case.stride_b, case.off_a, case.off_b, case.A, case.B,
                         bs, is_, js)
    np.testing.assert_array_equal(got, full[bs, is_, js])


def test_thread_count_does_not_change_bits():
    case = wl.random_gemm_case(6, wl.F32, 2, 33, 29, 301, False, True)
    np.testing.assert_array_equal(_gemm(case, 1), _gemm(case, 8))


# ----------------------------------------------------------------------------
# Rounding and decoding helpers against library conversions / exhaustive checks.
# ----------------------------------------------------------------------------

def test_decode_every_f16_and_bf16_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref16 = bits.view(np.float16).astype(np.float64)
    got16 = oracle.decode(wl.F16, bits)
    np.testing.assert_array_equal(np.isnan(got16), np.isnan(ref16))
    ok = ~np.isnan(ref16)
    np.testing.assert_array_equal(got16[ok], ref16[ok])
    assert np.array_equal(np.signbit(got16[ok]), np.signbit(ref16[ok]))
    refb = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    gotb = oracle.decode(wl.BF16, bits)
    ok = ~np.isnan(refb)
    np.testing.assert_array_equal(gotb[ok], refb[ok])
    assert np.all(np.isnan(gotb[~ok]))


def _round_candidates():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
        rng.standard_normal(2000) * 1e-7,            # f16 subnormal range
        rng.standard_normal(2000) * 1e-39,           # bf16/f32 subnormal range
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, 65536.0, -65520.0, 1e300, -1e300,
         3.3895313892515355e38, 3.402823466e38, 3.4e38, 2.0 ** -24, 2.0 ** -25,
         3 * 2.0 ** -26, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135],
    ])
    # Exact midpoints between neighbouring f16 and bf16 values (ties).
    h = np.arange(0, 0x7C00, 7, dtype=np.uint16)
    hv = h.view(np.float16).astype(np.float64)
    hv2 = (h + 1).view(np.float16).astype(np.float64)
    b = np.arange(0, 0x7F80, 5, dtype=np.uint32)
    bv = (b << 16).view(np.float32).astype(np.float64)
    bv2 = ((b + 1) << 16).view(np.float32).astype(np.float64)
    x = np.concatenate([x, (hv + hv2) / 2, -(hv + hv2) / 2, (bv + bv2) / 2])
    return x[np.isfinite(x)]


def test_round_f16_matches_numpy():
    x = _round_candidates()
    got = oracle.round_to(wl.F16, x)
    ref = x.astype(np.float16).view(np.uint16)    # numpy: correctly rounded double->half
    np.testing.assert_array_equal(got, ref)


def test_round_f32_matches_numpy():
    x = _round_candidates()
    np.testing.assert_array_equal(oracle.round_to(wl.F32, x).view(np.uint32),
                                  x.astype(np.float32).view(np.uint32))


def _nearest_bf16_bits(x: float) -> int:
    """Brute force: nearest finite bfloat16 by exact rational distance, ties to
    an even last bit, overflow past the largest finite value's half-ulp to inf."""
    if x == 0:
        return 0x8000 if np.signbit(x) else 0
    sign = 0x8000 if x < 0 else 0
    ax = Fraction(abs(x))
    pos = np.arange(0, 0x7F80, dtype=np.uint32)
    vals = (pos << 16).view(np.float32).astype(np.float64)
    i = int(np.searchsorted(vals, float(ax)))
    cands = [j for j in (i - 1, i, i + 1) if 0 <= j < len(vals)]
    max_finite = Fraction(float(vals[-1]))
    half_ulp = Fraction(2) ** (127 - 8)
    if ax >= max_finite + half_ulp:
        return sign | 0x7F80
    best = min(cands, key=lambda j: (abs(Fraction(float(vals[j])) - ax), j & 1))
    return sign | int(pos[best])


def test_round_bf16_bruteforce():
    x = _round_candidates()
    rng = np.random.default_rng(9)
    pick = np.concatenate([rng.choice(len(x), 600, replace=False),
                           np.arange(len(x) - 40, len(x))])
    got = oracle.round_to(wl.BF16, x[pick])
    ref = np.array([_nearest_bf16_bits(float(v)) for v in x[pick]], dtype=np.uint16)
    np.testing.assert_array_equal(got, ref)
    big = np.array([3.4e38, 3.3961e38, 1e39, -1e39])
    np.testing.assert_array_equal(oracle.round_to(wl.BF16, big),
                                  [_nearest_bf16_bits(float(v)) for v in big])


# ----------------------------------------------------------------------------
# Expert-ID matmul.
# ----------------------------------------------------------------------------

def _id(case: wl.IdCase, nthreads=0):
    return oracle.matmul_id(case.wdtype, case.m, case.n, case.k, case.top_k, case.n_experts,
                            case.expert_stride_bytes, case.layout, case.W, case.X, case.ids,
                            nthreads)


@pytest.mark.parametrize("wdt", DTYPES)
@pytest.mark.parametrize("layout", [0, 1])
def test_id_fraction_bruteforce_page_shape(wdt, layout):
    """m=9, n=7, k=35, top_k=2, E=4: the shape of the mlx-native page's test."""
    case = wl.random_id_case(21, wdt, 9, 7, 35, 2, 4, layout=layout, stride_pad_elems=3)
    case.ids[3, 1] = 7                     # out of range -> zero row
    case.ids[5, 0] = 0xFFFFFFFF            # -1 passed as u32 -> zero row
    out = _id(case)
    W = wl.storage_to_float(case.W, wdt)
    X = case.X.astype(np.float64)
    es = case.expert_stride_bytes // wl.ELT[wdt]
    for t in range(case.m):
        for s in range(case.top_k):
            r = t * case.top_k + s
            e = int(case.ids[t, s])
            if e >= case.n_experts:
                assert np.all(out[r] == 0) and not np.any(np.signbit(out[r]))
                continue
            xrow = X[t] if layout == 0 else X[r]
            for j in range(case.n):
                terms = [Fraction(W[e * es + j * case.k + p]) * Fraction(xrow[p])
                         for p in range(case.k)]
                exact = sum(terms, Fraction(0))
                bound = case.k * 2.0 ** -52 * float(sum(abs(q) for q in terms))
                assert abs(Fraction(out[r, j]) - exact) <= Fraction(bound)


def test_id_equals_loop_of_gemv():
    """Expert-stack invariant: row (t, s) equals the GEMV x_t . W_e^T computed by
    the GEMM definition, bit for bit (f32 weights, so both sides take f32 inputs;
    mixed-precision weights are pinned by the rational brute force above)."""
    case = wl.random_id_case(22, wl.F32, 5, 11, 40, 3, 6, distinct=False)
    out = _id(case)
    es = case.expert_stride_bytes // 4
    for t in range(case.m):
        for s in range(case.top_k):
            e = int(case.ids[t, s])
            w = case.W[e * es: e * es + case.n * case.k]
            g = oracle.gemm(wl.F32, 1, 1, case.n, case.k, False, True, case.k, case.k, 0, 0,
                            0, 0, case.X[t], w)
            np.testing.assert_array_equal(out[t * case.top_k + s], g[0, 0])


def test_id_single_expert_is_gemm():
    """E = 1: every id is 0 and the result is X . W_0^T."""
    case = wl.random_id_case(23, wl.F32, 6, 10, 24, 1, 1)
    out = _id(case)
    g = oracle.gemm(wl.F32, 1, case.m, case.n, case.k, False, True, case.k, case.k, 0, 0, 0, 0,
                    case.X, case.W)
    np.testing.assert_array_equal(out, g[0])


def test_id_top1_is_batched_gemv():
    """top_k = 1 with ids[t] = t mod E: row t is the GEMV of x_t against W_(t mod E)."""
    rng = np.random.default_rng(24)
    E, m, n, k = 3, 7, 5, 16
    w = rng.standard_normal((E, n, k))
    x = rng.standard_normal((m, k))
    ids = (np.arange(m) % E).astype(np.uint32)[:, None]
    case = wl.make_id_case(wl.F32, w, x, ids)
    out = _id(case)
    for t in range(m):
        g = oracle.gemm(wl.F32, 1, 1, n, k, False, True, k, k, 0, 0, 0, 0, case.X[t],
                        case.W[(t % E) * n * k:(t % E + 1) * n * k])
        np.testing.assert_array_equal(out[t], g[0, 0])


def test_id_rows_match_full():
    case = wl.random_id_case(25, wl.BF16, 6, 9, 33, 4, 5, layout=1, distinct=False)
    full = _id(case)
    rows = np.array([0, 5, 23, 7, 7])
    got = oracle.matmul_id_rows(case.wdtype, case.m, case.n, case.k, case.top_k,
                                case.n_experts, case.expert_stride_bytes, case.layout, case.W,
                                case.X, case.ids, rows)
    np.testing.assert_array_equal(got, full[rows])


def test_id_expert_stride_and_slot_row_matter():
    """Planting a wrong expert stride or the shared row for a slotted layout
    changes the result (the brute-force pin above would catch either)."""
    case = wl.random_id_case(26, wl.F32, 4, 6, 8, 2, 3, layout=1, stride_pad_elems=2)
    good = _id(case)
    wrong_layout = oracle.matmul_id(case.wdtype, case.m, case.n, case.k, case.top_k,
                                    case.n_experts, case.expert_stride_bytes, 0, case.W,
                                    case.X, case.ids)
    assert not np.array_equal(good, wrong_layout)


# ----------------------------------------------------------------------------
# Map pass.
# ----------------------------------------------------------------------------

def _bruteforce_map(ids, m, top_k, E):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    lists = {e: [r for r, v in enumerate(flat) if v == e] for e in range(E)}
    return lists, [v >= E for v in flat]


@pytest.mark.parametrize("m,top_k,E", [(9, 2, 4), (512, 8, 64), (33, 5, 1024), (7, 1, 1)])
def test_map_against_bruteforce(m, top_k, E):
    rng = np.random.default_rng(m + E)
    ids = wl.distinct_ids(rng, m, top_k, E)
    flat = ids.reshape(-1)
    flat[rng.choice(flat.size, max(1, flat.size // 17), replace=False)] = E + 3
    if flat.size > 2:
        flat[1] = 0xFFFFFFFF
    counts, routed, zero_row, broken = oracle.matmul_id_map(m, top_k, E, ids)
    lists, zr = _bruteforce_map(ids, m, top_k, E)
    assert not broken
    assert list(zero_row) == zr
    seen = []
    for e in range(E):
        assert counts[e] == len(lists[e]) <= m
        assert list(routed[e, :counts[e]]) == lists[e]          # ascending r
        assert np.all(routed[e, counts[e]:] == 0xFFFFFFFF)      # untouched
        seen += lists[e]
    valid = [r for r in range(m * top_k) if not zr[r]]
    assert sorted(seen) == valid                                # each valid row once
    assert int(counts.sum()) == len(valid)


def test_map_broken_promise_is_bounded():
    ids = np.zeros((4, 3), dtype=np.uint32)       # expert 0 repeated in every slot
    counts, routed, _, broken = oracle.matmul_id_map(4, 3, 2, ids)
    assert broken and counts[0] == 4 and counts[1] == 0
    assert list(routed[0]) == [0, 1, 2, 3]


def test_moe_workload_ids_are_distinct():
    rng = np.random.default_rng(4)
    ids = wl.distinct_ids(rng, 50, 8, 64)
    assert all(len(set(row)) == 8 for row in ids.tolist())
