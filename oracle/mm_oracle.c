/*
 * mm_oracle.c -- plain CPU oracle for the matrix-product dispatch and the
 * expert-ID matmul.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code,
 * header, table or helper with the GPU library: it has its own element
 * decoders, its own rounding and its own index arithmetic.
 *
 * What it computes is the plain definition of each operation, written out:
 * triple loops, fp64 accumulation in ascending contraction index, inputs read
 * from the exact stored bits the GPU receives. No blocking, fusion or
 * reordering.
 *
 * Sources (the pages this follows):
 *   [tract] tract-metal 0.23.6, src/kernels/matmul/mlx_gemm/mod.rs:
 *           `dispatch_eval`, `dispatch_metal_mlx_gemv`, `dispatch_metal_mlx_gemm`
 *           and the `gemv_wide_tests::check` CPU reference.
 *   [mlxn]  mlx-native 0.13.0, src/ops/dense_matmul_id.rs: module doc,
 *           `DenseMatmulIdInputLayout`, `dense_matmul_id_capability`,
 *           `dense_matmul_id`.
 *   [rlx]   rlx-metal 0.2.14, src/mps_blas.rs: `encode_mps_sgemm_t` (the
 *           op(A)/op(B) storage convention).
 *
 * Dtype codes: 0 = f32, 1 = f16 (IEEE binary16), 2 = bf16.
 * Every function returns 0 on success and a negative value on a bad argument.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

/* ------------------------------------------------------------------------ */
/* Element decoding: stored bits -> exact double.                            */
/* ------------------------------------------------------------------------ */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits. Normal: (1024 + f) * 2^(e - 25); subnormal: f * 2^-24. */
double orc_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x400), e - 25);
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double orc_bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Threads for one parallel loop: `requested` when positive, else the
 * OpenMP default. Passed per loop, so a call never changes the thread count
 * of later calls. */
static int threads_for(int requested)
{
#ifdef _OPENMP
    return requested > 0 ? requested : omp_get_max_threads();
#else
    (void)requested;
    return 1;
#endif
}

static size_t elt_size(int dtype)
{
    return dtype == ORC_F32 ? 4 : 2;
}

/* Element `idx` (in elements) of a buffer holding `dtype` values. */
static double load_elem(const void *base, int dtype, int64_t idx)
{
    if (dtype == ORC_F32) {
        float f;
        memcpy(&f, (const char *)base + idx * 4, 4);
        return (double)f;
    }
    uint16_t h;
    memcpy(&h, (const char *)base + idx * 2, 2);
    return dtype == ORC_F16 ? orc_half_to_double(h) : orc_bf16_to_double(h);
}

/* ------------------------------------------------------------------------ */
/* Rounding: exact double -> nearest stored value, ties to even.             */
/* ------------------------------------------------------------------------ */

/* Round x to a binary format with a p-bit significand whose smallest normal
 * binade starts at 2^emin (below it the spacing stays 2^(emin-p+1): gradual
 * underflow). The exponent is first taken as unbounded; a rounded magnitude
 * above the largest finite value becomes infinity (IEEE 754 overflow rule). */
static double round_to_format(double x, int p, int emin, double max_finite)
{
    if (x != x || isinf(x) || x == 0.0)
        return x;
    int e;
    frexp(x, &e);              /* |x| in [2^(e-1), 2^e) */
    int lead = e - 1;
    if (lead < emin)
        lead = emin;
    int q = lead - (p - 1);    /* exponent of one unit in the last place */
    double r = nearbyint(ldexp(x, -q)); /* default mode: nearest, ties even */
    double y = ldexp(r, q);
    if (fabs(y) > max_finite)
        return copysign(INFINITY, x);
    return y;
}

/* binary16: p = 11, emin = -14, largest finite 65504. Result as bits. */
uint16_t orc_round_half(double x)
{
    double y = round_to_format(x, 11, -14, 65504.0);
    uint16_t s = signbit(y) ? 0x8000 : 0;
    double a = fabs(y);
    if (a != a)
        return 0x7e00;
    if (isinf(a))
        return s | 0x7c00;
    if (a == 0.0)
        return s;
    int e;
    frexp(a, &e);
    int lead = e - 1;
    if (lead < -14)            /* subnormal: a = f * 2^-24 */
        return s | (uint16_t)ldexp(a, 24);
    uint16_t f = (uint16_t)(ldexp(a, 10 - lead) - 1024.0);
    return s | (uint16_t)((lead + 15) << 10) | f;
}

/* bfloat16: p = 8, emin = -126, largest finite (2 - 2^-7) * 2^127. */
uint16_t orc_round_bf16(double x)
{
    double y = round_to_format(x, 8, -126, ldexp(255.0, 120));
    uint16_t s = signbit(y) ? 0x8000 : 0;
    double a = fabs(y);
    if (a != a)
        return 0x7fc0;
    if (isinf(a))
        return s | 0x7f80;
    if (a == 0.0)
        return s;
    int e;
    frexp(a, &e);
    int lead = e - 1;
    if (lead < -126)           /* subnormal: a = f * 2^-133 */
        return s | (uint16_t)ldexp(a, 133);
    uint16_t f = (uint16_t)(ldexp(a, 7 - lead) - 128.0);
    return s | (uint16_t)((lead + 127) << 7) | f;
}

/* Round n doubles to `dtype`, writing the stored bits (4 or 2 bytes each).
 * f32 uses the C conversion, which is round-to-nearest-even on IEEE hosts. */
int orc_round(int dtype, const double *in, void *out, int64_t n)
{
    if (n < 0 || dtype < 0 || dtype > 2)
        return -1;
    for (int64_t i = 0; i < n; ++i) {
        if (dtype == ORC_F32) {
            float f = (float)in[i];
            memcpy((char *)out + i * 4, &f, 4);
        } else {
            uint16_t h = dtype == ORC_F16 ? orc_round_half(in[i]) : orc_round_bf16(in[i]);
            memcpy((char *)out + i * 2, &h, 2);
        }
    }
    return 0;
}

/* Decode n stored values to double (used by tests to read GPU results). */
int orc_decode(int dtype, const void *in, double *out, int64_t n)
{
    if (n < 0 || dtype < 0 || dtype > 2)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        out[i] = load_elem(in, dtype, i);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O1: C[b] = op(A[b]) . op(B[b]) with f64 accumulation.                     */
/* ------------------------------------------------------------------------ */
/*
 * Storage convention ([tract] `dispatch_metal_mlx_gemm` stride checks,
 * [rlx] `encode_mps_sgemm_t` doc): the logical product is [m,k].[k,n] = [m,n].
 *   trans_a = 0: A stored [m,k], element (i,p) at i*lda + p
 *   trans_a = 1: A stored [k,m], element (i,p) at p*lda + i
 *   trans_b = 0: B stored [k,n], element (p,j) at p*ldb + j
 *   trans_b = 1: B stored [n,k], element (p,j) at j*ldb + p
 * Batch b adds b*stride (elements; 0 broadcasts one matrix to every batch).
 * off_a / off_b are byte offsets into the buffers. The GEMV route of
 * [tract] `dispatch_eval` (m == 1 or n == 1) has this same definition.
 * Output: dense C[b][i][j] in f64 (unrounded), ascending-p summation.
 */
static double gemm_entry(int dtype, int64_t k, int ta, int tb, int64_t lda, int64_t ldb,
                         const void *A, int64_t a0, const void *B, int64_t b0,
                         int64_t i, int64_t j)
{
    double acc = 0.0;
    for (int64_t p = 0; p < k; ++p) {
        double a = load_elem(A, dtype, a0 + (ta ? p * lda + i : i * lda + p));
        double b = load_elem(B, dtype, b0 + (tb ? j * ldb + p : p * ldb + j));
        acc += a * b;
    }
    return acc;
}

int orc_gemm(int dtype, int64_t batch, int64_t m, int64_t n, int64_t k, int ta, int tb,
             int64_t lda, int64_t ldb, int64_t stride_a, int64_t stride_b, uint64_t off_a,
             uint64_t off_b, const void *A, const void *B, double *C, int nthreads)
{
    if (dtype < 0 || dtype > 2 || batch < 1 || m < 1 || n < 1 || k < 1)
        return -1;
    size_t es = elt_size(dtype);
    if (off_a % es || off_b % es)
        return -2;
    int64_t a_base = (int64_t)(off_a / es), b_base = (int64_t)(off_b / es);
    int nt = threads_for(nthreads);
    /* One work item per output element, so a single-row product (the GEMV
     * route) spreads over every thread too; each element is still one
     * ascending-p sum, so the bits do not depend on the thread count. */
#pragma omp parallel for collapse(3) schedule(static) num_threads(nt)
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t i = 0; i < m; ++i)
            for (int64_t j = 0; j < n; ++j)
                C[(b * m + i) * n + j] =
                    gemm_entry(dtype, k, ta, tb, lda, ldb, A, a_base + b * stride_a, B,
                               b_base + b * stride_b, i, j);
    return 0;
}

/* Same definition at `ns` sampled output positions (bs[s], is[s], js[s]). */
int orc_gemm_at(int dtype, int64_t k, int ta, int tb, int64_t lda, int64_t ldb,
                int64_t stride_a, int64_t stride_b, uint64_t off_a, uint64_t off_b,
                const void *A, const void *B, int64_t ns, const int64_t *bs, const int64_t *is,
                const int64_t *js, double *out, int nthreads)
{
    if (dtype < 0 || dtype > 2 || k < 1 || ns < 0)
        return -1;
    size_t es = elt_size(dtype);
    if (off_a % es || off_b % es)
        return -2;
    int64_t a_base = (int64_t)(off_a / es), b_base = (int64_t)(off_b / es);
    int nt = threads_for(nthreads);
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t s = 0; s < ns; ++s)
        out[s] = gemm_entry(dtype, k, ta, tb, lda, ldb, A, a_base + bs[s] * stride_a, B,
                            b_base + bs[s] * stride_b, is[s], js[s]);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O2: expert-ID matmul ([mlxn] module doc and `dense_matmul_id`).           */
/* ------------------------------------------------------------------------ */
/*
 * Routed row r = t*top_k + s (token t < m, slot s < top_k), e = ids[r].
 *   e >= n_experts: out[r][:] = +0.0 (no weight is touched)
 *   otherwise:      out[r][j] = sum_p W_e[j][p] * x_{t,s}[p]
 * W_e is row-major [n,k]; its element (j,p) sits at byte
 * e*expert_stride_bytes + (j*k + p)*elt. x_{t,s} is an f32 row of k values at
 * byte t*tok_stride + s*slot_stride with (tok_stride, slot_stride) =
 * (4k, 0) for the shared-per-token layout (layout 0) and (4k*top_k, 4k) for
 * the slotted layout (layout 1), as `dense_matmul_id` derives them.
 */
static double id_entry(int wdtype, uint32_t k, uint32_t top_k, uint32_t n_experts,
                       uint64_t expert_stride_bytes, int layout, const void *W, const float *X,
                       const uint32_t *ids, int64_t r, int64_t j)
{
    uint32_t e = ids[r];
    if (e >= n_experts)
        return 0.0;
    int64_t t = r / top_k, s = r % top_k;
    int64_t x_row = layout == 0 ? t : t * (int64_t)top_k + s; /* in units of k floats */
    const float *x = X + x_row * (int64_t)k;
    const char *We = (const char *)W + (uint64_t)e * expert_stride_bytes;
    double acc = 0.0;
    for (uint32_t p = 0; p < k; ++p) {
        double w = load_elem(We, wdtype, j * (int64_t)k + p);
        acc += w * (double)x[p];
    }
    return acc;
}

int orc_id(int wdtype, uint32_t m, uint32_t n, uint32_t k, uint32_t top_k, uint32_t n_experts,
           uint64_t expert_stride_bytes, int layout, const void *W, const float *X,
           const uint32_t *ids, double *out, int nthreads)
{
    if (wdtype < 0 || wdtype > 2 || !m || !n || !k || !top_k || !n_experts)
        return -1;
    if (layout != 0 && layout != 1)
        return -1;
    if (expert_stride_bytes % elt_size(wdtype))
        return -2;
    int nt = threads_for(nthreads);
    int64_t rows = (int64_t)m * top_k;
    /* One work item per output element (a decode has only top_k rows). */
#pragma omp parallel for collapse(2) schedule(static) num_threads(nt)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < (int64_t)n; ++j)
            out[r * (int64_t)n + j] = id_entry(wdtype, k, top_k, n_experts, expert_stride_bytes,
                                               layout, W, X, ids, r, j);
    return 0;
}

/* Same definition for `nr` selected routed rows; out is [nr][n]. */
int orc_id_rows(int wdtype, uint32_t m, uint32_t n, uint32_t k, uint32_t top_k,
                uint32_t n_experts, uint64_t expert_stride_bytes, int layout, const void *W,
                const float *X, const uint32_t *ids, int64_t nr, const int64_t *rows,
                double *out, int nthreads)
{
    if (wdtype < 0 || wdtype > 2 || !m || !n || !k || !top_k || !n_experts || nr < 0)
        return -1;
    if (layout != 0 && layout != 1)
        return -1;
    if (expert_stride_bytes % elt_size(wdtype))
        return -2;
    for (int64_t q = 0; q < nr; ++q)
        if (rows[q] < 0 || rows[q] >= (int64_t)m * top_k)
            return -3;
    int nt = threads_for(nthreads);
#pragma omp parallel for collapse(2) schedule(static) num_threads(nt)
    for (int64_t q = 0; q < nr; ++q)
        for (int64_t j = 0; j < (int64_t)n; ++j)
            out[q * (int64_t)n + j] = id_entry(wdtype, k, top_k, n_experts, expert_stride_bytes,
                                               layout, W, X, ids, rows[q], j);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O3: the map pass of the grouped route ([mlxn] `dense_matmul_id`, grouped  */
/* branch; scratch extents from `dense_matmul_id_capability`).               */
/* ------------------------------------------------------------------------ */
/*
 * counts[e]            = number of routed rows r < m*top_k with ids[r] == e
 * routed_rows[e*m + i] = the i-th smallest such r, for i < counts[e]
 * zero_row[r]          = 1 when ids[r] >= n_experts (that output row is +0.0)
 * Entries of routed_rows at i >= counts[e] are left as they were. The scan is
 * sequential in r, so each list is ascending. Under the distinct-per-token
 * promise counts[e] <= m; a list that would exceed m is cut at m and the
 * function returns 1 (the promise was broken).
 */
int orc_id_map(uint32_t m, uint32_t top_k, uint32_t n_experts, const uint32_t *ids,
               uint32_t *counts, uint32_t *routed_rows, uint8_t *zero_row)
{
    if (!m || !top_k || !n_experts)
        return -1;
    int broken = 0;
    for (uint32_t e = 0; e < n_experts; ++e)
        counts[e] = 0;
    int64_t rows = (int64_t)m * top_k;
    for (int64_t r = 0; r < rows; ++r) {
        uint32_t e = ids[r];
        zero_row[r] = e >= n_experts;
        if (e >= n_experts)
            continue;
        if (counts[e] >= m) {
            broken = 1;
            continue;
        }
        routed_rows[(int64_t)e * m + counts[e]] = (uint32_t)r;
        counts[e] += 1;
    }
    return broken;
}

/* Threads the OpenMP runtime would use (reported next to timings). */
int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
