// C ABI of libmm.so: validation, route selection and launch (see mm.h).
//
// Everything here is host code. Each entry point validates the whole call
// first (pure arithmetic on the descriptor and buffer ranges, no HIP call),
// then resolves every kernel family it will launch, and only then enqueues.
// A call that fails has enqueued nothing (mlx-native dense_matmul_id.rs,
// `dense_matmul_id`: pipelines resolved and limits checked before any
// encode). The library keeps no state across calls beyond per-thread error
// text and test counters.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "../../include/mm.h"
#include "kernels.hpp"

static_assert(MM_ID_GROUPED_MAX_EXPERTS == (unsigned)mmk::MM_GROUPED_MAX_E, "expert limit");

namespace {

thread_local std::string g_error;
thread_local std::string g_inject;
thread_local uint64_t g_launches = 0;

bool debug_sync() {
    static const bool on = [] {
        const char* v = std::getenv("MM_DEBUG_SYNC");
        return v && v[0] && std::strcmp(v, "0") != 0;
    }();
    return on;
}

mm_status fail(mm_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return st;
}

mm_status ok() {
    g_error.clear();
    return MM_OK;
}

uint64_t elt_size(int dt) { return dt == MM_F32 ? 4 : 2; }
bool valid_dtype(int dt) { return dt == MM_F32 || dt == MM_F16 || dt == MM_BF16; }

// Overflow-checked arithmetic on byte extents (mlx-native `checked_product`).
bool mul_ok(uint64_t a, uint64_t b, uint64_t* out) {
    if (a != 0 && b > UINT64_MAX / a) return false;
    *out = a * b;
    return true;
}
bool add_ok(uint64_t a, uint64_t b, uint64_t* out) {
    if (b > UINT64_MAX - a) return false;
    *out = a + b;
    return true;
}

struct Range {
    uint64_t lo, hi;  // [lo, hi)
};
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo < a.hi && b.lo < b.hi; }

// A buffer must start at an address aligned to `align`, be non-null and hold
// `need` bytes starting `offset` bytes in.
mm_status check_buf(const char* label, mm_buf buf, uint64_t offset, uint64_t need, uint64_t align,
                    Range* range) {
    if (buf.ptr == nullptr) return fail(MM_ERR_INVALID_ARGUMENT, "%s: null pointer", label);
    const uint64_t base = (uint64_t)(uintptr_t)buf.ptr;
    uint64_t start, end, used;
    if (!add_ok(base, offset, &start) || !add_ok(offset, need, &used) || !add_ok(start, need, &end))
        return fail(MM_ERR_INVALID_ARGUMENT, "%s: address range overflows", label);
    if (start % align != 0)
        return fail(MM_ERR_MISALIGNED, "%s: address %#llx (offset %llu) is not aligned to %llu bytes",
                    label, (unsigned long long)base, (unsigned long long)offset,
                    (unsigned long long)align);
    if (used > buf.bytes)
        return fail(MM_ERR_BUFFER_TOO_SMALL, "%s: needs %llu bytes from its pointer, buffer holds %llu",
                    label, (unsigned long long)used, (unsigned long long)buf.bytes);
    *range = Range{start, end};
    return MM_OK;
}

mm_status resolve(const char* family) {
    if (!g_inject.empty() && g_inject == family) {
        g_inject.clear();
        return fail(MM_ERR_UNSUPPORTED, "kernel family %s could not be resolved (injected failure)",
                    family);
    }
    return MM_OK;
}

mm_status finish(hipError_t err, hipStream_t s, const char* what) {
    if (err != hipSuccess)
        return fail(MM_ERR_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(err));
    if (debug_sync()) {
        err = hipStreamSynchronize(s);
        if (err == hipSuccess) err = hipGetLastError();
        if (err != hipSuccess)
            return fail(MM_ERR_DEVICE, "%s: kernel failed: %s", what, hipGetErrorString(err));
    }
    return MM_OK;
}

void set_receipt(mm_receipt* r, uint32_t route, uint32_t dtype, uint32_t n, const mmk::Launched& L) {
    if (!r) return;
    r->schema_version = MM_ID_SCHEMA_VERSION;
    r->route = route;
    r->dtype = dtype;
    r->dispatch_count = n;
    r->kernel = (uint32_t)L.kernel;
    r->variant = (uint32_t)L.variant;
}

// ---------------------------------------------------------------------------
// GEMM / GEMV
// ---------------------------------------------------------------------------
struct GemmPlan {
    int dt;
    int64_t batch, m, n, k, lda, ldb, ldc, sa, sb, sc;
    bool ta, tb;
    const char* a;
    const char* b;
    char* c;
    float alpha = 1.f, beta = 0.f;  // C = alpha * op(A) op(B) + beta * C_old
};

// Elements spanned by `nb` matrices of `rows` x `cols` with leading dimension
// ld and batch stride `stride` (0 = one shared matrix).
bool span_elems(int64_t nb, int64_t stride, int64_t rows, int64_t ld, int64_t cols, uint64_t* out) {
    uint64_t a, b, c;
    const uint64_t n_mats = stride == 0 ? 1 : (uint64_t)nb;
    if (!mul_ok(n_mats - 1, (uint64_t)stride, &a)) return false;
    if (!mul_ok((uint64_t)rows - 1, (uint64_t)ld, &b)) return false;
    if (!add_ok(a, b, &c)) return false;
    return add_ok(c, (uint64_t)cols, out);
}

mm_status plan_gemm(const mm_gemm_desc* d, mm_buf a, mm_buf b, mm_buf c, GemmPlan* p) {
    if (!d) return fail(MM_ERR_INVALID_ARGUMENT, "gemm: null descriptor");
    if (!valid_dtype(d->dtype))
        return fail(MM_ERR_UNSUPPORTED, "gemm: dtype %d is not f32, f16 or bf16", (int)d->dtype);
    if (d->batch < 1 || d->m < 1 || d->n < 1 || d->k < 1)
        return fail(MM_ERR_INVALID_ARGUMENT, "gemm: batch, m, n, k must be >= 1 (got %lld, %lld, %lld, %lld)",
                    (long long)d->batch, (long long)d->m, (long long)d->n, (long long)d->k);
    const int64_t lim = (int64_t)1 << 31;
    if (d->m >= lim || d->n >= lim || d->k >= lim)
        return fail(MM_ERR_INVALID_ARGUMENT, "gemm: m, n, k must each be below 2^31");
    if ((d->trans_a != 0 && d->trans_a != 1) || (d->trans_b != 0 && d->trans_b != 1))
        return fail(MM_ERR_INVALID_ARGUMENT, "gemm: trans_a / trans_b must be 0 or 1");
    const bool ta = d->trans_a, tb = d->trans_b;
    const int64_t tight_a = ta ? d->m : d->k, tight_b = tb ? d->k : d->n, tight_c = d->n;
    const int64_t lda = d->lda ? d->lda : tight_a;
    const int64_t ldb = d->ldb ? d->ldb : tight_b;
    const int64_t ldc = d->ldc ? d->ldc : tight_c;
    if (lda < tight_a)
        return fail(MM_ERR_INVALID_ARGUMENT, "gemm: lda %lld is below the stored row length %lld",
                    (long long)lda, (long long)tight_a);
    if (ldb < tight_b)
        return fail(MM_ERR_INVALID_ARGUMENT, "gemm: ldb %lld is below the stored row length %lld",
                    (long long)ldb, (long long)tight_b);
    if (ldc < tight_c)
        return fail(MM_ERR_INVALID_ARGUMENT, "gemm: ldc %lld is below n = %lld", (long long)ldc,
                    (long long)tight_c);
    if (d->stride_a < 0 || d->stride_b < 0 || d->stride_c < 0)
        return fail(MM_ERR_INVALID_ARGUMENT, "gemm: batch strides must be >= 0");
    uint64_t c_one;
    if (!span_elems(1, 0, d->m, ldc, d->n, &c_one))
        return fail(MM_ERR_INVALID_ARGUMENT, "gemm: C extent overflows");
    int64_t sc = d->stride_c;
    if (sc == 0) {
        uint64_t t;
        if (!mul_ok((uint64_t)d->m, (uint64_t)ldc, &t) || t > (uint64_t)INT64_MAX)
            return fail(MM_ERR_INVALID_ARGUMENT, "gemm: C stride overflows");
        sc = (int64_t)t;
    } else if (d->batch > 1 && (uint64_t)sc < c_one) {
        return fail(MM_ERR_INVALID_ARGUMENT,
                    "gemm: stride_c %lld makes output batches overlap (one matrix spans %llu elements)",
                    (long long)sc, (unsigned long long)c_one);
    }
    const uint64_t es = elt_size(d->dtype);
    if (d->offset_a % es || d->offset_b % es || d->offset_c % es)
        return fail(MM_ERR_MISALIGNED, "gemm: byte offsets must be multiples of %llu",
                    (unsigned long long)es);
    uint64_t ea, eb, ec;
    if (!span_elems(d->batch, d->stride_a, ta ? d->k : d->m, lda, ta ? d->m : d->k, &ea) ||
        !span_elems(d->batch, d->stride_b, tb ? d->n : d->k, ldb, tb ? d->k : d->n, &eb) ||
        !span_elems(d->batch, sc, d->m, ldc, d->n, &ec) || !mul_ok(ea, es, &ea) ||
        !mul_ok(eb, es, &eb) || !mul_ok(ec, es, &ec))
        return fail(MM_ERR_INVALID_ARGUMENT, "gemm: operand extent overflows");
    Range ra, rb, rc;
    mm_status st;
    if ((st = check_buf("gemm A", a, d->offset_a, ea, es, &ra)) != MM_OK) return st;
    if ((st = check_buf("gemm B", b, d->offset_b, eb, es, &rb)) != MM_OK) return st;
    if ((st = check_buf("gemm C", c, d->offset_c, ec, es, &rc)) != MM_OK) return st;
    if (overlap(rc, ra)) return fail(MM_ERR_OVERLAP, "gemm: C must not overlap A");
    if (overlap(rc, rb)) return fail(MM_ERR_OVERLAP, "gemm: C must not overlap B");
    *p = GemmPlan{(int)d->dtype, d->batch, d->m, d->n, d->k, lda, ldb, ldc, d->stride_a,
                  d->stride_b, sc, ta, tb,
                  static_cast<const char*>(a.ptr) + d->offset_a,
                  static_cast<const char*>(b.ptr) + d->offset_b,
                  static_cast<char*>(c.ptr) + d->offset_c};
    return MM_OK;
}

// tract-metal `dispatch_metal_mlx_gemv`: the matrix is B when n != 1, else A.
mmk::GemvArgs gemv_args(const GemmPlan& p) {
    mmk::GemvArgs g{};
    g.dtype = p.dt;
    g.alpha = p.alpha;
    g.beta = p.beta;
    g.k = p.k;
    g.batch = p.batch;
    g.out = p.c;
    g.out_bstride = p.sc;
    if (p.n != 1) {
        g.mat = p.b;
        g.vec = p.a;
        g.rows = p.n;
        g.ld = p.ldb;
        g.col_form = p.tb ? 0 : 1;  // B stored [n,k]: rows along k
        g.vec_inc = p.ta ? p.lda : 1;
        g.out_inc = 1;
        g.mat_bstride = p.sb;
        g.vec_bstride = p.sa;
    } else {
        g.mat = p.a;
        g.vec = p.b;
        g.rows = p.m;
        g.ld = p.lda;
        g.col_form = p.ta ? 1 : 0;  // A stored [m,k]: rows along k
        g.vec_inc = p.tb ? 1 : p.ldb;
        g.out_inc = p.ldc;
        g.mat_bstride = p.sa;
        g.vec_bstride = p.sb;
    }
    return g;
}

mm_status run_gemv(const GemmPlan& p, hipStream_t s, mm_receipt* r) {
    mm_status st = resolve("gemv");
    if (st != MM_OK) return st;
    ++g_launches;
    mmk::Launched L;
    st = finish(mmk::launch_gemv(gemv_args(p), s, &L), s, "gemv");
    if (st != MM_OK) return st;
    set_receipt(r, MM_ROUTE_GEMV, (uint32_t)p.dt, 1, L);
    return ok();
}

// tract-metal `gemv_wide_config`: a skinny product (2..64 rows on one side)
// against a matrix with rows along k streams that matrix once for all rows.
// Both operands must be stored with rows along k (trans_a = 0, trans_b = 1)
// and allow 16-byte chunks that never straddle a row end.
bool skinny_args(const GemmPlan& p, mmk::SkinnyArgs* g) {
    if (p.ta || !p.tb) return false;
    const bool x_is_a = p.m >= 2 && p.m <= 64 && p.n >= 2;
    const bool x_is_b = !x_is_a && p.n >= 2 && p.n <= 64 && p.m >= 2;
    if (!x_is_a && !x_is_b) return false;
    const int64_t ch = 16 / (int64_t)elt_size(p.dt);
    const auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
    if (p.k % ch || p.lda % ch || p.ldb % ch || p.sa % ch || p.sb % ch || !al16(p.a) || !al16(p.b))
        return false;
    *g = mmk::SkinnyArgs{};
    g->dtype = p.dt;
    g->alpha = p.alpha;
    g->beta = p.beta;
    g->k = p.k;
    g->batch = p.batch;
    g->out = p.c;
    g->so = p.sc;
    if (x_is_a) {  // C[i][j] = X(i) . W(j): W = B [n,k], X = A [m,k]
        g->W = p.b; g->ldw = p.ldb; g->sw = p.sb; g->nw = p.n;
        g->X = p.a; g->ldx = p.lda; g->sx = p.sa; g->nx = p.m;
        g->out_sx = p.ldc; g->out_sw = 1;
    } else {       // C[i][j] = W(i) . X(j): W = A [m,k], X = B [n,k]
        g->W = p.a; g->ldw = p.lda; g->sw = p.sa; g->nw = p.m;
        g->X = p.b; g->ldx = p.ldb; g->sx = p.sb; g->nx = p.n;
        g->out_sx = 1; g->out_sw = p.ldc;
    }
    // One batch's extents are addressed with 32-bit offsets.
    const uint64_t es = elt_size(p.dt);
    const uint64_t wb = ((uint64_t)(g->nw - 1) * g->ldw + p.k) * es;
    const uint64_t xb = ((uint64_t)(g->nx - 1) * g->ldx + p.k) * es;
    if (wb >= (1ull << 31) || xb >= (1ull << 31)) return false;
    g->w_bytes = (int64_t)wb;
    g->x_bytes = (int64_t)xb;
    return true;
}

// Whether the automatic dispatch takes the skinny route for a shape it fits
// (a forced route skips this). The kernel's blocks each stream 16 rows of W
// through LDS stages of 1 KiB per row, and a CU holds 3, 2, 1 or 1 of them
// for 1, 2, 3 or 4 activation fragments (registers). When all blocks are
// resident at once the route wins at every measured shape; when they come in
// rounds, each block's fixed cost recurs per round, and the tiled GEMM wins
// unless every block streams long rows (one or two fragments) or the rounds
// are few (three or four fragments). Thresholds from the short-k, batch 1 and
// 32 calibration on MI355X's 256 CUs.
bool skinny_pays(const mmk::SkinnyArgs& g, int dt) {
    const int nxf = (int)((g.nx + 15) / 16);
    const int per_cu = nxf == 1 ? 3 : nxf == 2 ? 2 : 1;
    const int64_t blocks = g.batch * ((g.nw + 15) / 16);
    const int64_t rounds = (blocks + 256 * per_cu - 1) / (256 * per_cu);
    if (rounds <= 1) return true;
    const int64_t row_bytes = g.k * (int64_t)elt_size(dt);
    if (nxf <= 2) return row_bytes >= (rounds <= 2 ? 512 : 1024);
    return rounds <= 3;
}

mm_status run_skinny(const mmk::SkinnyArgs& g, int dt, hipStream_t s, mm_receipt* r) {
    mm_status st = resolve("gemv_wide");
    if (st != MM_OK) return st;
    ++g_launches;
    mmk::Launched L;
    st = finish(mmk::launch_gemv_wide(g, s, &L), s, "gemv_wide");
    if (st != MM_OK) return st;
    set_receipt(r, MM_ROUTE_GEMV_WIDE, (uint32_t)dt, 1, L);
    return ok();
}

mm_status run_gemm(const GemmPlan& p, hipStream_t s, mm_receipt* r) {
    mm_status st = resolve("gemm");
    if (st != MM_OK) return st;
    mmk::GemmArgs g{p.a, p.b, p.c, p.m, p.n, p.k, p.lda, p.ldb, p.ldc, p.sa, p.sb, p.sc,
                    p.batch, p.dt, p.ta, p.tb, p.alpha, p.beta};
    ++g_launches;
    mmk::Launched L;
    st = finish(mmk::launch_gemm(g, s, &L), s, "gemm");
    if (st != MM_OK) return st;
    set_receipt(r, MM_ROUTE_GEMM, (uint32_t)p.dt, 1, L);
    return ok();
}

// ---------------------------------------------------------------------------
// Expert-ID matmul
// ---------------------------------------------------------------------------
// check_weights = false skips the weight dtype, stride and extent checks (the
// map pass never reads weights); weight_bytes is then reported as 0.
mm_status id_query(mm_dtype wdt, const mm_id_params* p, mm_id_capability* cap,
                   bool check_weights = true) {
    if (!p) return fail(MM_ERR_INVALID_ARGUMENT, "matmul_id: null params");
    if (!check_weights) wdt = MM_BF16;
    if (!valid_dtype(wdt))
        return fail(MM_ERR_UNSUPPORTED, "matmul_id: weights must be f32, f16 or bf16 (got %d)", (int)wdt);
    if (!p->m || !p->n || !p->k || !p->top_k || !p->n_experts)
        return fail(MM_ERR_INVALID_ARGUMENT, "matmul_id: m, n, k, top_k and n_experts must be nonzero");
    if (p->input_layout > 1 || p->multiplicity > 1 || p->route > 1)
        return fail(MM_ERR_INVALID_ARGUMENT, "matmul_id: input_layout, multiplicity and route must be 0 or 1");
    if (p->multiplicity == 0 && p->top_k > p->n_experts)
        return fail(MM_ERR_INVALID_ARGUMENT, "matmul_id: distinct top_k %u exceeds n_experts %u",
                    p->top_k, p->n_experts);
    const uint64_t es = elt_size(wdt);
    uint64_t matrix = 0, last = 0, wbytes = 0, total, in_rows, in_bytes, ids_bytes, out_bytes;
    if (check_weights) {
    if (!mul_ok((uint64_t)p->n * p->k, es, &matrix))
        return fail(MM_ERR_INVALID_ARGUMENT, "matmul_id: expert matrix byte extent overflows");
    if (p->expert_stride_bytes < matrix)
        return fail(MM_ERR_INVALID_ARGUMENT,
                    "matmul_id: expert stride %llu is smaller than one %llu-byte matrix",
                    (unsigned long long)p->expert_stride_bytes, (unsigned long long)matrix);
    if (p->expert_stride_bytes % es)
        return fail(MM_ERR_INVALID_ARGUMENT, "matmul_id: expert stride %llu is not a multiple of %llu",
                    (unsigned long long)p->expert_stride_bytes, (unsigned long long)es);
    if (!mul_ok((uint64_t)p->n_experts - 1, p->expert_stride_bytes, &last) ||
        !add_ok(last, matrix, &wbytes))
        return fail(MM_ERR_INVALID_ARGUMENT, "matmul_id: weight extent overflows");
    }
    total = (uint64_t)p->m * p->top_k;
    if (total > 0xffffffffull)
        return fail(MM_ERR_INVALID_ARGUMENT, "matmul_id: m*top_k = %llu exceeds the u32 row index",
                    (unsigned long long)total);
    in_rows = p->input_layout == 0 ? p->m : total;
    if (!mul_ok(in_rows * p->k, 4, &in_bytes) || !mul_ok(total, 4, &ids_bytes) ||
        !mul_ok(total * p->n, 4, &out_bytes) || (total && out_bytes / 4 / total != p->n))
        return fail(MM_ERR_INVALID_ARGUMENT, "matmul_id: input/ids/output extent overflows");
    if (p->route == 1 && p->multiplicity != 0)
        return fail(MM_ERR_INVALID_ARGUMENT,
                    "matmul_id: grouped prefill requires distinct expert ids per token");
    if (p->route == 1 && p->n_experts > MM_ID_GROUPED_MAX_EXPERTS)
        return fail(MM_ERR_INVALID_ARGUMENT, "matmul_id: grouped prefill supports at most %u experts",
                    MM_ID_GROUPED_MAX_EXPERTS);
    uint64_t counts = 0, routed = 0;
    if (p->route == 1) {
        counts = (uint64_t)p->n_experts * 4;
        if (!mul_ok((uint64_t)p->n_experts * p->m, 4, &routed))
            return fail(MM_ERR_INVALID_ARGUMENT, "matmul_id: routed-row scratch extent overflows");
    }
    if (cap) {
        std::memset(cap, 0, sizeof *cap);
        cap->schema_version = MM_ID_SCHEMA_VERSION;
        cap->weight_dtype = check_weights ? (uint32_t)wdt : (uint32_t)MM_F32;
        cap->route = p->route;
        cap->weight_bytes = wbytes;
        cap->input_bytes = in_bytes;
        cap->ids_bytes = ids_bytes;
        cap->output_bytes = out_bytes;
        cap->counts_bytes = counts;
        cap->routed_rows_bytes = routed;
    }
    return MM_OK;
}

mmk::IdArgs id_args(const mm_id_params* p, mm_dtype wdt) {
    mmk::IdArgs a{};
    a.m = p->m;
    a.n = p->n;
    a.k = p->k;
    a.top_k = p->top_k;
    a.n_experts = p->n_experts;
    a.layout = p->input_layout;
    a.expert_stride_bytes = p->expert_stride_bytes;
    const uint64_t row = (uint64_t)p->k * 4;
    // `dense_matmul_id`: shared -> (4k, 0); slotted -> (4k*top_k, 4k).
    a.x_tok_stride_bytes = p->input_layout == 0 ? row : row * p->top_k;
    a.x_slot_stride_bytes = p->input_layout == 0 ? 0 : row;
    a.wdtype = (int)wdt;
    a.dedup = p->input_layout == 0 ? 1 : 0;
    return a;
}

enum IdUse { USE_DIRECT, USE_MAP, USE_GROUPED, USE_PREFILL, USE_PREFILL_NOALLOC };

// Validates buffers for one use of the params (mlx-native
// `validate_dense_matmul_id_call`).
mm_status id_validate(IdUse use, const mm_id_params* p, mm_dtype wdt, mm_buf weights,
                      mm_buf input, mm_buf ids, mm_buf out, mm_buf counts, mm_buf routed,
                      mm_id_capability* cap) {
    mm_status st = id_query(wdt, p, cap, use != USE_MAP);
    if (st != MM_OK) return st;
    const uint32_t want_route = use == USE_DIRECT ? 0u : 1u;
    if (p->route != want_route)
        return fail(MM_ERR_INVALID_ARGUMENT, "matmul_id: params.route = %u does not match this entry point (%s)",
                    p->route, want_route ? "grouped prefill" : "direct");
    const bool need_w = use != USE_MAP, need_in = use != USE_MAP;
    // The allocation-free prefill keeps its scratch in the library's own array.
    const bool need_ids = use != USE_GROUPED;
    const bool need_scr = use != USE_DIRECT && use != USE_PREFILL_NOALLOC;
    Range rw{0, 0}, ri{0, 0}, rids{0, 0}, ro{0, 0}, rc{0, 0}, rr{0, 0};
    if (need_w && (st = check_buf("matmul_id weights", weights, 0, cap->weight_bytes,
                                  elt_size(wdt), &rw)) != MM_OK)
        return st;
    if (need_in && (st = check_buf("matmul_id input", input, 0, cap->input_bytes, 4, &ri)) != MM_OK)
        return st;
    if (need_ids && (st = check_buf("matmul_id ids", ids, 0, cap->ids_bytes, 4, &rids)) != MM_OK)
        return st;
    if ((st = check_buf("matmul_id output", out, 0, cap->output_bytes, 4, &ro)) != MM_OK) return st;
    if (need_w && overlap(ro, rw)) return fail(MM_ERR_OVERLAP, "matmul_id: output must not overlap weights");
    if (need_in && overlap(ro, ri)) return fail(MM_ERR_OVERLAP, "matmul_id: output must not overlap input");
    if (need_ids && overlap(ro, rids)) return fail(MM_ERR_OVERLAP, "matmul_id: output must not overlap expert ids");
    if (need_scr) {
        if (counts.ptr == nullptr || routed.ptr == nullptr)
            return fail(MM_ERR_SCRATCH, "matmul_id: grouped prefill requires caller-owned scratch");
        if (counts.bytes < cap->counts_bytes || routed.bytes < cap->routed_rows_bytes)
            return fail(MM_ERR_SCRATCH,
                        "matmul_id: scratch holds %llu/%llu bytes, needs %llu/%llu (counts/routed rows)",
                        (unsigned long long)counts.bytes, (unsigned long long)routed.bytes,
                        (unsigned long long)cap->counts_bytes, (unsigned long long)cap->routed_rows_bytes);
        if ((st = check_buf("matmul_id scratch counts", counts, 0, cap->counts_bytes, 4, &rc)) != MM_OK)
            return st;
        if ((st = check_buf("matmul_id scratch routed rows", routed, 0, cap->routed_rows_bytes, 4, &rr)) != MM_OK)
            return st;
        if (overlap(rc, rr)) return fail(MM_ERR_OVERLAP, "matmul_id: scratch counts overlap routed rows");
        if (overlap(rc, ro) || overlap(rr, ro)) return fail(MM_ERR_OVERLAP, "matmul_id: scratch must not overlap the output");
        if (need_ids && (overlap(rc, rids) || overlap(rr, rids)))
            return fail(MM_ERR_OVERLAP, "matmul_id: scratch must not overlap expert ids");
        if (need_w && (overlap(rc, rw) || overlap(rr, rw)))
            return fail(MM_ERR_OVERLAP, "matmul_id: scratch must not overlap weights");
        if (need_in && (overlap(rc, ri) || overlap(rr, ri)))
            return fail(MM_ERR_OVERLAP, "matmul_id: scratch must not overlap input");
    }
    return MM_OK;
}

mmk::IdArgs fill_ptrs(mmk::IdArgs a, mm_buf weights, mm_buf input, mm_buf ids, mm_buf out,
                      mm_buf counts, mm_buf routed) {
    a.W = weights.ptr;
    a.X = static_cast<const float*>(input.ptr);
    a.ids = static_cast<const uint32_t*>(ids.ptr);
    a.out = static_cast<float*>(out.ptr);
    a.counts = static_cast<const uint32_t*>(counts.ptr);
    a.routed_rows = static_cast<const uint32_t*>(routed.ptr);
    a.counts_w = static_cast<uint32_t*>(counts.ptr);
    a.routed_rows_w = static_cast<uint32_t*>(routed.ptr);
    return a;
}

// Route choice: skinny, else GEMV, else tiled GEMM (see mm.h).
mm_status dispatch_gemm(const GemmPlan& p, void* stream, mm_receipt* receipt) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    mmk::SkinnyArgs g;
    if (skinny_args(p, &g) && skinny_pays(g, p.dt)) return run_skinny(g, p.dt, s, receipt);
    if (p.m == 1 || p.n == 1) return run_gemv(p, s, receipt);
    return run_gemm(p, s, receipt);
}

// Route suggestion. Crossover between the routes, in routed rows per expert
// (m * top_k / n_experts), measured on MI355X over token counts 1..512 for
// 64-expert 1408 x 2048 and 16-expert 2048 x 2048 layers with bf16, f16 and
// f32 weights: the grouped route wins from 2 rows per expert on, where the
// direct route would read each expert's weights about twice. Routing
// concentrated on a hot subset of 8 to 32 experts moves the crossover by at
// most one doubling of the token count, because the grouped pass sizes its
// tiles for min(n_experts, m * top_k) experts. Layouts that leave the
// grouped pass on FMA tiles (f16/f32 weights with k % 128 != 0 or unaligned
// operands) need about 16 rows per expert.
mm_status route_hint(mm_dtype weight_dtype, const mm_id_params* params, uint32_t* route) {
    if (!params || !route) return fail(MM_ERR_INVALID_ARGUMENT, "matmul_id route hint: null argument");
    mm_id_params q = *params;
    q.route = 0;
    mm_id_capability tmp;
    mm_status st = id_query(weight_dtype, &q, &tmp);
    if (st != MM_OK) return st;
    const uint64_t rows = (uint64_t)q.m * q.top_k;
    uint32_t r = 0;
    if (q.multiplicity == 0 && q.n_experts <= MM_ID_GROUPED_MAX_EXPERTS) {
        const bool fma_tiles = weight_dtype != MM_BF16 && q.k % 128 != 0;
        const uint64_t per_expert = fma_tiles ? 16 : 2;
        if (rows >= per_expert * q.n_experts) r = 1;
    }
    *route = r;
    return ok();
}

}  // namespace

extern "C" {

mm_status mm_gemm(const mm_gemm_desc* desc, mm_buf a, mm_buf b, mm_buf c, void* stream,
                  mm_receipt* receipt) {
    GemmPlan p;
    mm_status st = plan_gemm(desc, a, b, c, &p);
    if (st != MM_OK) return st;
    return dispatch_gemm(p, stream, receipt);
}

mm_status mm_gemm_ex(const mm_gemm_desc* desc, float alpha, float beta, mm_buf a, mm_buf b,
                     mm_buf c, void* stream, mm_receipt* receipt) {
    GemmPlan p;
    mm_status st = plan_gemm(desc, a, b, c, &p);
    if (st != MM_OK) return st;
    p.alpha = alpha;
    p.beta = beta;
    return dispatch_gemm(p, stream, receipt);
}

mm_status mm_gemm_route(const mm_gemm_desc* desc, uint32_t route, float alpha, float beta,
                        mm_buf a, mm_buf b, mm_buf c, void* stream, mm_receipt* receipt) {
    GemmPlan p;
    mm_status st = plan_gemm(desc, a, b, c, &p);
    if (st != MM_OK) return st;
    p.alpha = alpha;
    p.beta = beta;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (route) {
        case MM_ROUTE_GEMV:
            if (p.m != 1 && p.n != 1)
                return fail(MM_ERR_UNSUPPORTED, "gemm route: GEMV needs m == 1 or n == 1 (got m = %lld, n = %lld)",
                            (long long)p.m, (long long)p.n);
            return run_gemv(p, s, receipt);
        case MM_ROUTE_GEMV_WIDE: {
            mmk::SkinnyArgs g;
            if (!skinny_args(p, &g))
                return fail(MM_ERR_UNSUPPORTED,
                            "gemm route: the skinny route needs trans_a = 0, trans_b = 1, one side of "
                            "2..64 rows and the 16-byte layout");
            return run_skinny(g, p.dt, s, receipt);
        }
        case MM_ROUTE_GEMM:
            return run_gemm(p, s, receipt);
        default:
            return fail(MM_ERR_INVALID_ARGUMENT, "gemm route: %u is not a GEMM route", route);
    }
}

mm_status mm_gemv(const mm_gemm_desc* desc, mm_buf a, mm_buf b, mm_buf c, void* stream,
                  mm_receipt* receipt) {
    GemmPlan p;
    mm_status st = plan_gemm(desc, a, b, c, &p);
    if (st != MM_OK) return st;
    if (p.m != 1 && p.n != 1)
        return fail(MM_ERR_INVALID_ARGUMENT, "gemv: needs m == 1 or n == 1 (got m = %lld, n = %lld)",
                    (long long)p.m, (long long)p.n);
    return run_gemv(p, static_cast<hipStream_t>(stream), receipt);
}

mm_status mm_id_query(mm_dtype weight_dtype, const mm_id_params* params, mm_id_capability* out) {
    mm_id_capability tmp;
    mm_status st = id_query(weight_dtype, params, out ? out : &tmp);
    return st == MM_OK ? ok() : st;
}

mm_status mm_id_route_hint(mm_dtype weight_dtype, const mm_id_params* params, uint32_t* route) {
    return route_hint(weight_dtype, params, route);
}

mm_status mm_id_direct(const mm_id_params* params, mm_dtype weight_dtype, mm_buf weights,
                       mm_buf input, mm_buf ids, mm_buf out, void* stream, mm_receipt* receipt) {
    mm_id_capability cap;
    mm_status st = id_validate(USE_DIRECT, params, weight_dtype, weights, input, ids, out,
                               mm_buf{nullptr, 0}, mm_buf{nullptr, 0}, &cap);
    if (st != MM_OK) return st;
    if ((st = resolve("id_direct")) != MM_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    mmk::IdArgs a = fill_ptrs(id_args(params, weight_dtype), weights, input, ids, out,
                              mm_buf{nullptr, 0}, mm_buf{nullptr, 0});
    ++g_launches;
    mmk::Launched L;
    if ((st = finish(mmk::launch_id_direct(a, s, &L), s, "id_direct")) != MM_OK) return st;
    set_receipt(receipt, MM_ROUTE_ID_DIRECT, (uint32_t)weight_dtype, 1, L);
    return ok();
}

mm_status mm_id_map(const mm_id_params* params, mm_buf ids, mm_buf counts, mm_buf routed_rows,
                    mm_buf out, void* stream, mm_receipt* receipt) {
    mm_id_capability cap;
    // The map pass reads no weights: their dtype, stride and extent are not checked.
    mm_status st = id_validate(USE_MAP, params, MM_F32, mm_buf{nullptr, 0}, mm_buf{nullptr, 0},
                               ids, out, counts, routed_rows, &cap);
    if (st != MM_OK) return st;
    if ((st = resolve("id_map")) != MM_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    mmk::IdArgs a = fill_ptrs(id_args(params, MM_F32), mm_buf{nullptr, 0}, mm_buf{nullptr, 0}, ids,
                              out, counts, routed_rows);
    ++g_launches;
    mmk::Launched L;
    if ((st = finish(mmk::launch_id_map(a, s, &L), s, "id_map")) != MM_OK) return st;
    set_receipt(receipt, MM_ROUTE_ID_MAP, (uint32_t)MM_F32, 1, L);
    return ok();
}

mm_status mm_id_grouped(const mm_id_params* params, mm_dtype weight_dtype, mm_buf weights,
                        mm_buf input, mm_buf counts, mm_buf routed_rows, mm_buf out, void* stream,
                        mm_receipt* receipt) {
    mm_id_capability cap;
    mm_status st = id_validate(USE_GROUPED, params, weight_dtype, weights, input,
                               mm_buf{nullptr, 0}, out, counts, routed_rows, &cap);
    if (st != MM_OK) return st;
    if ((st = resolve("id_grouped")) != MM_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    mmk::IdArgs a = fill_ptrs(id_args(params, weight_dtype), weights, input, mm_buf{nullptr, 0},
                              out, counts, routed_rows);
    ++g_launches;
    mmk::Launched L;
    if ((st = finish(mmk::launch_id_grouped(a, s, &L), s, "id_grouped")) != MM_OK) return st;
    set_receipt(receipt, MM_ROUTE_ID_GROUPED, (uint32_t)weight_dtype, 1, L);
    return ok();
}

mm_status mm_id(const mm_id_params* params, mm_dtype weight_dtype, mm_buf weights, mm_buf input,
                mm_buf ids, mm_buf out, mm_buf counts, mm_buf routed_rows, void* stream,
                mm_receipt* receipt) {
    if (params && params->route == 0)
        return mm_id_direct(params, weight_dtype, weights, input, ids, out, stream, receipt);
    mm_id_capability cap;
    mm_status st = id_validate(USE_PREFILL, params, weight_dtype, weights, input, ids, out,
                               counts, routed_rows, &cap);
    if (st != MM_OK) return st;
    // Resolve both launches before enqueueing the first.
    if ((st = resolve("id_map")) != MM_OK) return st;
    if ((st = resolve("id_grouped")) != MM_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    mmk::IdArgs a = fill_ptrs(id_args(params, weight_dtype), weights, input, ids, out, counts,
                              routed_rows);
    mmk::Launched L;
    ++g_launches;
    if ((st = finish(mmk::launch_id_map(a, s, &L), s, "id_map")) != MM_OK) return st;
    ++g_launches;
    if ((st = finish(mmk::launch_id_grouped(a, s, &L), s, "id_grouped")) != MM_OK) return st;
    set_receipt(receipt, MM_ROUTE_ID_PREFILL, (uint32_t)weight_dtype, 2, L);
    return ok();
}

mm_status mm_id_prefill_noalloc(const mm_id_params* params, mm_dtype weight_dtype, mm_buf weights,
                                mm_buf input, mm_buf ids, mm_buf out, void* stream,
                                mm_receipt* receipt) {
    mm_id_capability cap;
    mm_status st = id_validate(USE_PREFILL_NOALLOC, params, weight_dtype, weights, input, ids, out,
                               mm_buf{nullptr, 0}, mm_buf{nullptr, 0}, &cap);
    if (st != MM_OK) return st;
    const uint64_t counts_span = (cap.counts_bytes + 255) / 256 * 256;
    if (counts_span + cap.routed_rows_bytes > mmk::kStaticScratchBytes)
        return fail(MM_ERR_SCRATCH,
                    "matmul_id no-alloc prefill: scratch needs %llu + %llu bytes, the library's "
                    "array holds %llu",
                    (unsigned long long)counts_span, (unsigned long long)cap.routed_rows_bytes,
                    (unsigned long long)mmk::kStaticScratchBytes);
    if ((st = resolve("id_map")) != MM_OK) return st;
    if ((st = resolve("id_grouped")) != MM_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* base = nullptr;
    hipError_t err = mmk::static_scratch(s, &base);
    if (err != hipSuccess)
        return fail(MM_ERR_DEVICE, "matmul_id no-alloc prefill: scratch address lookup failed: %s",
                    hipGetErrorString(err));
    mm_buf counts{base, cap.counts_bytes};
    mm_buf routed{static_cast<char*>(base) + counts_span, cap.routed_rows_bytes};
    mmk::IdArgs a = fill_ptrs(id_args(params, weight_dtype), weights, input, ids, out, counts,
                              routed);
    mmk::Launched L;
    ++g_launches;
    if ((st = finish(mmk::launch_id_map(a, s, &L), s, "id_map")) != MM_OK) return st;
    ++g_launches;
    if ((st = finish(mmk::launch_id_grouped(a, s, &L), s, "id_grouped")) != MM_OK) return st;
    set_receipt(receipt, MM_ROUTE_ID_PREFILL, (uint32_t)weight_dtype, 2, L);
    return ok();
}

mm_status mm_capabilities(int device, mm_device_caps* out) {
    if (!out) return fail(MM_ERR_INVALID_ARGUMENT, "capabilities: null output");
    hipDeviceProp_t prop;
    hipError_t err = hipGetDeviceProperties(&prop, device);
    if (err != hipSuccess)
        return fail(MM_ERR_DEVICE, "capabilities: hipGetDeviceProperties(%d): %s", device,
                    hipGetErrorString(err));
    std::memset(out, 0, sizeof *out);
    std::snprintf(out->arch, sizeof out->arch, "%s", prop.gcnArchName);
    out->cu_count = prop.multiProcessorCount;
    out->max_clock_mhz = prop.clockRate / 1000;
    out->l2_bytes = prop.l2CacheSize;
    out->hbm_bytes = prop.totalGlobalMem;
    out->xcd_count = 8;
    out->dtype_mask = (1u << MM_F32) | (1u << MM_F16) | (1u << MM_BF16);
    out->max_grouped_experts = MM_ID_GROUPED_MAX_EXPERTS;
    out->abi_version = MM_ABI_VERSION;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(MM_ERR_UNSUPPORTED, "capabilities: device %d is %s; the kernels are built for gfx950",
                    device, prop.gcnArchName);
    return ok();
}

const char* mm_status_string(mm_status s) {
    switch (s) {
        case MM_OK: return "ok";
        case MM_ERR_INVALID_ARGUMENT: return "invalid argument";
        case MM_ERR_UNSUPPORTED: return "unsupported";
        case MM_ERR_BUFFER_TOO_SMALL: return "buffer too small";
        case MM_ERR_MISALIGNED: return "misaligned";
        case MM_ERR_OVERLAP: return "overlapping buffers";
        case MM_ERR_SCRATCH: return "scratch missing or too small";
        case MM_ERR_DEVICE: return "device error";
    }
    return "unknown status";
}

const char* mm_last_error(void) { return g_error.c_str(); }

void mm_test_inject_resolve_failure(const char* name) { g_inject = name ? name : ""; }

uint64_t mm_test_launch_count(void) { return g_launches; }

}  // extern "C"
