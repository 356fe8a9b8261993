// Kernel argument blocks and host-side launchers. The launchers (defined in
// gemv.hip, gemm.hip, mmid.hip) pick a template instance, size the grid and
// enqueue exactly one kernel; they never validate (the C ABI layer has done
// that), report the kernel family and instance they chose through a
// `Launched` record, and return the hipError_t of the enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mm.h"

namespace mmk {

// Largest expert count of the grouped route (sizes the in-block tile table).
constexpr int MM_GROUPED_MAX_E = 1024;

// What a launcher enqueued: the mm_kernel family and a family-specific
// instance number (mm_receipt.variant).
struct Launched {
    int kernel = -1;
    int variant = 0;
};

// out[o * out_inc] = sum_p M(o, p) * vec[p * vec_inc] for o < rows, with
// M(o, p) = mat[o * ld + p] (row form) or mat[p * ld + o] (column form).
struct GemvArgs {
    const void* mat;
    const void* vec;
    void* out;
    int64_t rows, k, ld;
    int64_t vec_inc, out_inc;
    int64_t mat_bstride, vec_bstride, out_bstride;  // elements; 0 = shared
    int64_t batch;
    int32_t dtype;       // 0 f32, 1 f16, 2 bf16
    int32_t col_form;    // 1: M(o, p) = mat[p * ld + o]
    float alpha, beta;   // out = alpha * sum + beta * out_old (beta == 0: out_old unread)
};
// Launchers enqueue one kernel on `s` and describe it in *L.
hipError_t launch_gemv(const GemvArgs& a, hipStream_t s, Launched* L);

// Skinny product: out[b][x * out_sx + w * out_sw] = sum_p W[b](w, p) * X[b](x, p)
// for w < nw, x < nx (nx <= 64); W(w, p) = W[w * ldw + p], X(x, p) = X[x * ldx + p].
struct SkinnyArgs {
    const void* W;
    const void* X;
    void* out;
    int64_t nw, nx, k;
    int64_t ldw, ldx;
    int64_t out_sx, out_sw;
    int64_t sw, sx, so;  // batch strides, elements; 0 = shared
    int64_t batch;
    int64_t w_bytes, x_bytes;  // extent of one batch's W and X (each below 2^31)
    int32_t dtype;
    float alpha, beta;   // out = alpha * sum + beta * out_old (beta == 0: out_old unread)
};
hipError_t launch_gemv_wide(const SkinnyArgs& a, hipStream_t s, Launched* L);

// C[b] = op(A[b]) . op(B[b]); pointers already include the byte offsets.
struct GemmArgs {
    const void* A;
    const void* B;
    void* C;
    int64_t m, n, k;
    int64_t lda, ldb, ldc;
    int64_t sa, sb, sc;  // batch strides, elements
    int64_t batch;
    int32_t dtype;
    int32_t ta, tb;
    float alpha, beta;   // C = alpha * op(A) op(B) + beta * C_old (beta == 0: C_old unread)
};
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s, Launched* L);

// Expert-ID matmul. Byte strides locate the activation row of (token, slot).
struct IdArgs {
    const void* W;
    const float* X;
    const uint32_t* ids;
    float* out;
    const uint32_t* counts;       // grouped only
    const uint32_t* routed_rows;  // grouped only
    uint32_t* counts_w;           // map only
    uint32_t* routed_rows_w;      // map only
    uint32_t m, n, k, top_k, n_experts;
    uint32_t layout;              // 0 shared per token, 1 slotted
    uint64_t expert_stride_bytes;
    uint64_t x_tok_stride_bytes, x_slot_stride_bytes;
    int32_t wdtype;
    int32_t dedup;                // direct: repeated ids of one token share one pass
};
hipError_t launch_id_direct(const IdArgs& a, hipStream_t s, Launched* L);
hipError_t launch_id_map(const IdArgs& a, hipStream_t s, Launched* L);
hipError_t launch_id_grouped(const IdArgs& a, hipStream_t s, Launched* L);

// Library-held scratch for the allocation-free prefill call: its size, and
// its device address on the GPU of stream `s` (looked up once per GPU).
constexpr uint64_t kStaticScratchBytes = MM_ID_NOALLOC_SCRATCH_BYTES;
hipError_t static_scratch(hipStream_t s, void** out);

}  // namespace mmk
