/*
 * mm.h -- C ABI of the MI355X (gfx950) matrix-product dispatch library
 * (libmm.so): C = op(A).op(B) with a GEMV route and an MFMA GEMM route, and
 * the expert-ID matmul (direct route; map + grouped route).
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Memory: the caller owns all device memory and the stream. The library
 *   never allocates device memory on a call, keeps no state between calls and
 *   holds no pointer after returning. (mlx-native dense_matmul_id.rs, module
 *   doc: no conversion, shadow allocation or dequantization; caller-owned
 *   scratch.)
 * - Buffers are passed as mm_buf {ptr, bytes}: a device pointer and the
 *   number of bytes the caller vouches for from that pointer. Every call
 *   checks that the bytes it will touch lie inside [ptr, ptr + bytes).
 * - Fail-closed: each call validates everything on the host before it
 *   enqueues anything (mlx-native dense_matmul_id.rs, `dense_matmul_id`:
 *   every pipeline is resolved and every limit checked before encoding; test
 *   `grouped_pipeline_resolution_failure_does_not_mutate_encoder`). A call
 *   that returns an error other than MM_ERR_DEVICE has enqueued nothing.
 *   MM_ERR_DEVICE means the HIP runtime refused a launch after validation;
 *   the one call that makes two launches (mm_id with the grouped route) may
 *   then leave its first launch, the map pass, enqueued (see mm_id).
 * - Asynchrony: on MM_OK the work is enqueued on `stream` (a hipStream_t; 0 =
 *   the null stream) and results are valid once the stream has reached that
 *   point. Stream order is the only ordering: a map launch followed by a
 *   grouped launch on the same stream sees the map's results, and a later
 *   call reusing the same scratch waits for the earlier one. Using one
 *   scratch buffer on two streams at once is the caller's race.
 * - Errors: an mm_status code; mm_last_error() gives a per-thread message
 *   for the last failing call on that thread.
 * - Receipts: every compute entry point takes an optional mm_receipt* that
 *   is filled on success with the route taken and the number of kernel
 *   launches enqueued (mlx-native `DenseMatmulIdDispatchReceipt`).
 * - Setting MM_DEBUG_SYNC=1 in the environment makes each launch synchronize
 *   its stream and report a device error as MM_ERR_DEVICE (the analogue of
 *   the `debug` wait in tract-metal `dispatch_metal_mlx_gemm`).
 */
#ifndef MM_H
#define MM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MM_ABI_VERSION 1u
/* Schema version of capability/receipt records (mlx-native
 * `DENSE_MATMUL_ID_SCHEMA_VERSION`). */
#define MM_ID_SCHEMA_VERSION 5u
/* Largest expert count the grouped route accepts (mlx-native
 * `GROUPED_MAX_EXPERTS`). */
#define MM_ID_GROUPED_MAX_EXPERTS 1024u

typedef enum {
    MM_OK = 0,
    MM_ERR_INVALID_ARGUMENT = 1, /* bad dimension, flag, stride or route */
    MM_ERR_UNSUPPORTED = 2,      /* dtype or device the library does not handle */
    MM_ERR_BUFFER_TOO_SMALL = 3, /* an extent exceeds the buffer's byte length */
    MM_ERR_MISALIGNED = 4,       /* address not aligned to the element size */
    MM_ERR_OVERLAP = 5,          /* an output range overlaps an input range */
    MM_ERR_SCRATCH = 6,          /* grouped-route scratch missing or too small */
    MM_ERR_DEVICE = 7            /* the HIP runtime reported an error */
} mm_status;

typedef enum { MM_F32 = 0, MM_F16 = 1, MM_BF16 = 2 } mm_dtype;

typedef struct {
    void *ptr;      /* device address */
    uint64_t bytes; /* bytes valid from ptr */
} mm_buf;

typedef enum {
    MM_ROUTE_GEMV = 0,
    MM_ROUTE_GEMM = 1,
    MM_ROUTE_ID_DIRECT = 2,
    MM_ROUTE_ID_MAP = 3,
    MM_ROUTE_ID_GROUPED = 4,
    MM_ROUTE_ID_PREFILL = 5, /* map + grouped in one call */
    MM_ROUTE_GEMV_WIDE = 6   /* skinny product: 2..64 rows on one side */
} mm_route;

/* Kernel family of a launch (reported in receipts; the choice depends on
 * shape, layout and alignment). */
typedef enum {
    MM_KERNEL_GEMV_ROWS = 0,         /* matrix rows along K, 16-byte streaming loads */
    MM_KERNEL_GEMV_ROWS_ELEM = 1,    /* matrix rows along K, element loads */
    MM_KERNEL_GEMV_COLS = 2,         /* outputs contiguous in the matrix */
    MM_KERNEL_GEMM_TILED = 3,        /* 128 x 128 MFMA tiles, any layout and edge */
    MM_KERNEL_GEMM_LARGE = 4,        /* DMA-pipelined MFMA tiles of 256 x 256 or 128 x 128, any layout, any m, n; k % 128 == 0 */
    MM_KERNEL_GEMM_F32 = 5,          /* f32 FMA tiles */
    MM_KERNEL_ID_DIRECT_FAST = 6,    /* direct route, 16-byte loads, one id-row load */
    MM_KERNEL_ID_DIRECT = 7,         /* direct route, general */
    MM_KERNEL_ID_MAP = 8,            /* map pass */
    MM_KERNEL_ID_GROUPED_MFMA = 9,   /* grouped pass on MFMA (bf16 weights; f16/f32 when k % 128 == 0 and aligned) */
    MM_KERNEL_ID_GROUPED_FMA = 10,   /* grouped pass, FMA tiles (other f16/f32 layouts) */
    MM_KERNEL_GEMV_WIDE = 11,        /* skinny route, one to four 16 x 16 MFMA fragments per block */
    MM_KERNEL_GEMM_F32_SMALL = 12,   /* f32, k <= 128, few tiles: one wave per 16 x 16 f32 MFMA tile */
    MM_KERNEL_GEMM_PANEL = 13        /* NT, k in {32, 64, 128}: 64- or 128-row A panel in LDS, B tiles streamed */
} mm_kernel;

typedef struct {
    uint32_t schema_version;  /* MM_ID_SCHEMA_VERSION */
    uint32_t route;           /* mm_route actually taken */
    uint32_t dtype;           /* mm_dtype of A/B/C or of the expert weights */
    uint32_t dispatch_count;  /* kernel launches enqueued by the call */
    uint32_t kernel;          /* mm_kernel of the last launch */
    uint32_t variant;         /* instance of that kernel family: for
                                 MM_KERNEL_ID_GROUPED_MFMA the 16-output
                                 fragment slots per wave of the pipelined
                                 form (2 or 4 on 4 waves; 3 + 256 * 8 for its
                                 8-wave instance), 0 for the 8-wave
                                 LDS-split bf16 form; for MM_KERNEL_ID_DIRECT_FAST 0
                                 when activations come from L2, 1 when the
                                 block stages its activation row in LDS, 2
                                 when it also reuses a repeated expert's
                                 weights across slots (slotted layout); for
                                 MM_KERNEL_GEMV_WIDE the activation fragments
                                 per block (one per 16 rows, up to 4);
                                 for MM_KERNEL_GEMM_PANEL the number of blocks
                                 a panel's B tiles are split over, plus 256
                                 times the panel height in rows (64 or 128);
                                 for MM_KERNEL_GEMM_LARGE the tile edge
                                 (256 or 128), plus 1 for the paired-stage
                                 form (two k-stages per LDS region); 0 for
                                 every other family */
} mm_receipt;

/* ------------------------------------------------------------------------ */
/* Matrix product C = op(A) . op(B)                                          */
/* ------------------------------------------------------------------------ */
/*
 * tract-metal 0.23.6 mlx_gemm/mod.rs, `dispatch_eval`,
 * `dispatch_metal_mlx_gemv` and `dispatch_metal_mlx_gemm`; rlx-metal 0.2.14
 * mps_blas.rs, `encode_mps_sgemm_t` for the op() storage convention.
 *
 * For b < batch, i < m, j < n:
 *   C[b][i][j] = sum_{p<k} op(A)[b][i][p] * op(B)[b][p][j]
 * A, B and C share one dtype (f32, f16 or bf16); products are accumulated in
 * f32 and the result is rounded once to the dtype (nearest, ties to even).
 * C is overwritten (alpha = 1, beta = 0).
 *
 * Storage (all element counts, not bytes, except the offsets):
 *   trans_a = 0: A[b] stored [m, k], element (i,p) at i*lda + p
 *   trans_a = 1: A[b] stored [k, m], element (i,p) at p*lda + i
 *   trans_b = 0: B[b] stored [k, n], element (p,j) at p*ldb + j
 *   trans_b = 1: B[b] stored [n, k], element (p,j) at j*ldb + p
 *   C[b] stored [m, n],             element (i,j) at i*ldc + j
 *   matrix b of X starts at offset_x / elt + b * stride_x.
 * lda/ldb/ldc = 0 means tight (the stored row length); otherwise they must be
 * at least that. stride_a / stride_b = 0 broadcasts one matrix to every batch;
 * stride_c = 0 means m*ldc, and a nonzero stride_c must keep batches
 * disjoint. Offsets are bytes and must be multiples of the element size.
 * All of batch, m, n, k must be >= 1.
 */
typedef struct {
    mm_dtype dtype;
    int32_t trans_a, trans_b;
    int64_t batch, m, n, k;
    int64_t lda, ldb, ldc;
    int64_t stride_a, stride_b, stride_c;
    uint64_t offset_a, offset_b, offset_c;
} mm_gemm_desc;

/*
 * Dispatch (tract-metal `dispatch_eval`, with `gemv_wide_config` deciding the
 * skinny case first):
 *   - skinny route (MM_ROUTE_GEMV_WIDE) when trans_a == 0, trans_b == 1, one
 *     of m, n is in 2..64 and the other is >= 2, and the 16-byte layout holds:
 *     k, lda, ldb, stride_a and stride_b multiples of 16 / element size and
 *     16-byte aligned A and B (after their offsets); and the route's blocks
 *     (batch x ceil(other side / 16), 768, 512 or 256 resident at once for
 *     up to 16, 32 or 64 skinny rows) run in one round, or in more rounds with
 *     long rows: k x element size >= 512 bytes for two rounds and >= 1024
 *     beyond with up to 32 skinny rows, at most three rounds with 33..64
 *     (measured crossover against the tiled GEMM);
 *   - the GEMV route when m == 1 or n == 1 (the matrix operand is B when
 *     n != 1, else A);
 *   - the tiled MFMA GEMM route otherwise.
 * All routes compute the same product. Errors: INVALID_ARGUMENT (dims, flags, ld, strides),
 * UNSUPPORTED (dtype), MISALIGNED (ptr + offset not element aligned),
 * BUFFER_TOO_SMALL, OVERLAP (C's range meets A's or B's), DEVICE.
 */
mm_status mm_gemm(const mm_gemm_desc *desc, mm_buf a, mm_buf b, mm_buf c, void *stream,
                  mm_receipt *receipt);

/*
 * Same dispatch with an output epilogue (tract-metal `dispatch_metal_mlx_gemm`
 * function constants `do_axpby` and `use_out_source`, present but switched off
 * there; rlx-metal `encode_mps_sgemm_t` passes alpha = 1, beta = 0):
 *   C[b][i][j] = alpha * sum_p op(A)[b][i][p] * op(B)[b][p][j] + beta * C_old[b][i][j]
 * computed in f32 from the f32 accumulator and the old value as stored,
 * rounded once to the dtype. With beta == 0 the old C is never read (its
 * contents, NaN included, do not matter); mm_gemm is alpha = 1, beta = 0.
 * Same routes, validation and errors as mm_gemm.
 */
mm_status mm_gemm_ex(const mm_gemm_desc *desc, float alpha, float beta, mm_buf a, mm_buf b,
                     mm_buf c, void *stream, mm_receipt *receipt);

/*
 * The same product on a route the caller names (route = MM_ROUTE_GEMV,
 * MM_ROUTE_GEMV_WIDE or MM_ROUTE_GEMM), with the mm_gemm_ex epilogue. For
 * callers that choose or calibrate routes themselves (mlx-native
 * dense_matmul_id.rs, `DenseMatmulIdParams`: route selection belongs to the
 * caller; rlx-metal mps_blas.rs module doc: the route crossover is measured,
 * not assumed). Every route computes the same values. Fails with
 * UNSUPPORTED when the named route cannot take the problem (GEMV: m != 1 and
 * n != 1; skinny: the shape and layout conditions of mm_gemm's skinny case,
 * without its rounds rule), else as
 * mm_gemm_ex; INVALID_ARGUMENT for any other route value.
 */
mm_status mm_gemm_route(const mm_gemm_desc *desc, uint32_t route, float alpha, float beta,
                        mm_buf a, mm_buf b, mm_buf c, void *stream, mm_receipt *receipt);

/* The GEMV route only; INVALID_ARGUMENT unless m == 1 or n == 1
 * (tract-metal `dispatch_metal_mlx_gemv`). Same validation as mm_gemm. */
mm_status mm_gemv(const mm_gemm_desc *desc, mm_buf a, mm_buf b, mm_buf c, void *stream,
                  mm_receipt *receipt);

/* ------------------------------------------------------------------------ */
/* Expert-ID matmul                                                          */
/* ------------------------------------------------------------------------ */
/*
 * mlx-native 0.13.0 dense_matmul_id.rs: module doc, `DenseMatmulIdParams`,
 * `dense_matmul_id_capability`, `dense_matmul_id`.
 *
 * Weights: a stack of n_experts row-major [n, k] matrices (f32, f16 or bf16);
 * expert e starts expert_stride_bytes * e bytes after weights.ptr. Input:
 * f32. Ids: u32 [m, top_k]. Output: f32 [m, top_k, n]. For the routed row
 * r = t*top_k + s (token t, slot s) and e = ids[r]:
 *   e <  n_experts: out[r][j] = sum_p W_e[j][p] * x_{t,s}[p]  (f32 accumulate)
 *   e >= n_experts: out[r][:] = +0.0, and no weight address is formed
 * x_{t,s} is row t of a [m, k] input (layout 0: shared per token) or row r of
 * a [m*top_k, k] input (layout 1: slotted).
 */
typedef struct {
    uint32_t m, n, k, top_k, n_experts; /* all >= 1 */
    uint64_t expert_stride_bytes;       /* >= n*k*elt and a multiple of elt */
    uint32_t input_layout;              /* 0 shared per token, 1 slotted */
    uint32_t multiplicity;              /* 0 distinct per token (a caller promise), 1 may repeat */
    uint32_t route;                     /* 0 direct, 1 grouped prefill (chosen by the caller) */
} mm_id_params;

typedef struct {
    uint32_t schema_version; /* MM_ID_SCHEMA_VERSION */
    uint32_t weight_dtype;   /* mm_dtype */
    uint32_t route;          /* 0 direct, 1 grouped prefill */
    uint32_t reserved;
    uint64_t weight_bytes;   /* (n_experts-1)*expert_stride_bytes + n*k*elt */
    uint64_t input_bytes;    /* (m or m*top_k) * k * 4 */
    uint64_t ids_bytes;      /* m*top_k*4 */
    uint64_t output_bytes;   /* m*top_k*n*4 */
    uint64_t counts_bytes;   /* grouped: n_experts*4; direct: 0 */
    uint64_t routed_rows_bytes; /* grouped: n_experts*m*4; direct: 0 */
} mm_id_capability;

/*
 * Host-only capability and exact byte extents (mlx-native
 * `dense_matmul_id_capability`); touches no device. Fails with
 * INVALID_ARGUMENT when a dimension is 0, distinct top_k exceeds n_experts,
 * the stride is too small or misaligned, an extent overflows 64 bits,
 * m*top_k exceeds 2^32-1, the grouped route is asked for with may-repeat ids
 * or more than MM_ID_GROUPED_MAX_EXPERTS experts; UNSUPPORTED for a weight
 * dtype outside f32/f16/bf16.
 */
mm_status mm_id_query(mm_dtype weight_dtype, const mm_id_params *params, mm_id_capability *out);

/*
 * Route suggestion (host only). The pages leave the route to the caller
 * (mlx-native `DenseMatmulIdParams`: route chosen by the caller); this
 * reports the one measured to be faster on MI355X for the given problem:
 * 1 (grouped prefill) when the grouped route is allowed (distinct ids per
 * token, n_experts <= MM_ID_GROUPED_MAX_EXPERTS) and
 * m * top_k >= c * n_experts, with c = 2, or c = 16 for f16/f32 weights
 * when k % 128 != 0 (the grouped pass then runs FMA tiles); otherwise 0
 * (direct). params->route is ignored. Errors as
 * mm_id_query (validation of everything but the route).
 */
mm_status mm_id_route_hint(mm_dtype weight_dtype, const mm_id_params *params, uint32_t *route);

/*
 * Direct route: one launch computes every routed row
 * (mlx-native `DenseMatmulIdRoute::Direct`). Requires params->route == 0.
 * Repeated ids are allowed. Buffers: weights (weight_dtype), input f32, ids
 * u32, out f32, each at least its capability extent; out must not overlap
 * weights, input or ids (OVERLAP); every pointer must be aligned to its
 * element size (MISALIGNED).
 */
mm_status mm_id_direct(const mm_id_params *params, mm_dtype weight_dtype, mm_buf weights,
                       mm_buf input, mm_buf ids, mm_buf out, void *stream, mm_receipt *receipt);

/*
 * Map pass of the grouped route (mlx-native `dense_matmul_id`, grouped
 * branch, first dispatch). Writes
 *   counts[e]            = #{ r < m*top_k : ids[r] == e }             (u32 [n_experts])
 *   routed_rows[e*m + i] = the i-th smallest such r, i < counts[e]    (u32 [n_experts, m])
 * and sets out[r][:] = +0.0 for every r with ids[r] >= n_experts. Lists are
 * ascending, so the results are deterministic. Entries past counts[e] are
 * unspecified. Requires params->route == 1 (distinct ids per token,
 * n_experts <= 1024); counts and routed_rows must hold the capability's
 * scratch extents (SCRATCH) and overlap neither each other, ids nor out
 * (OVERLAP). If the distinct promise is broken a list is cut at m entries,
 * so no write leaves the buffers; the output is then unspecified.
 */
mm_status mm_id_map(const mm_id_params *params, mm_buf ids, mm_buf counts, mm_buf routed_rows,
                    mm_buf out, void *stream, mm_receipt *receipt);

/*
 * Grouped pass (second dispatch): for every expert e and each routed row r
 * in its list, out[r][:] = W_e . x_{t,s}. Reads counts and routed_rows as
 * the map pass left them on this stream; rows of invalid ids are not
 * touched here. Same buffer rules as mm_id_direct plus the scratch rules of
 * mm_id_map; routed_rows entries outside [0, m*top_k) are skipped.
 */
mm_status mm_id_grouped(const mm_id_params *params, mm_dtype weight_dtype, mm_buf weights,
                        mm_buf input, mm_buf counts, mm_buf routed_rows, mm_buf out,
                        void *stream, mm_receipt *receipt);

/*
 * The whole expert-ID matmul in one call, by params->route: the direct launch,
 * or the map launch followed by the grouped launch (mlx-native
 * `dense_matmul_id`). Everything for both launches is validated and resolved
 * before the first is enqueued. counts / routed_rows are ignored by the
 * direct route. If the HIP runtime refuses the grouped launch after the map
 * launch was accepted, the call returns MM_ERR_DEVICE with the map pass still
 * enqueued: it then writes only the scratch (counts, routed_rows) and the
 * +0.0 rows of invalid ids, and the rest of the output is unspecified.
 */
mm_status mm_id(const mm_id_params *params, mm_dtype weight_dtype, mm_buf weights, mm_buf input,
                mm_buf ids, mm_buf out, mm_buf counts, mm_buf routed_rows, void *stream,
                mm_receipt *receipt);

/*
 * The grouped prefill (map launch, then grouped launch) without caller
 * scratch and without any allocation: for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same results, validation and errors as
 * mm_id with params->route == 1, except that counts and routed_rows live in
 * an array the library holds on each GPU (MM_ID_NOALLOC_SCRATCH_BYTES, kept
 * until the process ends): counts at its start, routed rows at the next
 * 256-byte boundary. A problem whose scratch does not fit
 * (round_up(4 * n_experts, 256) + 4 * n_experts * m bytes above the limit)
 * fails with MM_ERR_SCRATCH before anything is enqueued. The call makes no
 * hipMalloc / hipFree and calls no allocating routine; its first call on a
 * GPU looks up that GPU's array address once (a runtime query, not a stream
 * operation: make that first call outside stream capture; later calls can be
 * captured in a HIP graph and replayed). Every call on one GPU shares
 * the array: calls that overlap on one GPU (two streams at once) race and
 * give unspecified results. The caller still passes inputs and outputs.
 */
#define MM_ID_NOALLOC_SCRATCH_BYTES (4u << 20)
mm_status mm_id_prefill_noalloc(const mm_id_params *params, mm_dtype weight_dtype,
                                mm_buf weights, mm_buf input, mm_buf ids, mm_buf out,
                                void *stream, mm_receipt *receipt);

/* ------------------------------------------------------------------------ */
/* Device and library information                                            */
/* ------------------------------------------------------------------------ */

typedef struct {
    char arch[64];                /* gcnArchName, e.g. "gfx950:sramecc+:xnack-" */
    int32_t cu_count;
    int32_t max_clock_mhz;
    int32_t l2_bytes;
    int32_t xcd_count;            /* 8 on MI355X */
    uint64_t hbm_bytes;
    uint32_t dtype_mask;          /* bit d set: dtype d supported */
    uint32_t max_grouped_experts; /* MM_ID_GROUPED_MAX_EXPERTS */
    uint32_t abi_version;         /* MM_ABI_VERSION */
    uint32_t reserved;
} mm_device_caps;

/* Fills `out` for HIP device `device`; UNSUPPORTED when it is not a gfx950
 * (the only architecture the kernels are built for), DEVICE on a HIP error.
 * The counterpart of tract-metal mlx_gemm/mod.rs `device_arch_gen`, which
 * reads the GPU architecture generation once and gates kernels on it; here
 * the gate is the architecture name. */
mm_status mm_capabilities(int device, mm_device_caps *out);

/* Static description of a status code. The codes are the error classes of
 * mlx-native dense_matmul_id.rs (`MlxError::InvalidArgument` and friends
 * returned by `dense_matmul_id_capability` / `dense_matmul_id`), split by
 * cause. */
const char *mm_status_string(mm_status status);

/* Message for the last failing call on the calling thread ("" if none): the
 * detail text that mlx-native dense_matmul_id.rs puts inside each
 * `MlxError::InvalidArgument` (which dimension, extent or buffer failed). */
const char *mm_last_error(void);

/* ------------------------------------------------------------------------ */
/* Test hooks (host-side; used by the CPU test suite)                        */
/* ------------------------------------------------------------------------ */

/* Make the next launch-resolution step on this thread fail for the kernel
 * family `name` ("gemv", "gemv_wide", "gemm", "id_direct", "id_map",
 * "id_grouped"), before
 * anything is enqueued, like the pipeline-lookup failure injected in
 * mlx-native's `grouped_pipeline_resolution_failure_does_not_mutate_encoder`.
 * NULL clears it. */
void mm_test_inject_resolve_failure(const char *name);

/* Number of kernel launches this thread has attempted (enqueue calls made). */
uint64_t mm_test_launch_count(void);

#ifdef __cplusplus
}
#endif

#endif /* MM_H */
