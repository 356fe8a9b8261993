// Tiled GEMM route: C[b] = op(A[b]) . op(B[b]) for m > 1 and n > 1
// (tract-metal 0.23.6 mlx_gemm/mod.rs, `dispatch_metal_mlx_gemm`: tiled
// kernel over (n tiles, m tiles, batch), all four transpose layouts, batch
// strides, an aligned main K loop with a ragged tail; alpha = 1, beta = 0).
//
// f16/bf16: CDNA4 MFMA (v_mfma_f32_16x16x32_{f16,bf16}, f32 accumulate) on
// tiles staged through LDS in a K-contiguous [row][k] layout; operands stored
// with K strided are transposed while being written to LDS. f32: LDS-tiled
// FMA. Edges in M, N and K are zero-filled on load and masked on store.
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "kernels.hpp"

namespace mmk {

namespace {

// ---------------------------------------------------------------------------
// f16 / bf16 MFMA kernel (any layout)
// ---------------------------------------------------------------------------
constexpr int GBM = 128, GBN = 128, GBK = 32;
constexpr int GLDK = GBK + 8;  // LDS row pitch in elements (80 bytes)
constexpr int GThreads = 256;

template <class T>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (T::code == 1)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Tile staging, split into a global fetch (into registers, so later k-tiles
// are in flight while the current one is multiplied) and an LDS store.
// A chunk is 8 elements: 8 consecutive k of one row (KCONTIG: element (row, p)
// at base[row * ld + p]) or 8 consecutive rows at one k (else: base[p * ld +
// row]); out-of-range elements are zero.
//
// VEC (16-byte aligned chunks): one buffer load per chunk, unconditional, over
// a resource that spans exactly the operand's valid elements, so chunks past
// the last row (or k) read zero from the range check; the k (or row) tail of a
// chunk that straddles the edge is masked when the chunk is stored (`nv` keeps
// the valid count). Nothing touches a loaded value before the store, so the
// loads of several k-tiles stay in flight together.
constexpr int GCH = (GBM * GBK / 8) / GThreads;  // chunks per thread per operand

__device__ __forceinline__ u32x4 keep_first(u32x4 v, int64_t nvalid) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t lo = 2 * t < nvalid ? 0x0000ffffu : 0u;
        const uint32_t hi = 2 * t + 1 < nvalid ? 0xffff0000u : 0u;
        v[t] &= lo | hi;
    }
    return v;
}

template <bool KCONTIG, bool VEC>
__device__ __forceinline__ void fetch_tile(const uint16_t* __restrict__ base, int64_t ld,
                                           int64_t nrows, int64_t K, int64_t row0, int64_t k0,
                                           u32x4 (&v)[GCH], int (&nv)[GCH]) {
    const int tid = threadIdx.x;
    if constexpr (VEC) {
        // Valid span: (nrows-1)*ld + K elements (KCONTIG) or (K-1)*ld + nrows.
        const int64_t span = KCONTIG ? (nrows - 1) * ld + K : (K - 1) * ld + nrows;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(base), (short)0, (int)(span * 2), 0x00020000);
#pragma unroll
        for (int u = 0; u < GCH; ++u) {
            const int q = tid + u * GThreads;
            int64_t off, nvalid;
            if constexpr (KCONTIG) {
                const int row = q >> 2, kc = (q & 3) * 8;
                off = (row0 + row) * ld + k0 + kc;
                nvalid = K - (k0 + kc);
            } else {
                const int p = q >> 4, rc = (q & 15) * 8;
                off = (k0 + p) * ld + row0 + rc;
                nvalid = (k0 + p < K) ? nrows - (row0 + rc) : 0;
            }
            // Offsets past the span read zero; clamp so that 32 bits hold them.
            off = off < span ? off : span;
            v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       rs, (int)(off * 2), 0, 0));
            nv[u] = (int)(nvalid < 0 ? 0 : (nvalid > 8 ? 8 : nvalid));
        }
        return;
    }
#pragma unroll
    for (int u = 0; u < GCH; ++u) {
        const int q = tid + u * GThreads;
        uint32_t h[8];
        if constexpr (KCONTIG) {
            const int row = q >> 2, kc = (q & 3) * 8;
            const int64_t gr = row0 + row, gk = k0 + kc;
#pragma unroll
            for (int t = 0; t < 8; ++t)
                h[t] = (gr < nrows && gk + t < K) ? base[gr * ld + gk + t] : 0u;
        } else {
            const int p = q >> 4, rc = (q & 15) * 8;
            const int64_t gk = k0 + p, gr = row0 + rc;
#pragma unroll
            for (int t = 0; t < 8; ++t)
                h[t] = (gk < K && gr + t < nrows) ? base[gk * ld + gr + t] : 0u;
        }
        v[u] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                     h[6] | (h[7] << 16)};
        nv[u] = 8;
    }
}

// Write fetched chunks into LDS as [row][k] (pitch GLDK), zeroing the
// elements past each chunk's valid count.
template <bool KCONTIG>
__device__ __forceinline__ void store_tile(const u32x4 (&v)[GCH], const int (&nv)[GCH],
                                           uint16_t* __restrict__ lds) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < GCH; ++u) {
        const int q = tid + u * GThreads;
        const u32x4 c = keep_first(v[u], nv[u]);
        if constexpr (KCONTIG) {
            const int row = q >> 2, kc = (q & 3) * 8;
            *reinterpret_cast<u32x4*>(lds + row * GLDK + kc) = c;
        } else {
            const int p = q >> 4, rc = (q & 15) * 8;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                lds[(rc + 2 * t) * GLDK + p] = (uint16_t)(c[t] & 0xffffu);
                lds[(rc + 2 * t + 1) * GLDK + p] = (uint16_t)(c[t] >> 16);
            }
        }
    }
}

// Work item of the 128 x 128 kernels: (batch, tile) in an order where each
// XCD (blockIdx % 8) runs a contiguous run, batch-major, and within a batch
// groups of GGM tile-rows column-major: blocks resident on one XCD at a time
// share A and B panels in its L2. `slot` counts this block's items.
constexpr int GGM = 4;

struct TileItem {
    int64_t b, m0, n0;
};

__device__ __forceinline__ bool tile_item(const GemmArgs& a, int64_t slot, TileItem* it) {
    const int64_t tiles_m = (a.m + GBM - 1) / GBM, tiles_n = (a.n + GBN - 1) / GBN;
    const int64_t tiles = tiles_m * tiles_n, total = tiles * a.batch;
    const int64_t per_xcd = (total + 7) / 8;
    if (slot >= per_xcd) return false;
    const int64_t t = (int64_t)(blockIdx.x % 8) * per_xcd + slot;
    if (t >= total) return false;
    const int64_t r = t % tiles;
    const int64_t group = r / (GGM * tiles_n);
    const int64_t first_m = group * GGM;
    const int64_t gsize = tiles_m - first_m < GGM ? tiles_m - first_m : GGM;
    it->b = t / tiles;
    it->m0 = (first_m + (r % (GGM * tiles_n)) % gsize) * GBM;
    it->n0 = ((r % (GGM * tiles_n)) / gsize) * GBN;
    return true;
}

// Epilogue of the 128 x 128 kernels: lane holds C[m = lane%16][n = 4*(lane/16) + q]
// of each 16 x 16 fragment; rounded to the storage type, masked at the edges.
template <class T>
__device__ __forceinline__ void store_c(const GemmArgs& a, int64_t b, int64_t m0, int64_t n0,
                                        int wm, int wn, int lane, const f32x4 (&acc)[4][4]) {
    uint16_t* C = reinterpret_cast<uint16_t*>(a.C) + b * a.sc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t gm = m0 + wm * 64 + i * 16 + (lane & 15);
        if (gm >= a.m) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t gn = n0 + wn * 64 + j * 16 + 4 * (lane >> 4);
            uint16_t* dst = C + gm * a.ldc + gn;
            if (a.beta == 0.f && gn + 4 <= a.n && (a.ldc & 3) == 0 &&
                (reinterpret_cast<uintptr_t>(dst) & 7) == 0) {
                u32x2 v;
                v[0] = (uint32_t)narrow(T{}, a.alpha * acc[i][j][0]) | ((uint32_t)narrow(T{}, a.alpha * acc[i][j][1]) << 16);
                v[1] = (uint32_t)narrow(T{}, a.alpha * acc[i][j][2]) | ((uint32_t)narrow(T{}, a.alpha * acc[i][j][3]) << 16);
                *reinterpret_cast<u32x2*>(dst) = v;
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (gn + q < a.n) dst[q] = axpby<T>(acc[i][j][q], a.alpha, a.beta, dst + q);
            }
        }
    }
}

// Epilogue through LDS for interior tiles (the whole 128 x 128 tile inside C,
// ldc % 8 == 0, 16-byte aligned C, beta == 0): each wave's 64 x 64 piece goes to LDS in
// two halves of 32 rows (row pitch 72 elements, so the 16 rows one write
// instruction covers land in distinct banks) and leaves as 16-byte row
// pieces, eight rows x 128 bytes per store instruction, instead of the
// 16 rows x 32 bytes of the register layout. `stage` is block LDS of at least
// 4 x 32 x 72 elements that no wave still reads; ends with a barrier.
template <class T>
__device__ __forceinline__ bool store_c_staged(const GemmArgs& a, int64_t b, int64_t m0, int64_t n0,
                                               int wm, int wn, int lane, int wave,
                                               const f32x4 (&acc)[4][4], uint16_t* stage) {
    uint16_t* Cb = reinterpret_cast<uint16_t*>(a.C) + b * a.sc;
    const bool fits = a.beta == 0.f && m0 + GBM <= a.m && n0 + GBN <= a.n && (a.ldc & 7) == 0 &&
                      (reinterpret_cast<uintptr_t>(Cb) & 15) == 0;
    if (!fits) return false;  // block-uniform
    uint16_t* stg = stage + wave * (32 * 72);
    uint16_t* C = Cb + (m0 + wm * 64) * a.ldc + n0 + wn * 64;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4& v4 = acc[2 * h + ii][j];
                u32x2 v;
                v[0] = (uint32_t)narrow(T{}, a.alpha * v4[0]) | ((uint32_t)narrow(T{}, a.alpha * v4[1]) << 16);
                v[1] = (uint32_t)narrow(T{}, a.alpha * v4[2]) | ((uint32_t)narrow(T{}, a.alpha * v4[3]) << 16);
                *reinterpret_cast<u32x2*>(stg + (ii * 16 + (lane & 15)) * 72 + j * 16 + 4 * (lane >> 4)) = v;
            }
        }
        // LDS instructions of one wave complete in order: the reads below see
        // the writes above, and the next half's writes follow these reads.
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int r = p * 8 + (lane >> 3), c = (lane & 7) * 8;
            const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * 72 + c);
            *reinterpret_cast<u32x4*>(C + (int64_t)(h * 32 + r) * a.ldc + c) = v;
        }
    }
    __syncthreads();  // the stage is free for the next item's tiles
    return true;
}

// Block = 4 waves (2 x 2), tile 128 x 128 x 32, each wave 64 x 64 with
// v_mfma_f32_16x16x32. Double-buffered LDS: k-tile kt+1 is fetched into
// registers before tile kt is multiplied and stored to the other LDS buffer
// after it, so one barrier per k-tile separates the writes from the reads.
template <class T, bool TA, bool TB, bool VEC>
__global__ __launch_bounds__(GThreads) void gemm_mfma_generic(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][GBM * GLDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][GBN * GLDK];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t nk = (a.k + GBK - 1) / GBK;
    TileItem it;
    for (int64_t slot = blockIdx.x / 8; tile_item(a, slot, &it); slot += gridDim.x / 8) {
        const int64_t b = it.b, m0 = it.m0, n0 = it.n0;
        const uint16_t* A = reinterpret_cast<const uint16_t*>(a.A) + b * a.sa;
        const uint16_t* B = reinterpret_cast<const uint16_t*>(a.B) + b * a.sb;
        f32x4 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        u32x4 va[GCH], vb[GCH];
        int na[GCH], nb[GCH];
        fetch_tile<!TA, VEC>(A, a.lda, a.m, a.k, m0, 0, va, na);
        fetch_tile<TB, VEC>(B, a.ldb, a.n, a.k, n0, 0, vb, nb);
        __syncthreads();  // the previous item's readers are done with buffer 0
        store_tile<!TA>(va, na, As[0]);
        store_tile<TB>(vb, nb, Bs[0]);
        __syncthreads();
        for (int64_t kt = 0; kt < nk; ++kt) {
            const int cur = (int)(kt & 1);
            const bool more = kt + 1 < nk;
            if (more) {
                fetch_tile<!TA, VEC>(A, a.lda, a.m, a.k, m0, (kt + 1) * GBK, va, na);
                fetch_tile<TB, VEC>(B, a.ldb, a.n, a.k, n0, (kt + 1) * GBK, vb, nb);
            }
            u32x4 af[4], bf[4];
            const int kofs = (lane >> 4) * 8;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const u32x4*>(&As[cur][(wm * 64 + i * 16 + (lane & 15)) * GLDK + kofs]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = *reinterpret_cast<const u32x4*>(&Bs[cur][(wn * 64 + j * 16 + (lane & 15)) * GLDK + kofs]);
            // D[n][m] = sum_k B(n,k) A(m,k): lane holds C[m = lane%16][n = 4*(lane/16) + q].
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma16<T>(bf[j], af[i], acc[i][j]);
            if (more) {
                store_tile<!TA>(va, na, As[cur ^ 1]);
                store_tile<TB>(vb, nb, Bs[cur ^ 1]);
            }
            __syncthreads();
        }

        if (!store_c_staged<T>(a, b, m0, n0, wm, wn, lane, wave, acc, &As[0][0]))
            store_c<T>(a, b, m0, n0, wm, wn, lane, acc);
    }
}

// Short-K form (k <= 128): every k-tile is fetched up front, so the global
// latency is paid once, the whole K slab is stored to LDS, and one barrier
// precedes the (up to) 4 x 16 MFMAs per wave. For shallow products (a batch
// of small GEMMs) the per-k-tile round trips of the loop above dominate.
constexpr int GSK = 4;  // k-tiles held

template <class T, bool TA, bool TB, bool VEC>
__global__ __launch_bounds__(GThreads) void gemm_mfma_shortk(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t As[GSK][GBM * GLDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[GSK][GBN * GLDK];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int nk = (int)((a.k + GBK - 1) / GBK);  // 1 .. GSK
    TileItem it;
    for (int64_t slot = blockIdx.x / 8; tile_item(a, slot, &it); slot += gridDim.x / 8) {
        const int64_t b = it.b, m0 = it.m0, n0 = it.n0;
        const uint16_t* A = reinterpret_cast<const uint16_t*>(a.A) + b * a.sa;
        const uint16_t* B = reinterpret_cast<const uint16_t*>(a.B) + b * a.sb;
        // All GSK k-tiles are fetched and stored (those past k come out zero),
        // so no load sits under a branch.
        u32x4 va[GSK][GCH], vb[GSK][GCH];
        int na[GSK][GCH], nb[GSK][GCH];
#pragma unroll
        for (int t = 0; t < GSK; ++t) {
            fetch_tile<!TA, VEC>(A, a.lda, a.m, a.k, m0, t * GBK, va[t], na[t]);
            fetch_tile<TB, VEC>(B, a.ldb, a.n, a.k, n0, t * GBK, vb[t], nb[t]);
        }
        __syncthreads();  // the previous item's readers are done
#pragma unroll
        for (int t = 0; t < GSK; ++t) {
            store_tile<!TA>(va[t], na[t], As[t]);
            store_tile<TB>(vb[t], nb[t], Bs[t]);
        }
        __syncthreads();
        f32x4 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int kofs = (lane >> 4) * 8;
#pragma unroll
        for (int t = 0; t < GSK; ++t) {
            if (t < nk) {
                u32x4 af[4], bf[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    af[i] = *reinterpret_cast<const u32x4*>(&As[t][(wm * 64 + i * 16 + (lane & 15)) * GLDK + kofs]);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    bf[j] = *reinterpret_cast<const u32x4*>(&Bs[t][(wn * 64 + j * 16 + (lane & 15)) * GLDK + kofs]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = mfma16<T>(bf[j], af[i], acc[i][j]);
            }
        }
        __syncthreads();  // every wave is done reading As before it holds the epilogue stage
        if (!store_c_staged<T>(a, b, m0, n0, wm, wn, lane, wave, acc, &As[0][0]))
            store_c<T>(a, b, m0, n0, wm, wn, lane, acc);
    }
}

// ---------------------------------------------------------------------------
// Pipelined f16 / bf16 kernel: C = A . B^T with A [m,k] and B [n,k] both
// K-contiguous, k % 128 == 0, k >= 256, 16-byte aligned, m and n multiples of
// the tile edge 32 TF (TF = 8: 256; TF = 4: 128).
//
// Block = 4 waves, each 16 TF x 16 TF as TF x TF fragments of 16 x 16
// (v_mfma_f32_16x16x32). TF = 8 is the large-product form: one block per CU,
// one wave per SIMD with 64 accumulators of 4 f32 in AGPRs; a 128 x 128 wave
// tile halves the LDS fragment reads per MFMA compared with 128 x 64. TF = 4
// gives four times the tiles for products too small to fill the GPU with
// 256 x 256 ones, at two blocks per CU. The description below is for TF = 8;
// TF = 4 halves every tile dimension, the DMA instructions per wave and the
// MFMAs per group.
//
// Operands go from global memory straight into LDS (buffer_load ... lds, no
// VGPR staging) in k-tiles of 32: four LDS stages of 32 KiB (A 16 KiB, B 16 KiB).
// One DMA instruction fills 1 KiB = 16 tile rows x 64 bytes; lane i fetches
// the global chunk that belongs at LDS slot i, so the XOR swizzle (chunk c of
// row r at slot c ^ ((r >> 2) & 3)) costs nothing on the write side and the
// fragment reads of 16 consecutive rows hit distinct banks.
//
// Per k-tile kt (stage kt % 4), each wave runs two groups of 32 MFMAs: A rows
// 0-63 of its wave tile, then rows 64-127, each against all eight B
// fragments. The second half's A fragments are read while the first group
// runs. Between the two groups sits the only barrier of the k-tile: after it
// tile kt+1 is resident and stage kt % 4 is free, so the next tile's first A
// half and its B fragments (into the other B register set) are read, and
// the DMA of tile kt+4 into the freed stage starts. Its eight instructions
// are spread one per eight MFMAs over the next two groups (a burst would
// fill the address queue and stall MFMA issue behind it); tile kt+4 is
// needed three barriers later. Loops are unrolled by the stage count so every
// LDS offset, stage and wait count is a compile-time constant. In same-run
// comparisons the 16x16x32 form beat the 32x32x16 form of the same pipeline
// by about 4% on 8192^3.
//
// Tile order: groups of 4 tile-rows, column-major inside a group, each XCD
// (blockIdx % 8) taking a contiguous run, so resident blocks on one XCD share
// A and B panels in its L2.
// ---------------------------------------------------------------------------
constexpr int LBK = 32, LSTAGES = 4;
constexpr int LThreads = 256;
constexpr int LCPR = LBK / 8;                  // 16-byte chunks per tile row
constexpr int LRPI = 64 / LCPR;                // tile rows per 1 KiB DMA instruction
constexpr int LGM = 4;                         // tile-rows per group
// Shape of the kernel with TF x TF fragments per wave: 16 TF x 16 TF wave
// tiles, 32 TF x 32 TF block tiles (256 for TF = 8, 128 for TF = 4).
template <int TF>
struct LTile {
    static constexpr int BM = 32 * TF;              // block tile edge
    static constexpr int STAGE_H = 2 * BM * LBK;    // halves per stage (A then B)
    static constexpr int IPW = BM / 4 / LRPI;       // DMA instructions per wave per operand per tile
    static constexpr int LPS = 2 * IPW;             // DMA instructions per wave per tile
    static constexpr size_t LDS = (size_t)LSTAGES * STAGE_H * sizeof(uint16_t);
};

template <int... I, class F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, I...>, F&& f) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int V> using ic = std::integral_constant<int, V>;
template <bool V> using bc = std::integral_constant<bool, V>;

// s_waitcnt immediate: vmcnt <= n, lgkmcnt <= 0, expcnt untouched.
constexpr int wait_vm_lgkm0(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4); }

__device__ __forceinline__ int lswz(int r) { return (r >> 2) & 3; }

#define MM_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// ---------------------------------------------------------------------------
// Batched short-K NT kernel: C[b] = A[b] . B[b]^T with A [m,k] and B [n,k]
// both K-contiguous, k in {32, 64, 128}, m % 64 == 0, n % 128 == 0, 16-byte
// aligned operands and C, beta == 0.
//
// With k this short the product is bound by memory (the batched 32 x 512 x
// 512 x 128 workload does 85 FLOP per byte, below the MFMA ridge), and the
// 128 x 128 kernels run fetch, MFMA and stores in lockstep across the whole
// grid. Here a block owns one panel of PMT = 64 or 128 rows of A (loaded into
// LDS once; each wave then keeps its A fragments in registers for the whole
// block) and walks the batch's B in tiles of PN rows through LA + 1 LDS
// stages: B tiles t+1 .. t+LA are in flight by DMA (buffer_load ... lds,
// 1 KiB per instruction) while tile t is multiplied and its PMT x PN output
// leaves through a per-wave LDS stage as 16-byte row pieces, so the output
// stores of one tile overlap the fetch of the next ones. Those stores carry
// the device-scope write-through policy (sc0 sc1 nt): the output then
// streams to HBM while the blocks run, instead of staying dirty in the L2s
// until the write-back at the end of the kernel. The 64-row form at k = 128
// keeps plain stores: measured on MI355X, write-through was faster for the
// 128-row form and for the 64-row form at k = 32 and 64, slower there. The
// block has
// PMT / 16 waves, each computing 32 x PN / 2 (2 x PN / 32 fragments of
// v_mfma_f32_16x16x32); a 128-row panel streams each B tile once for twice
// the rows of a 64-row one, halving B's reads from L2. Rows of S = k / 8 16-byte chunks
// are stored with chunk c of row r at slot c ^ ((r / (16 / S)) & (S - 1)), so
// the fragment reads of 16 consecutive rows at one chunk index hit 16
// distinct 16-byte bank groups; each DMA lane fetches the chunk that belongs
// at its slot. Blocks are ordered so that the panels of one batch item run
// on one XCD and share its B in L2.
// ---------------------------------------------------------------------------
// B stages: three for 64-row panels (two blocks per CU), four for 128-row
// ones (one block per CU; a block's four B tiles of the batched workload are
// then all in flight from its start).
__host__ __device__ constexpr int panel_stages(int PMT) { return PMT == 128 ? 4 : 3; }
// Cache-policy bits of a buffer store: sc0 (1) | nt (2) | sc1 (16).
constexpr int kStoreThrough = 1 | 2 | 16;

template <int S>
__device__ __forceinline__ int pswz(int r) {
    return (r / (16 / S)) & (S - 1);
}

// Epilogue staging row pitch (halves) for a wave tile PN / 2 wide: 8 halves
// of padding put the 16 rows one staging write covers in distinct banks.
__host__ __device__ constexpr int panel_pitch(int PN) { return PN / 2 + 8; }

// LDS of one block: A panel of PMT rows, panel_stages(PMT) B stages of PN rows, one
// 32-row epilogue stage per wave (PMT / 16 waves).
__host__ __device__ constexpr size_t panel_lds_bytes(int S, int PN, int PMT) {
    return ((size_t)(PMT + panel_stages(PMT) * PN) * S * 8 + (PMT / 16) * 32 * panel_pitch(PN)) *
           sizeof(uint16_t);
}

// Block = one (batch item, PMT-row panel of A, group of B tiles); `nsplit`
// groups split the batch item's n / PN tiles (more blocks when there are few
// panels), and the groups of one panel follow each other in the block order.
template <class T, int S, int PN, int PMT>
__global__ __launch_bounds__(PMT * 4, 1) void gemm_nt_panel(GemmArgs a, int nsplit) {
    constexpr int K = S * 8;          // contraction length
    constexpr int NW = PMT / 16;      // waves: PMT / 32 row slabs x 2 column halves
    constexpr int RPI = 64 / S;       // tile rows per 1 KiB DMA instruction
    constexpr int NA = PMT / RPI / NW;  // A instructions per wave (= S / 4)
    constexpr int NB = PN / RPI / NW;   // B instructions per wave per tile
    static_assert(NA * RPI * NW == PMT && NB * RPI * NW == PN, "whole DMA instructions per wave");
    constexpr int NV = S / 4;         // lane offset patterns (the swizzle repeats every 16 rows)
    constexpr int WN = PN / 2;        // wave tile: 32 rows x WN columns
    constexpr int FN = WN / 16;       // 16-column fragments per wave
    constexpr int NST = PN / 32;      // store instructions per wave per tile (1 KiB each)
    constexpr int SRW = 1024 / PN;    // rows per store instruction
    constexpr int SLN = PN / 16;      // lanes per stored row (16 bytes each)
    constexpr int AH = PMT * K, BH = PN * K;  // halves per A panel / B stage
    constexpr int PSP = panel_pitch(PN);
    constexpr int PS = panel_stages(PMT), LA = PS - 1;  // B stages, tiles fetched ahead
    constexpr int CPOL = PMT == 64 && S == 16 ? 0 : kStoreThrough;  // output store policy
    extern __shared__ __attribute__((aligned(1024))) uint16_t lds[];
    uint16_t* const As = lds;
    uint16_t* const Bs = lds + AH;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = w >> 1, wn = w & 1;
    uint16_t* const stg = lds + AH + PS * BH + w * 32 * PSP;

    const int64_t panels = a.m / PMT;
    const int64_t items = panels * a.batch * nsplit;
    const int64_t per_xcd = (items + 7) / 8;
    const int64_t item = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (item >= items) return;
    const int64_t pi = item / nsplit;
    const int h = (int)(item % nsplit);
    const int64_t b = pi / panels, m0 = (pi % panels) * PMT;
    const int all_tiles = (int)(a.n / PN);
    const int t_begin = (int)((int64_t)all_tiles * h / nsplit);
    const int ntiles = (int)((int64_t)all_tiles * (h + 1) / nsplit) - t_begin;
    const int lda = (int)a.lda, ldb = (int)a.ldb;

    const uint16_t* Ab = reinterpret_cast<const uint16_t*>(a.A) + b * a.sa;
    const uint16_t* Bb = reinterpret_cast<const uint16_t*>(a.B) + b * a.sb;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(Ab), (short)0, (int)(((a.m - 1) * a.lda + K) * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(Bb), (short)0, (int)(((a.n - 1) * a.ldb + K) * 2), 0x00020000);
    // DMA lane offsets (bytes): the lane covers row lane / S of an
    // instruction and fetches the chunk that the swizzle puts at slot
    // lane % S. The swizzle depends on the row modulo 16, so instruction j
    // of a tile (rows j * RPI ..) uses pattern j % NV (NV <= 4); named
    // scalars, one per pattern. (A wave's first B instruction need not start
    // at a multiple of 16 rows: with eight waves it starts at row 8 * w.)
    const int lrow = lane / S, lslot = lane % S;
    const int c0 = lslot ^ pswz<S>(lrow), c1 = lslot ^ pswz<S>(RPI + lrow);
    const int c2 = lslot ^ pswz<S>(2 * RPI + lrow), c3 = lslot ^ pswz<S>(3 * RPI + lrow);
    const int voa0 = (lrow * lda + c0 * 8) * 2, voa1 = (lrow * lda + c1 * 8) * 2;
    const int voa2 = (lrow * lda + c2 * 8) * 2, voa3 = (lrow * lda + c3 * 8) * 2;
    const int vob0 = (lrow * ldb + c0 * 8) * 2, vob1 = (lrow * ldb + c1 * 8) * 2;
    const int vob2 = (lrow * ldb + c2 * 8) * 2, vob3 = (lrow * ldb + c3 * 8) * 2;
    auto dma_a = [&]() {
#pragma unroll
        for (int jj = 0; jj < NA; ++jj) {
            const int j = w * NA + jj, pat = j % NV;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, MM_LDS(As + j * RPI * K), 16,
                                                     pat == 0 ? voa0 : pat == 1 ? voa1 : pat == 2 ? voa2 : voa3,
                                                     (int)((m0 + j * RPI) * lda * 2), 0, 0);
        }
    };
    auto dma_b = [&](int t, int st) {  // t: tile index within the batch item
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) {
            const int j = w * NB + jj, pat = j % NV;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, MM_LDS(Bs + st * BH + j * RPI * K), 16,
                                                     pat == 0 ? vob0 : pat == 1 ? vob1 : pat == 2 ? vob2 : vob3,
                                                     (t * PN + j * RPI) * ldb * 2, 0, 0);
        }
    };
    // Fragment reads: lane -> row lane % 16 of a 16-row slab, chunk 4 * ks + lane / 16.
    const int lr = lane & 15, lq = lane >> 4;
    auto frag = [&](const uint16_t* base, int row0, int ks) {
        return *reinterpret_cast<const u32x4*>(base + (row0 + lr) * K +
                                               (((4 * ks + lq) ^ pswz<S>(lr)) << 3));
    };
    // vmcnt <= NB * nb + NST * ns (lgkmcnt <= 0): at most nb < LA B tiles'
    // DMA and 1 <= ns <= LA tiles' stores younger than the awaited tile.
    auto wait_vm = [](int nb, int ns) {
        static_for(std::make_integer_sequence<int, LA>{}, [&](auto NB_) {
            static_for(std::make_integer_sequence<int, LA>{}, [&](auto NS_) {
                constexpr int cnt = NB * decltype(NB_)::value + NST * (decltype(NS_)::value + 1);
                static_assert(cnt <= 63, "vmcnt range");
                if (nb == decltype(NB_)::value && ns == decltype(NS_)::value + 1)
                    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(cnt));
            });
        });
    };

    // Prologue: the A panel and the first LA B tiles; wait for A and tile 0.
    dma_a();
    const int pre = ntiles < LA ? ntiles : LA;
    dma_b(t_begin, 0);
    if (pre > 1) dma_b(t_begin + 1, 1);
    if (LA > 2 && pre > 2) dma_b(t_begin + 2, 2);
    static_assert(LA <= 3, "prologue issues at most three tiles");
    if (pre == 3) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(2 * NB));
    else if (pre == 2) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(NB));
    else __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
    __builtin_amdgcn_s_barrier();

    // The wave's A fragments do not change from tile to tile: read them from
    // LDS once (2 x K / 32 fragments, at most 32 registers) and keep them.
    u32x4 fa[K / 32][2];
#pragma unroll
    for (int ks = 0; ks < K / 32; ++ks)
#pragma unroll
        for (int i = 0; i < 2; ++i) fa[ks][i] = frag(As, wm * 32 + i * 16, ks);

    // C of this batch item spans below 2 GiB (checked by the launcher).
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<uint16_t*>(a.C) + b * a.sc, (short)0, (int)(((a.m - 1) * a.ldc + a.n) * 2), 0x00020000);
    const int cbase = (int)(((m0 + wm * 32) * a.ldc + wn * WN) * 2);
    for (int t = 0; t < ntiles; ++t) {
        const int st = t % PS;
        // Stage (t + LA) % PS held tile t - 1, which every wave finished before the barrier.
        if (t + LA < ntiles) dma_b(t_begin + t + LA, (t + LA) % PS);
        const uint16_t* Bt = Bs + st * BH;
        f32x4 acc[2][FN];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < K / 32; ++ks) {
            u32x4 fb[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) fb[j] = frag(Bt, wn * WN + j * 16, ks);
            // D[n][m] = sum_k B(n,k) A(m,k): lane holds C[m = lane%16][n = 4*(lane/16) + q].
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma16<T>(fb[j], fa[ks][i], acc[i][j]);
        }
        // Epilogue: the wave's 32 x WN piece through its LDS stage (LDS
        // instructions of one wave complete in order), then 16-byte row
        // pieces, 1 KiB per store instruction (written through but in the
        // 64-row form at k = 128).
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const f32x4& v4 = acc[i][j];
                u32x2 v;
                v[0] = (uint32_t)narrow(T{}, a.alpha * v4[0]) | ((uint32_t)narrow(T{}, a.alpha * v4[1]) << 16);
                v[1] = (uint32_t)narrow(T{}, a.alpha * v4[2]) | ((uint32_t)narrow(T{}, a.alpha * v4[3]) << 16);
                *reinterpret_cast<u32x2*>(stg + (i * 16 + lr) * PSP + j * 16 + 4 * lq) = v;
            }
        const int64_t col0 = (int64_t)(t_begin + t) * PN;
#pragma unroll
        for (int p = 0; p < NST; ++p) {
            const int r = p * SRW + lane / SLN, c = (lane % SLN) * 8;
            const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * PSP + c);
            __builtin_amdgcn_raw_buffer_store_b128(v, rc, cbase + (int)((r * a.ldc + col0 + c) * 2), 0,
                                                   CPOL);
        }
        if (t + 1 < ntiles) {
            // Tile t + 1 has landed once at most these remain: the DMA of
            // tiles t + 2 .. t + LA (those issued) and the stores of the
            // iterations since tile t + 1's DMA was issued.
            const int last = t + LA < ntiles - 1 ? t + LA : ntiles - 1;
            const int since = t + 1 - LA > 0 ? t + 1 - LA : 0;
            wait_vm(last - (t + 1), t - since + 1);
            __builtin_amdgcn_s_barrier();
        }
    }
}

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group,
// output lane j receives element j % 4 of the four 16-bit elements at the
// addresses of lanes j / 4, j / 4 + 4, j / 4 + 8 and j / 4 + 12 of the group.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(const_cast<void*>(p)));
    return __builtin_bit_cast(u32x2, v);
}

// Chunk swizzle of a k-major stage row r (K-strided operands): the 16 rows
// that one transposing read touches spread over 8 distinct 32-byte bank
// segments.
__device__ __forceinline__ int kswz(int r) { return 2 * ((r & 3) + 4 * ((r >> 3) & 1)); }

// LDS stage S of K-strided operand OP (N halves): each stage its own array,
// so that the compiler can tell the transposing reads of one stage apart from
// DMA into the others (with one array for all stages it waits for every DMA
// in flight before each such read).
template <int N, int S, int OP>
__device__ __forceinline__ uint16_t* kmajor_stage() {
    __shared__ __attribute__((aligned(1024))) uint16_t st[N];
    return st;
}

// Dynamic LDS of the pipelined kernel: both operands' stages when both are
// K-contiguous, else only the K-contiguous operand's (K-strided ones use
// kmajor_stage).
template <int TF>
constexpr size_t pipelined_lds_bytes(bool ka, bool kb) {
    return ka && kb ? LTile<TF>::LDS
                    : (ka || kb ? (size_t)LSTAGES * LTile<TF>::BM * LBK * sizeof(uint16_t) : 0);
}

// Tile of this block in the pipelined kernels' order: groups of LGM
// tile-rows, column-major inside a group, each XCD (blockIdx % 8) taking a
// contiguous run so that its resident blocks share A and B panels in its L2.
// False when the block has no tile.
template <int BM, bool RAG>
__device__ __forceinline__ bool pipelined_tile(const GemmArgs& a, int64_t& m0, int64_t& n0) {
    const int64_t tiles_m = RAG ? (a.m + BM - 1) / BM : a.m / BM;
    const int64_t tiles_n = RAG ? (a.n + BM - 1) / BM : a.n / BM;
    const int64_t ntiles = tiles_m * tiles_n;
    const int64_t bid = blockIdx.x;
    const int64_t per_xcd = (ntiles + 7) / 8;
    const int64_t t = (bid % 8) * per_xcd + bid / 8;
    if (t >= ntiles) return false;
    const int64_t group = t / (LGM * tiles_n);
    const int64_t first_m = group * LGM;
    const int64_t gsize = tiles_m - first_m < LGM ? tiles_m - first_m : LGM;
    m0 = (first_m + (t % (LGM * tiles_n)) % gsize) * BM;
    n0 = ((t % (LGM * tiles_n)) / gsize) * BM;
    return true;
}

// Buffer resource over one operand's tile of batch item b: BM rows from row0
// (K-contiguous: rows of k elements ld apart) or BM columns from column col0
// of k rows ld apart (K-strided). With RAG the range stops at the operand's
// true extent (`rows` of the BM inside it), so reads past it return zeros.
template <int BM, bool KC, bool RAG>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pipelined_rsrc(const void* base, int64_t batch_off,
                                                                 int64_t first, int64_t ld, int64_t k,
                                                                 int64_t rows) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + batch_off + (KC ? first * ld : first);
    const int bytes = RAG ? (int)((KC ? (rows - 1) * ld + k : (k - 1) * ld + rows) * 2)
                          : (KC ? BM * (int)ld * 2 : (int)(((k - 1) * ld + BM) * 2));
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), (short)0, bytes, 0x00020000);
}

// Epilogue of the pipelined kernels: the wave's TF x TF fragments (lane holds
// C[m = 16i-slab base + lane%16][n = 16j-slab base + 4 (lane/16) + q]) into C
// of batch item b as alpha * acc + beta * C_old; four-element stores when
// beta == 0 and the piece lies inside C, element stores otherwise.
template <class T, int TF, bool RAG>
__device__ __forceinline__ void pipelined_store(const GemmArgs& a, int64_t b, int64_t m0, int64_t n0,
                                                int wm, int wn, int lr, int lq, const f32x4 (&acc)[TF][TF]) {
    constexpr int WT = 16 * TF;
    uint16_t* C = reinterpret_cast<uint16_t*>(a.C) + b * a.sc;
#pragma unroll
    for (int i = 0; i < TF; ++i) {
        const int64_t gm = m0 + wm * WT + i * 16 + lr;
        if (RAG && gm >= a.m) continue;
#pragma unroll
        for (int j = 0; j < TF; ++j) {
            const int64_t gn = n0 + wn * WT + j * 16 + lq * 4;
            uint16_t* dst = C + gm * a.ldc + gn;
            if (RAG && gn + 4 > a.n) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (gn + q < a.n) dst[q] = axpby<T>(acc[i][j][q], a.alpha, a.beta, dst + q);
            } else if (a.beta == 0.f) {
                u32x2 v;
                v[0] = (uint32_t)narrow(T{}, a.alpha * acc[i][j][0]) |
                       ((uint32_t)narrow(T{}, a.alpha * acc[i][j][1]) << 16);
                v[1] = (uint32_t)narrow(T{}, a.alpha * acc[i][j][2]) |
                       ((uint32_t)narrow(T{}, a.alpha * acc[i][j][3]) << 16);
                *reinterpret_cast<u32x2*>(dst) = v;
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) dst[q] = axpby<T>(acc[i][j][q], a.alpha, a.beta, dst + q);
            }
        }
    }
}

// RAG: m or n not a multiple of the tile edge. Edge tiles then read through
// buffer resources cut at the operand's true extent (rows or columns past it
// read zeros, and any other data in padding columns only feeds outputs that
// are never stored), and the epilogue stores only inside C.
template <class T, int TF, bool KA = true, bool KB = true, bool RAG = false>
__global__ __launch_bounds__(LThreads, TF == 8 ? 1 : 2) void gemm_mfma_large(GemmArgs a) {
    using L = LTile<TF>;
    constexpr int BM = L::BM, SH = L::STAGE_H, IPW = L::IPW, LLPS = L::LPS;
    constexpr int HF = TF / 2;        // A fragments per half of the wave tile
    constexpr int WT = 16 * TF;       // wave tile edge
    constexpr int RPW = BM / 4;       // tile rows each wave moves per operand and k-tile
    constexpr int NR = IPW;           // DMA instructions per half k-tile = MFMA runs per group
    constexpr int MPR = HF * TF / NR; // MFMAs per run
    extern __shared__ __attribute__((aligned(1024))) uint16_t lds[];  // [stage][A | B][row][32]
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = w >> 1, wn = w & 1;
    int64_t m0, n0;
    if (!pipelined_tile<BM, RAG>(a, m0, n0)) return;
    const int nk = (int)(a.k / LBK);  // a multiple of LSTAGES, at least 2 * LSTAGES
    const int lda = (int)a.lda, ldb = (int)a.ldb;

    // DMA lane mapping, K-contiguous operand (A [m,k], B [n,k]): instruction
    // j of a wave covers tile rows w*RPW + j*16 + lane/4; lane writes LDS slot
    // lane%4 of its row with the chunk that the swizzle puts there. The row's
    // swizzle does not depend on j.
    const int chunk = (lane % LCPR) ^ lswz(lane / LCPR);
    const int voa = ((w * RPW + lane / LCPR) * lda + chunk * 8) * 2;
    const int vob = ((w * RPW + lane / LCPR) * ldb + chunk * 8) * 2;
    // K-strided operand (A [k,m], B [k,n]): the stage holds the k-tile as 32
    // rows of BM elements (row = k), chunk c of row r at slot c ^ kswz(r).
    // Instruction j of a wave covers rows (w*IPW + j)*RPK + lane/CPK; the
    // lane's slot is lane % CPK. The swizzle depends on j only through j % 2.
    constexpr int CPK = BM / 8;   // 16-byte chunks per k-row
    constexpr int RPK = 64 / CPK; // k-rows per DMA instruction
    const int kr0 = (w * IPW) * RPK + lane / CPK, kr1 = kr0 + RPK, kslot = lane % CPK;
    const int voka0 = ((lane / CPK) * lda + 8 * (kslot ^ kswz(kr0))) * 2;
    const int voka1 = ((lane / CPK) * lda + 8 * (kslot ^ kswz(kr1))) * 2;
    const int vokb0 = ((lane / CPK) * ldb + 8 * (kslot ^ kswz(kr0))) * 2;
    const int vokb1 = ((lane / CPK) * ldb + 8 * (kslot ^ kswz(kr1))) * 2;
    // Fragment reads, K-contiguous: lane -> row lane%16 of a 16-row slab, chunk lane/16.
    const int lr = lane & 15, lq = lane >> 4;
    const int foff = lr * LBK + ((lq ^ lswz(lr)) << 3);
    // Fragment reads, K-strided: two transposing reads per fragment (k 0-3
    // and 4-7 of the lane's eight). Lane s of 16-lane group g addresses row
    // 8g + 4h + s/4 (h = read), columns 4 (s % 4) .. + 3 of the fragment;
    // the byte offset of fragment f is the wave's base XOR 32 f.
    const int kg = lane >> 4, ks = lane & 15, kx = (ks & 3) >> 1;
    const int kr_0 = 8 * kg + (ks >> 2), kr_1 = kr_0 + 4;
    const int kb0 = kr_0 * 2 * BM + 8 * (ks & 1) + 16 * (kx ^ kswz(kr_0));
    const int kb1 = kr_1 * 2 * BM + 8 * (ks & 1) + 16 * (kx ^ kswz(kr_1));
    const int kA0 = kb0 ^ (32 * TF * wm), kA1 = kb1 ^ (32 * TF * wm);
    const int kB0 = kb0 ^ (32 * TF * wn), kB1 = kb1 ^ (32 * TF * wn);
    constexpr int DSA = KA ? 1 : 2, DSB = KB ? 1 : 2;  // LDS reads per fragment
    // Stage bases by compile-time stage index: a K-contiguous operand in the
    // dynamic array ([stage][A | B] when both are, else [stage][that one]),
    // a K-strided one in its own per-stage arrays.
    constexpr int DSTR = KA && KB ? SH : BM * LBK;
    // (A K-contiguous operand's stage may also be named by a run-time int.)
    auto stage_a = [&](auto S_) -> uint16_t* {
        if constexpr (KA) return lds + (int)S_ * DSTR;
        else return kmajor_stage<BM * LBK, decltype(S_)::value, 0>();
    };
    auto stage_b = [&](auto S_) -> uint16_t* {
        if constexpr (KB) return lds + (int)S_ * DSTR + (KA ? BM * LBK : 0);
        else return kmajor_stage<BM * LBK, decltype(S_)::value, 1>();
    };

    for (int64_t b = blockIdx.y; b < a.batch; b += gridDim.y) {
        // Rows (K-contiguous) or columns (K-strided) of this tile inside the operand.
        const int64_t mrows = RAG && a.m - m0 < BM ? a.m - m0 : BM;
        const int64_t nrows = RAG && a.n - n0 < BM ? a.n - n0 : BM;
        const __amdgpu_buffer_rsrc_t ra = pipelined_rsrc<BM, KA, RAG>(a.A, b * a.sa, m0, a.lda, a.k, mrows);
        const __amdgpu_buffer_rsrc_t rb = pipelined_rsrc<BM, KB, RAG>(a.B, b * a.sb, n0, a.ldb, a.k, nrows);

        // Half p (instructions IPW/2 * p .. of each operand) of k-tile kt into a stage.
        auto dma_half = [&](auto S_, int kt, int p) {
            uint16_t *sa, *sb;
            if constexpr (KA && KB) {
                const int stage = S_;
                sa = lds + stage * SH + w * RPW * LBK;
                sb = sa + BM * LBK;
            } else {
                sa = stage_a(S_) + w * RPW * LBK;
                sb = stage_b(S_) + w * RPW * LBK;
            }
            uint16_t* ska = stage_a(S_);   // k-major: row r at r * BM
            uint16_t* skb = stage_b(S_);
#pragma unroll
            for (int jj = 0; jj < IPW / 2; ++jj) {
                const int j = IPW / 2 * p + jj;
                const int kr = (w * IPW + j) * RPK;  // first k-row of a k-major instruction
                if constexpr (KA)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, MM_LDS(sa + j * LRPI * LBK), 16, voa,
                                                             (j * LRPI * lda + kt * LBK) * 2, 0, 0);
                else
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, MM_LDS(ska + kr * BM), 16,
                                                             j % 2 ? voka1 : voka0,
                                                             (kt * LBK + kr) * lda * 2, 0, 0);
                if constexpr (KB)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, MM_LDS(sb + j * LRPI * LBK), 16, vob,
                                                             (j * LRPI * ldb + kt * LBK) * 2, 0, 0);
                else
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, MM_LDS(skb + kr * BM), 16,
                                                             j % 2 ? vokb1 : vokb0,
                                                             (kt * LBK + kr) * ldb * 2, 0, 0);
            }
        };
        f32x4 acc[TF][TF];
#pragma unroll
        for (int i = 0; i < TF; ++i)
#pragma unroll
            for (int j = 0; j < TF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        // A fragments of half hh (wave rows hh*WT/2 + 16i) / all TF B fragments of a stage.
        auto rda = [&](auto S_, int hh, u32x4 (&fa)[HF]) {
            if constexpr (KA && KB) {
                const int stage = S_;
                const uint16_t* sa = lds + stage * SH + (wm * WT + hh * (WT / 2)) * LBK;
#pragma unroll
                for (int i = 0; i < HF; ++i) fa[i] = *reinterpret_cast<const u32x4*>(sa + i * 16 * LBK + foff);
            } else if constexpr (KA) {
                const uint16_t* sa = stage_a(S_) + (wm * WT + hh * (WT / 2)) * LBK;
#pragma unroll
                for (int i = 0; i < HF; ++i) fa[i] = *reinterpret_cast<const u32x4*>(sa + i * 16 * LBK + foff);
            } else {
                const char* sa = reinterpret_cast<const char*>(stage_a(S_));
#pragma unroll
                for (int i = 0; i < HF; ++i) {
                    const int f = 16 * TF * hh + 32 * i;
                    const u32x2 lo = lds_read_tr16(sa + (kA0 ^ f)), hi = lds_read_tr16(sa + (kA1 ^ f));
                    fa[i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
                }
            }
        };
        auto rdb = [&](auto S_, u32x4 (&fb)[TF]) {
            if constexpr (KA && KB) {
                const int stage = S_;
                const uint16_t* sb = lds + stage * SH + BM * LBK + wn * WT * LBK;
#pragma unroll
                for (int j = 0; j < TF; ++j) fb[j] = *reinterpret_cast<const u32x4*>(sb + j * 16 * LBK + foff);
            } else if constexpr (KB) {
                const uint16_t* sb = stage_b(S_) + wn * WT * LBK;
#pragma unroll
                for (int j = 0; j < TF; ++j) fb[j] = *reinterpret_cast<const u32x4*>(sb + j * 16 * LBK + foff);
            } else {
                const char* sb = reinterpret_cast<const char*>(stage_b(S_));
#pragma unroll
                for (int j = 0; j < TF; ++j) {
                    const u32x2 lo = lds_read_tr16(sb + (kB0 ^ (32 * j))), hi = lds_read_tr16(sb + (kB1 ^ (32 * j)));
                    fb[j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
                }
            }
        };
        // D[n][m] = sum_k B(n,k) A(m,k): the lane's four consecutive values run along n.
        auto mm = [&](int hh, const u32x4 (&fa)[HF], const u32x4 (&fb)[TF]) {
#pragma unroll
            for (int i = 0; i < HF; ++i)
#pragma unroll
                for (int j = 0; j < TF; ++j) acc[hh * HF + i][j] = mfma16<T>(fb[j], fa[i], acc[hh * HF + i][j]);
        };
        // Scheduling of one group: its NDS fragment reads first, then NR runs
        // of MPR MFMAs, each followed by one DMA instruction when ndma == NR.
        auto weave = [&](auto NDS, int ndma) {
            __builtin_amdgcn_sched_group_barrier(0x100, decltype(NDS)::value, 0);
#pragma unroll
            for (int q = 0; q < NR; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, MPR, 0);
                if (q < ndma) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        };
        u32x4 fa0[HF], fa1[HF], fb0[TF], fb1[TF];
        // One k-tile. S_: stage (kt % 4), whose B fragments sit in fb0 (even
        // stage) or fb1; P1: finish tile kt+3 (second half); NEXT: tile kt+1
        // exists; DMA0: start tile kt+4; VM: DMA instructions allowed in
        // flight after tile kt+1's at the barrier.
        auto ktile = [&](auto S_, auto P1, auto NEXT, auto DMA0, auto VM, int kt) {
            constexpr int s = decltype(S_)::value;
            auto& fb = (s % 2 == 0) ? fb0 : fb1;
            auto& fbn = (s % 2 == 0) ? fb1 : fb0;
            rda(ic<s>{}, 1, fa1);
            if constexpr (decltype(P1)::value) dma_half(ic<(s + 3) % LSTAGES>{}, kt + 3, 1);
            mm(0, fa0, fb);
            weave(ic<HF * DSA>{}, decltype(P1)::value ? NR : 0);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (decltype(NEXT)::value) {
                __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(decltype(VM)::value));
                __builtin_amdgcn_s_barrier();
                rda(ic<(s + 1) % LSTAGES>{}, 0, fa0);
                rdb(ic<(s + 1) % LSTAGES>{}, fbn);
                if constexpr (decltype(DMA0)::value) dma_half(ic<s>{}, kt + LSTAGES, 0);
            }
            mm(1, fa1, fb);
            weave(ic<decltype(NEXT)::value ? HF * DSA + TF * DSB : 0>{}, decltype(DMA0)::value ? NR : 0);
            __builtin_amdgcn_sched_barrier(0);
        };

        // Prologue: tiles 0-3 whole; wait for tile 0.
        if constexpr (KA && KB) {
#pragma unroll
            for (int st = 0; st < LSTAGES; ++st) {
                dma_half(st, st, 0);
                dma_half(st, st, 1);
            }
        } else {
            static_for(std::make_integer_sequence<int, LSTAGES>{}, [&](auto S_) {
                dma_half(S_, decltype(S_)::value, 0);
                dma_half(S_, decltype(S_)::value, 1);
            });
        }
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(LLPS * (LSTAGES - 1)));
        __builtin_amdgcn_s_barrier();
        rda(ic<0>{}, 0, fa0);
        rdb(ic<0>{}, fb0);
        constexpr int VMS = LLPS * (LSTAGES - 2);  // steady state: tiles kt+2, kt+3 in flight
        // First round: tile 3 went out whole, so no second half at kt = 0.
        ktile(ic<0>{}, bc<false>{}, bc<true>{}, bc<true>{}, ic<VMS>{}, 0);
        static_for(std::integer_sequence<int, 1, 2, 3>{}, [&](auto S_) {
            ktile(S_, bc<true>{}, bc<true>{}, bc<true>{}, ic<VMS>{}, decltype(S_)::value);
        });
        int kt0 = LSTAGES;
        for (; kt0 + 2 * LSTAGES <= nk; kt0 += LSTAGES) {
            static_for(std::make_integer_sequence<int, LSTAGES>{}, [&](auto S_) {
                ktile(S_, bc<true>{}, bc<true>{}, bc<true>{}, ic<VMS>{}, kt0 + decltype(S_)::value);
            });
        }
        // Last round: no new tiles; finish the second half of tile nk-1 at s = 0.
        static_for(std::make_integer_sequence<int, LSTAGES>{}, [&](auto S_) {
            constexpr int s = decltype(S_)::value;
            ktile(S_, bc<s == 0>{}, bc<(s < LSTAGES - 1)>{}, bc<false>{},
                  ic<LLPS * (LSTAGES - 2 - s < 0 ? 0 : LSTAGES - 2 - s)>{}, kt0 + s);
        });

        pipelined_store<T, TF, RAG>(a, b, m0, n0, wm, wn, lr, lq, acc);
        // The next batch's prologue overwrites every stage.
        __syncthreads();
    }
}

// Paired-stage form of the pipelined kernel: the four 32-k stages are taken
// in pairs. A K-contiguous operand keeps both stages of a pair in one LDS
// region with 128-byte tile rows (chunk c at slot c ^ (row & 7)), so that one
// DMA instruction moves 8 rows x 128 B instead of 16 rows x 64 B: HBM and L2
// see 128-byte pieces of each row. A K-strided operand keeps its k-major
// stages (already 2 k-rows of 2 BM bytes per instruction). A pair's stages are
// refilled once both have been read, which the barrier of every odd k-tile
// establishes; even k-tiles need none. The DMA of pair P + 2 is issued during
// the second half of k-tile 2P + 1 and the first half of k-tile 2P + 2.
template <class T, int TF, bool KA = true, bool KB = true, bool RAG = false, int NREG = 2>
__global__ __launch_bounds__(LThreads, TF == 8 || NREG > 2 ? 1 : 2) void gemm_mfma_pair(GemmArgs a) {
    using L = LTile<TF>;
    constexpr int BM = L::BM, IPW = L::IPW;
    constexpr int HF = TF / 2;          // A fragments per half of the wave tile
    constexpr int WT = 16 * TF;         // wave tile edge
    constexpr int RH = 2 * LBK;         // halves per K-contiguous tile row (one pair of stages)
    constexpr int OPH = BM * RH;        // halves per K-contiguous operand and region
    constexpr int REG = ((KA ? 1 : 0) + (KB ? 1 : 0)) * OPH;  // halves per region
    constexpr int OFB = KA ? OPH : 0;   // B's offset inside a region
    constexpr int NDP = BM / 32;        // DMA instructions per wave, operand and pair
    constexpr int LPP = 2 * NDP;        // DMA instructions per wave and pair
    constexpr int MPR = HF * TF / NDP;  // MFMAs per DMA instruction while a half-pair goes out
    constexpr int DSA = KA ? 1 : 2, DSB = KB ? 1 : 2;  // LDS reads per fragment
    static_assert(2 * IPW == NDP, "a pair of k-major stages takes as many DMA instructions");
    static_assert(NREG > 2 || 2 * REG * sizeof(uint16_t) == pipelined_lds_bytes<TF>(KA, KB),
                  "two regions take the LDS of four stages");
    constexpr int NS = 2 * NREG;        // stages in the ring
    extern __shared__ __attribute__((aligned(1024))) uint16_t lds[];  // [region][A | B][row][64]
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = w >> 1, wn = w & 1;
    int64_t m0, n0;
    if (!pipelined_tile<BM, RAG>(a, m0, n0)) return;
    const int nk = (int)(a.k / LBK);  // a multiple of NS, at least 2 * NS
    const int lda = (int)a.lda, ldb = (int)a.ldb;

    // DMA, K-contiguous operand: instruction j of a wave covers tile rows
    // w*BM/4 + 8j + lane/8; the lane fetches the chunk that belongs at slot
    // lane%8 of its row.
    const int dch = (lane & 7) ^ (lane >> 3);
    const int voa = ((w * (BM / 4) + (lane >> 3)) * lda + dch * 8) * 2;
    const int vob = ((w * (BM / 4) + (lane >> 3)) * ldb + dch * 8) * 2;
    // K-strided operand: as in the four-stage form (32 k-rows of BM elements
    // per stage, chunk c of row r at slot c ^ kswz(r)).
    constexpr int CPK = BM / 8, RPK = 64 / CPK;
    const int kr0 = (w * IPW) * RPK + lane / CPK, kr1 = kr0 + RPK, kslot = lane % CPK;
    const int voka0 = ((lane / CPK) * lda + 8 * (kslot ^ kswz(kr0))) * 2;
    const int voka1 = ((lane / CPK) * lda + 8 * (kslot ^ kswz(kr1))) * 2;
    const int vokb0 = ((lane / CPK) * ldb + 8 * (kslot ^ kswz(kr0))) * 2;
    const int vokb1 = ((lane / CPK) * ldb + 8 * (kslot ^ kswz(kr1))) * 2;
    // Fragment reads, K-contiguous: lane -> row lane%16 of a 16-row slab,
    // chunk 4h + lane/16 of the pair (h: the stage within the pair).
    const int lr = lane & 15, lq = lane >> 4;
    const int foff0 = lr * RH + ((lq ^ (lr & 7)) << 3);
    const int foff1 = lr * RH + (((4 + lq) ^ (lr & 7)) << 3);
    // K-strided: two transposing reads per fragment, as in the four-stage form.
    const int kg = lane >> 4, ks = lane & 15, kx = (ks & 3) >> 1;
    const int kr_0 = 8 * kg + (ks >> 2), kr_1 = kr_0 + 4;
    const int kb0 = kr_0 * 2 * BM + 8 * (ks & 1) + 16 * (kx ^ kswz(kr_0));
    const int kb1 = kr_1 * 2 * BM + 8 * (ks & 1) + 16 * (kx ^ kswz(kr_1));
    const int kA0 = kb0 ^ (32 * TF * wm), kA1 = kb1 ^ (32 * TF * wm);
    const int kB0 = kb0 ^ (32 * TF * wn), kB1 = kb1 ^ (32 * TF * wn);

    for (int64_t b = blockIdx.y; b < a.batch; b += gridDim.y) {
        // Rows (K-contiguous) or columns (K-strided) of this tile inside the operand.
        const int64_t mrows = RAG && a.m - m0 < BM ? a.m - m0 : BM;
        const int64_t nrows = RAG && a.n - n0 < BM ? a.n - n0 : BM;
        const __amdgpu_buffer_rsrc_t ra = pipelined_rsrc<BM, KA, RAG>(a.A, b * a.sa, m0, a.lda, a.k, mrows);
        const __amdgpu_buffer_rsrc_t rb = pipelined_rsrc<BM, KB, RAG>(a.B, b * a.sb, n0, a.ldb, a.k, nrows);

        // DMA instruction q (operand q % 2, its instruction q / 2) of pair
        // `pair` into region R (stages 2R and 2R + 1).
        auto dma = [&](auto R_, int pair, auto Q_) {
            constexpr int R = decltype(R_)::value, q = decltype(Q_)::value, j = q / 2;
            constexpr int h = j / IPW, jj = j % IPW;  // k-major form: stage 2R + h, instruction jj
            const int kr = (w * IPW + jj) * RPK;
            if constexpr (q % 2 == 0) {
                if constexpr (KA)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        ra, MM_LDS(lds + R * REG + (w * (BM / 4) + j * 8) * RH), 16, voa,
                        (j * 8 * lda + pair * RH) * 2, 0, 0);
                else
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        ra, MM_LDS((kmajor_stage<BM * LBK, 2 * R + h, 0>() + kr * BM)), 16,
                        jj % 2 ? voka1 : voka0, ((2 * pair + h) * LBK + kr) * lda * 2, 0, 0);
            } else {
                if constexpr (KB)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rb, MM_LDS(lds + R * REG + OFB + (w * (BM / 4) + j * 8) * RH), 16, vob,
                        (j * 8 * ldb + pair * RH) * 2, 0, 0);
                else
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rb, MM_LDS((kmajor_stage<BM * LBK, 2 * R + h, 1>() + kr * BM)), 16,
                        jj % 2 ? vokb1 : vokb0, ((2 * pair + h) * LBK + kr) * ldb * 2, 0, 0);
            }
        };
        f32x4 acc[TF][TF];
#pragma unroll
        for (int i = 0; i < TF; ++i)
#pragma unroll
            for (int j = 0; j < TF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        // Stage s of the ring: region s / 2, half s % 2 (K-contiguous), or
        // k-major array s (K-strided).
        auto rda = [&](auto S_, int hh, u32x4 (&fa)[HF]) {
            constexpr int s = decltype(S_)::value;
            if constexpr (KA) {
                const uint16_t* sa = lds + (s / 2) * REG + (wm * WT + hh * (WT / 2)) * RH + (s % 2 ? foff1 : foff0);
#pragma unroll
                for (int i = 0; i < HF; ++i) fa[i] = *reinterpret_cast<const u32x4*>(sa + i * 16 * RH);
            } else {
                const char* sa = reinterpret_cast<const char*>(kmajor_stage<BM * LBK, s, 0>());
#pragma unroll
                for (int i = 0; i < HF; ++i) {
                    const int f = 16 * TF * hh + 32 * i;
                    const u32x2 lo = lds_read_tr16(sa + (kA0 ^ f)), hi = lds_read_tr16(sa + (kA1 ^ f));
                    fa[i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
                }
            }
        };
        auto rdb = [&](auto S_, u32x4 (&fb)[TF]) {
            constexpr int s = decltype(S_)::value;
            if constexpr (KB) {
                const uint16_t* sb = lds + (s / 2) * REG + OFB + wn * WT * RH + (s % 2 ? foff1 : foff0);
#pragma unroll
                for (int j = 0; j < TF; ++j) fb[j] = *reinterpret_cast<const u32x4*>(sb + j * 16 * RH);
            } else {
                const char* sb = reinterpret_cast<const char*>(kmajor_stage<BM * LBK, s, 1>());
#pragma unroll
                for (int j = 0; j < TF; ++j) {
                    const u32x2 lo = lds_read_tr16(sb + (kB0 ^ (32 * j))), hi = lds_read_tr16(sb + (kB1 ^ (32 * j)));
                    fb[j] = u32x4{lo[0], lo[1], hi[0], hi[1]};
                }
            }
        };
        auto mm = [&](int hh, const u32x4 (&fa)[HF], const u32x4 (&fb)[TF]) {
#pragma unroll
            for (int i = 0; i < HF; ++i)
#pragma unroll
                for (int j = 0; j < TF; ++j) acc[hh * HF + i][j] = mfma16<T>(fb[j], fa[i], acc[hh * HF + i][j]);
        };
        // One half k-tile: its NDS fragment reads first, then NDP runs of MPR
        // MFMAs, each followed by one DMA instruction when dma is set.
        auto weave = [&](auto NDS, bool dma_on) {
            __builtin_amdgcn_sched_group_barrier(0x100, decltype(NDS)::value, 0);
#pragma unroll
            for (int q = 0; q < NDP; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, MPR, 0);
                if (dma_on) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        };
        u32x4 fa0[HF], fa1[HF], fb0[TF], fb1[TF];
        // k-tile kt in stage S_ (kt % 4). DQ: 2 = second half of pair pq in
        // the first half (even kt), 1 = first half of pair pq in the second
        // (odd kt), 0 = none. NEXT: tile kt+1 exists; an odd kt then waits
        // for all DMA (pair (kt+1)/2) and holds the barrier.
        auto ktile = [&](auto S_, auto NEXT, auto DQ, auto VM, int pq) {
            constexpr int s = decltype(S_)::value, sn = (s + 1) % NS;
            constexpr int dq = decltype(DQ)::value;
            constexpr bool nx = decltype(NEXT)::value;
            constexpr int RQ = s % 2 ? s / 2 : (s / 2 + NREG - 1) % NREG;  // region of the pair going out
            auto& fb = (s % 2 == 0) ? fb0 : fb1;
            auto& fbn = (s % 2 == 0) ? fb1 : fb0;
            rda(S_, 1, fa1);
            if constexpr (dq == 2)
                static_for(std::make_integer_sequence<int, NDP>{},
                           [&](auto Q_) { dma(ic<RQ>{}, pq, ic<NDP + decltype(Q_)::value>{}); });
            mm(0, fa0, fb);
            weave(ic<HF * DSA>{}, dq == 2);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (nx) {
                if constexpr (s % 2 == 1) {
                    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(decltype(VM)::value));
                    __builtin_amdgcn_s_barrier();
                }
                rda(ic<sn>{}, 0, fa0);
                rdb(ic<sn>{}, fbn);
            }
            if constexpr (dq == 1)
                static_for(std::make_integer_sequence<int, NDP>{},
                           [&](auto Q_) { dma(ic<RQ>{}, pq, ic<decltype(Q_)::value>{}); });
            mm(1, fa1, fb);
            weave(ic<nx ? HF * DSA + TF * DSB : 0>{}, dq == 1);
            __builtin_amdgcn_sched_barrier(0);
        };

        // Prologue: pairs 0 .. NREG-1 (k-tiles 0 .. NS-1); wait for pair 0.
        static_for(std::make_integer_sequence<int, NREG>{}, [&](auto R_) {
            static_for(std::make_integer_sequence<int, LPP>{}, [&](auto Q_) { dma(R_, decltype(R_)::value, Q_); });
        });
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((NREG - 1) * LPP));
        __builtin_amdgcn_s_barrier();
        rda(ic<0>{}, 0, fa0);
        rdb(ic<0>{}, fb0);
        // Odd k-tile kt = 2P + 1 sends out the first half of pair P + NREG,
        // the even k-tile after it the second half; an odd k-tile's barrier
        // lets the pairs after P + 1 stay in flight (VMS instructions).
        constexpr int VMS = (NREG - 2) * LPP;
        auto round = [&](auto FIRST, int kt0) {
            static_for(std::make_integer_sequence<int, NS>{}, [&](auto S_) {
                constexpr int s = decltype(S_)::value;
                constexpr int dq = s % 2 ? 1 : (decltype(FIRST)::value && s == 0 ? 0 : 2);
                ktile(S_, bc<true>{}, ic<dq>{}, ic<VMS>{}, kt0 / 2 + s / 2 + (s % 2 ? NREG : NREG - 1));
            });
        };
        // First round: pair NREG-1's second half went out with the prologue.
        round(bc<true>{}, 0);
        int kt0 = NS;
        for (; kt0 + 2 * NS <= nk; kt0 += NS) round(bc<false>{}, kt0);
        // Last round: the second half of the last pair, then no new tiles.
        static_for(std::make_integer_sequence<int, NS>{}, [&](auto S_) {
            constexpr int s = decltype(S_)::value;
            constexpr int vm = NREG - 2 - s / 2 > 0 ? (NREG - 2 - s / 2) * LPP : 0;
            ktile(S_, bc<(s < NS - 1)>{}, ic<s == 0 ? 2 : 0>{}, ic<vm>{}, kt0 / 2 + NREG - 1);
        });

        pipelined_store<T, TF, RAG>(a, b, m0, n0, wm, wn, lr, lq, acc);
        // The next batch's prologue overwrites every stage.
        __syncthreads();
    }
}
#undef MM_LDS

// ---------------------------------------------------------------------------
// f32 kernel: TILE x TILE tile (64, or 32 when there are few tiles), BK = 16,
// 256 threads x (TILE/16)^2 outputs, FMA. Double-buffered LDS: k-tile kt+1
// is fetched into registers before tile kt is used and stored after it.
// ---------------------------------------------------------------------------
constexpr int FBK = 16;

template <bool TA, bool TB, int TILE>
__global__ __launch_bounds__(256) void gemm_f32_fma(GemmArgs a) {
    constexpr int R = TILE / 16;              // outputs per thread per dimension
    constexpr int LD = TILE * FBK / 256;      // elements per thread per operand and k-tile
    __shared__ float As[2][FBK][TILE + 4];    // [k][m]
    __shared__ float Bs[2][FBK][TILE + 4];    // [k][n]
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int64_t tiles_n = (a.n + TILE - 1) / TILE;
    const int64_t m0 = (blockIdx.x / tiles_n) * TILE, n0 = (blockIdx.x % tiles_n) * TILE;
    const int64_t nk = (a.k + FBK - 1) / FBK;
    // Element u of this thread: A (i, p) and B (p, j) walk the stored-contiguous index.
    auto a_ip = [&](int u, int& i, int& p) {
        const int q = tid + u * 256;
        if (TA) { i = q % TILE; p = q / TILE; } else { p = q % FBK; i = q / FBK; }
    };
    auto b_pj = [&](int u, int& p, int& j) {
        const int q = tid + u * 256;
        if (TB) { p = q % FBK; j = q / FBK; } else { j = q % TILE; p = q / TILE; }
    };
    for (int64_t b = blockIdx.y; b < a.batch; b += gridDim.y) {
        const float* A = reinterpret_cast<const float*>(a.A) + b * a.sa;
        const float* B = reinterpret_cast<const float*>(a.B) + b * a.sb;
        float va[LD], vb[LD];
        auto fetch = [&](int64_t k0) {
#pragma unroll
            for (int u = 0; u < LD; ++u) {
                int i, p, j, pb;
                a_ip(u, i, p);
                const int64_t gi = m0 + i, gp = k0 + p;
                va[u] = (gi < a.m && gp < a.k) ? A[TA ? gp * a.lda + gi : gi * a.lda + gp] : 0.f;
                b_pj(u, pb, j);
                const int64_t gj = n0 + j, gpb = k0 + pb;
                vb[u] = (gj < a.n && gpb < a.k) ? B[TB ? gj * a.ldb + gpb : gpb * a.ldb + gj] : 0.f;
            }
        };
        auto store = [&](int buf) {
#pragma unroll
            for (int u = 0; u < LD; ++u) {
                int i, p, j, pb;
                a_ip(u, i, p);
                As[buf][p][i] = va[u];
                b_pj(u, pb, j);
                Bs[buf][pb][j] = vb[u];
            }
        };
        float acc[R][R] = {};
        fetch(0);
        __syncthreads();  // the previous item's readers are done with buffer 0
        store(0);
        __syncthreads();
        for (int64_t kt = 0; kt < nk; ++kt) {
            const int cur = (int)(kt & 1);
            const bool more = kt + 1 < nk;
            if (more) fetch((kt + 1) * FBK);
#pragma unroll
            for (int p = 0; p < FBK; ++p) {
                float av[R], bv[R];
#pragma unroll
                for (int r = 0; r < R; ++r) av[r] = As[cur][p][ty * R + r];
#pragma unroll
                for (int c = 0; c < R; ++c) bv[c] = Bs[cur][p][tx * R + c];
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int c = 0; c < R; ++c) acc[r][c] = __builtin_fmaf(av[r], bv[c], acc[r][c]);
            }
            if (more) store(cur ^ 1);
            __syncthreads();
        }
        float* C = reinterpret_cast<float*>(a.C) + b * a.sc;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t gi = m0 + ty * R + r;
            if (gi >= a.m) continue;
#pragma unroll
            for (int c = 0; c < R; ++c) {
                const int64_t gj = n0 + tx * R + c;
                if (gj < a.n) C[gi * a.ldc + gj] = axpby<TF32>(acc[r][c], a.alpha, a.beta, &C[gi * a.ldc + gj]);
            }
        }
    }
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <class T>
const void* pick_mfma(bool ta, bool tb, bool vec, bool shortk) {
#define MM_PICK(TA_, TB_)                                                                     \
    if (ta == TA_ && tb == TB_) {                                                             \
        if (shortk)                                                                           \
            return vec ? reinterpret_cast<const void*>(&gemm_mfma_shortk<T, TA_, TB_, true>)  \
                       : reinterpret_cast<const void*>(&gemm_mfma_shortk<T, TA_, TB_, false>); \
        return vec ? reinterpret_cast<const void*>(&gemm_mfma_generic<T, TA_, TB_, true>)     \
                   : reinterpret_cast<const void*>(&gemm_mfma_generic<T, TA_, TB_, false>);   \
    }
    MM_PICK(false, false)
    MM_PICK(false, true)
    MM_PICK(true, false)
    MM_PICK(true, true)
#undef MM_PICK
    return nullptr;
}

// ---------------------------------------------------------------------------
// Small f32 products (k <= 128, at most 1024 tiles of 16 x 16 per batch
// item): one wave per 16 x 16 tile on f32 MFMA 16x16x4. Latency, not
// throughput, bounds these: every operand element of the tile is requested
// at once (one memory round trip; contraction indices past k read through an
// offset beyond the buffer resource's range and come back as zero), then
// k / 4 MFMAs run in four independent chains that are summed in a fixed
// order. Lane l supplies A(m0 + l % 16, 4t + l / 16) and B(4t + l / 16,
// n0 + l % 16) to MFMA t and ends with C rows m0 + 4 (l / 16) + q of column
// n0 + l % 16.
// ---------------------------------------------------------------------------
constexpr int SFK = 128;

template <bool TA, bool TB>
__global__ __launch_bounds__(kWave) void gemm_f32_mfma_small(GemmArgs a) {
    constexpr uint32_t kOff = 0x80000000u;
    const int lane = threadIdx.x;
    const int r = lane & 15, g = lane >> 4;
    const int64_t tiles_n = (a.n + 15) / 16;
    const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * 16, n0 = (int64_t)(blockIdx.x % tiles_n) * 16;
    const int64_t i = m0 + r < a.m ? m0 + r : a.m - 1;
    const int64_t j = n0 + r < a.n ? n0 + r : a.n - 1;
    const int64_t span_a = TA ? (a.k - 1) * a.lda + a.m : (a.m - 1) * a.lda + a.k;
    const int64_t span_b = TB ? (a.n - 1) * a.ldb + a.k : (a.k - 1) * a.ldb + a.n;
    for (int64_t b = blockIdx.y; b < a.batch; b += gridDim.y) {
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(reinterpret_cast<const float*>(a.A) + b * a.sa), (short)0,
            (int)(span_a * 4), 0x00020000);
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(reinterpret_cast<const float*>(a.B) + b * a.sb), (short)0,
            (int)(span_b * 4), 0x00020000);
        float av[SFK / 4], bv[SFK / 4];
#pragma unroll
        for (int t = 0; t < SFK / 4; ++t) {
            const int64_t p = 4 * t + g;
            const bool live = p < a.k;
            const int64_t ea = TA ? p * a.lda + i : i * a.lda + p;
            const int64_t eb = TB ? j * a.ldb + p : p * a.ldb + j;
            av[t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                        ra, live ? (uint32_t)(ea * 4) : kOff, 0, 0));
            bv[t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                        rb, live ? (uint32_t)(eb * 4) : kOff, 0, 0));
        }
        f32x4 acc[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < SFK / 4; ++t)
            acc[t & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[t], bv[t], acc[t & 3], 0, 0, 0);
        const f32x4 sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        float* C = reinterpret_cast<float*>(a.C) + b * a.sc;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t row = m0 + 4 * g + q, col = n0 + r;
            if (row < a.m && col < a.n) {
                float* dst = C + row * a.ldc + col;
                *dst = axpby<TF32>(sum[q], a.alpha, a.beta, dst);
            }
        }
    }
}

// The pipelined kernel for a transpose layout: A K-contiguous unless ta, B
// K-contiguous when tb; the paired-stage form when `pair` (NT, and NN / TT
// that are not ragged).
template <class T, int TF, bool RAG, int NREG = 2>
const void* pick_pipelined(bool ta, bool tb, bool pair) {
    if (pair && !(ta && !tb)) {  // (the launcher never pairs TN, nor ragged NN / TT)
        if (!ta && tb) return reinterpret_cast<const void*>(&gemm_mfma_pair<T, TF, true, true, RAG, NREG>);
        if constexpr (!RAG) {
            if (!ta) return reinterpret_cast<const void*>(&gemm_mfma_pair<T, TF, true, false, false, NREG>);
            return reinterpret_cast<const void*>(&gemm_mfma_pair<T, TF, false, true, false, NREG>);
        }
    }
    if (!ta && tb) return reinterpret_cast<const void*>(&gemm_mfma_large<T, TF, true, true, RAG>);
    if (!ta) return reinterpret_cast<const void*>(&gemm_mfma_large<T, TF, true, false, RAG>);
    if (tb) return reinterpret_cast<const void*>(&gemm_mfma_large<T, TF, false, true, RAG>);
    return reinterpret_cast<const void*>(&gemm_mfma_large<T, TF, false, false, RAG>);
}
template <class T, int TF>
const void* pick_pipelined(bool ta, bool tb, bool rag, bool pair) {
    return rag ? pick_pipelined<T, TF, true>(ta, tb, pair) : pick_pipelined<T, TF, false>(ta, tb, pair);
}
// 128 x 128 tiles, paired stages in four regions (one block per CU).
template <class T>
const void* pick_pair4(bool ta, bool tb, bool rag) {
    return rag ? pick_pipelined<T, 4, true, 4>(ta, tb, true) : pick_pipelined<T, 4, false, 4>(ta, tb, true);
}
// Dynamic LDS of the paired-stage form with NREG regions.
template <int TF, int NREG>
constexpr size_t pair_lds_bytes(bool ka, bool kb) {
    return (size_t)NREG * ((ka ? 1 : 0) + (kb ? 1 : 0)) * LTile<TF>::BM * 2 * LBK * sizeof(uint16_t);
}

template <int TILE>
const void* pick_f32(bool ta, bool tb) {
    if (!ta && !tb) return reinterpret_cast<const void*>(&gemm_f32_fma<false, false, TILE>);
    if (!ta && tb) return reinterpret_cast<const void*>(&gemm_f32_fma<false, true, TILE>);
    if (ta && !tb) return reinterpret_cast<const void*>(&gemm_f32_fma<true, false, TILE>);
    return reinterpret_cast<const void*>(&gemm_f32_fma<true, true, TILE>);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s, Launched* L) {
    void* args[] = {const_cast<GemmArgs*>(&a)};
    const unsigned gy = (unsigned)(a.batch < 65535 ? a.batch : 65535);
    if (a.dtype == 0) {
        const int64_t t16 = ((a.m + 15) / 16) * ((a.n + 15) / 16);
        const int64_t span_a = a.ta ? (a.k - 1) * a.lda + a.m : (a.m - 1) * a.lda + a.k;
        const int64_t span_b = a.tb ? (a.n - 1) * a.ldb + a.k : (a.k - 1) * a.ldb + a.n;
        if (a.k <= SFK && t16 <= 1024 && span_a < (1ll << 29) && span_b < (1ll << 29)) {
            const void* fn = !a.ta && !a.tb ? (const void*)&gemm_f32_mfma_small<false, false>
                             : !a.ta        ? (const void*)&gemm_f32_mfma_small<false, true>
                             : !a.tb        ? (const void*)&gemm_f32_mfma_small<true, false>
                                            : (const void*)&gemm_f32_mfma_small<true, true>;
            L->kernel = MM_KERNEL_GEMM_F32_SMALL;
            return hipLaunchKernel(fn, dim3((unsigned)t16, gy), dim3(kWave), args, 0, s);
        }
        // 64 x 64 tiles, or 32 x 32 when that leaves fewer blocks than CUs.
        const int64_t t64 = ((a.m + 63) / 64) * ((a.n + 63) / 64);
        const bool small = t64 * a.batch < 256;
        const int64_t tiles = small ? ((a.m + 31) / 32) * ((a.n + 31) / 32) : t64;
        L->kernel = MM_KERNEL_GEMM_F32;
        return hipLaunchKernel(small ? pick_f32<32>(a.ta, a.tb) : pick_f32<64>(a.ta, a.tb),
                               dim3((unsigned)tiles, gy), dim3(256), args, 0, s);
    }
    // 16-byte chunks; one batch's operand spans below 2 GiB (buffer offsets).
    const int64_t span_a = a.ta ? (a.k - 1) * a.lda + a.m : (a.m - 1) * a.lda + a.k;
    const int64_t span_b = a.tb ? (a.n - 1) * a.ldb + a.k : (a.k - 1) * a.ldb + a.n;
    const bool vec = aligned16(a.A) && aligned16(a.B) && a.lda % 8 == 0 && a.ldb % 8 == 0 &&
                     a.sa % 8 == 0 && a.sb % 8 == 0 && span_a < (1ll << 30) && span_b < (1ll << 30);
    // Products on the DMA-pipelined MFMA kernel, any transpose layout and any
    // m, n: 256 x 256 tiles when at least 192 of them cover the batch, else 128 x 128
    // tiles of the same pipeline (two blocks per CU). Measured on MI355X (NT):
    // 256 x 256 from 192 tiles on, 128 x 128 at 128 tiles and below, and
    // 128 x 128 ahead of the 128 x 128 register-staged kernel at every
    // measured shape.
    const bool pipelined = vec && a.k % (LSTAGES * LBK) == 0 &&
                           a.k >= 2 * LSTAGES * LBK && a.lda < (1 << 22) && a.ldb < (1 << 22) &&
                           a.ldc % 4 == 0 && (reinterpret_cast<uintptr_t>(a.C) & 7) == 0 && a.sc % 4 == 0;
    // m or n need not be multiples of the tile edge (edge tiles are cut at
    // the operands' extents and masked at the store).
    const int64_t big_tiles = ((a.m + 255) / 256) * ((a.n + 255) / 256);
    const bool big = pipelined && big_tiles * a.batch >= 192;
    const bool mid = !big && pipelined;
    if (big || mid) {
        const int edge = big ? LTile<8>::BM : LTile<4>::BM;
        const bool rag = a.m % edge != 0 || a.n % edge != 0;
        const int64_t tiles = big ? big_tiles : ((a.m + 127) / 128) * ((a.n + 127) / 128);
        // The paired-stage form (128-byte pieces of K-contiguous operands, a
        // barrier every second k-tile, DMA one k-tile less ahead). Measured on
        // MI355X: for NT faster with 256 x 256 tiles at every measured shape
        // and with 128 x 128 tiles when there are more of them than CUs (two
        // resident blocks per CU then hide the shorter lookahead); with at
        // most one 128 x 128 tile per CU the four-stage form is faster. NN and
        // TT (one K-strided operand) gain 2-3% at 4096^3 and 8192^3, but a
        // ragged NN product lost 9%, so ragged NN / TT keep the four-stage
        // form; TN (both K-strided) spills registers in the paired form's loop
        // and keeps it too.
        const bool ka = !a.ta, kb = a.tb;  // operands K-contiguous
        const bool pairable = (ka && kb) || (ka != kb && !rag);
        const bool pair = (big || tiles * a.batch > 256) && pairable;
        // At most one 128 x 128 tile per CU: the paired form in four regions
        // (three pairs of lookahead) when k allows whole rounds of them.
        const bool pair4 = !big && !pair && pairable && a.k % (8 * LBK) == 0 && a.k >= 16 * LBK;
        const void* fn = big    ? (a.dtype == 1 ? pick_pipelined<TF16, 8>(a.ta, a.tb, rag, pair)
                                                : pick_pipelined<TBF16, 8>(a.ta, a.tb, rag, pair))
                       : pair4 ? (a.dtype == 1 ? pick_pair4<TF16>(a.ta, a.tb, rag)
                                               : pick_pair4<TBF16>(a.ta, a.tb, rag))
                               : (a.dtype == 1 ? pick_pipelined<TF16, 4>(a.ta, a.tb, rag, pair)
                                               : pick_pipelined<TBF16, 4>(a.ta, a.tb, rag, pair));
        const unsigned grid = (unsigned)(((tiles + 7) / 8) * 8);
        L->kernel = MM_KERNEL_GEMM_LARGE;
        L->variant = (big ? LTile<8>::BM : LTile<4>::BM) + (pair || pair4 ? 1 : 0);
        return hipLaunchKernel(fn, dim3(grid, gy), dim3(LThreads), args,
                               big     ? pipelined_lds_bytes<8>(ka, kb)
                               : pair4 ? pair_lds_bytes<4, 4>(ka, kb)
                                       : pipelined_lds_bytes<4>(ka, kb),
                               s);
    }
    constexpr int PNW = 64;  // B tile rows of the panel kernel
    const int64_t panel_items = (a.m / 64) * a.batch;
    const int64_t ptiles = a.n / PNW;
    const int64_t split64 = ptiles < 32 ? ptiles : 32;  // most blocks per 64-row panel
    if (vec && !a.ta && a.tb && (a.k == 32 || a.k == 64 || a.k == 128) && a.m % 64 == 0 &&
        a.n % PNW == 0 && a.beta == 0.f && a.ldc % 8 == 0 && aligned16(a.C) && a.sc % 8 == 0 &&
        (panel_items >= 128 || panel_items * split64 >= 512) && panel_items < (1ll << 28) &&
        a.m * a.ldc < (1ll << 30)) {
        // Short-K NT products: A panel resident, B tiles streamed, the tiles
        // of a panel split over several blocks, so that few panels still
        // fill the GPU. 128-row panels (one 8-wave block per CU, 116 KiB of
        // LDS at k = 128) read each B tile once per 128 rows; they are taken
        // for k = 64 or 128 when they can fill every CU with up to 4 blocks
        // per panel, or, for panels of more than 8 tiles, up to 16 blocks of
        // at least two tiles each. Otherwise 64-row panels (two 4-wave blocks
        // per CU, 74 KiB each at k = 128), split over up to 32 blocks so that
        // at least 512 blocks run.
        static_assert(2 * panel_lds_bytes(16, PNW, 64) <= 160 * 1024, "two blocks per CU");
        static_assert(panel_lds_bytes(16, PNW, 128) <= 160 * 1024, "one block per CU");
        const int S = (int)(a.k / 8);
        const int64_t tiles = ptiles;
        const int64_t split128 = tiles <= 8 ? (tiles < 4 ? tiles : 4) : (tiles / 2 < 16 ? tiles / 2 : 16);
        const bool tall = S >= 8 && a.m % 128 == 0 && (a.m / 128) * a.batch * split128 >= 256;
        const int pm = tall ? 128 : 64;
        const int64_t items0 = (a.m / pm) * a.batch;
        const int64_t want = tall ? 256 : 512;
        const int64_t max_split = tall ? split128 : split64;
        int nsplit = (int)((want + items0 - 1) / items0);
        if (nsplit > max_split) nsplit = (int)max_split;
        const void* fn = nullptr;
#define MM_PANEL(T) (tall ? (S == 8 ? (const void*)&gemm_nt_panel<T, 8, PNW, 128>           \
                                    : (const void*)&gemm_nt_panel<T, 16, PNW, 128>)          \
                          : S == 4 ? (const void*)&gemm_nt_panel<T, 4, PNW, 64>              \
                          : S == 8 ? (const void*)&gemm_nt_panel<T, 8, PNW, 64>              \
                                   : (const void*)&gemm_nt_panel<T, 16, PNW, 64>)
        fn = a.dtype == 1 ? MM_PANEL(TF16) : MM_PANEL(TBF16);
#undef MM_PANEL
        const int64_t items = items0 * nsplit;
        const unsigned grid = (unsigned)(((items + 7) / 8) * 8);
        void* pargs[] = {const_cast<GemmArgs*>(&a), &nsplit};
        L->kernel = MM_KERNEL_GEMM_PANEL;
        L->variant = nsplit | (pm << 8);
        return hipLaunchKernel(fn, dim3(grid), dim3(pm * 4), pargs, panel_lds_bytes(S, PNW, pm), s);
    }
    const int64_t total = ((a.m + GBM - 1) / GBM) * ((a.n + GBN - 1) / GBN) * a.batch;
    int64_t per_xcd = (total + 7) / 8;
    if (per_xcd > (1 << 24)) per_xcd = 1 << 24;  // blocks then loop over their items
    const bool shortk = a.k <= GSK * GBK;
    const void* fn = a.dtype == 1 ? pick_mfma<TF16>(a.ta, a.tb, vec, shortk)
                                  : pick_mfma<TBF16>(a.ta, a.tb, vec, shortk);
    L->kernel = MM_KERNEL_GEMM_TILED;
    return hipLaunchKernel(fn, dim3((unsigned)(8 * per_xcd)), dim3(GThreads), args, 0, s);
}

}  // namespace mmk
