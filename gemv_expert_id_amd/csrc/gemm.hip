// Tiled GEMM route: C[b] = op(A[b]) . op(B[b]) for m > 1 and n > 1
// (tract-metal 0.23.6 mlx_gemm/mod.rs, `dispatch_metal_mlx_gemm`: tiled
// kernel over (n tiles, m tiles, batch), all four transpose layouts, batch
// strides, an aligned main K loop with a ragged tail; alpha = 1, beta = 0).
//
// f16/bf16: CDNA4 MFMA (v_mfma_f32_16x16x32_{f16,bf16}, f32 accumulate) on
// tiles staged through LDS in a K-contiguous [row][k] layout; operands stored
// with K strided are transposed while being written to LDS. f32: LDS-tiled
// FMA. Edges in M, N and K are zero-filled on load and masked on store.
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

// Stage one BM x BK (or BN x BK) tile into LDS as [row][k].
// kcontig: element (row, p) at base[row * ld + p]; else at base[p * ld + row].
template <bool KCONTIG, bool VEC>
__device__ __forceinline__ void stage_tile(const uint16_t* __restrict__ base, int64_t ld,
                                           int64_t nrows, int64_t K, int64_t row0, int64_t k0,
                                           uint16_t* __restrict__ lds) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < (GBM * GBK / 8) / GThreads; ++u) {
        const int q = tid + u * GThreads;
        if constexpr (KCONTIG) {
            const int row = q >> 2, kc = (q & 3) * 8;
            const int64_t gr = row0 + row, gk = k0 + kc;
            uint16_t* dst = lds + row * GLDK + kc;
            if (VEC && gr < nrows && gk + 8 <= K) {
                *reinterpret_cast<u32x4*>(dst) = ld16(base + gr * ld + gk);
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    dst[t] = (gr < nrows && gk + t < K) ? base[gr * ld + gk + t] : (uint16_t)0;
            }
        } else {
            const int p = q >> 4, rc = (q & 15) * 8;
            const int64_t gk = k0 + p, gr = row0 + rc;
            if (VEC && gk < K && gr + 8 <= nrows) {
                u32x4 v = ld16(base + gk * ld + gr);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    lds[(rc + 2 * t) * GLDK + p] = (uint16_t)(v[t] & 0xffffu);
                    lds[(rc + 2 * t + 1) * GLDK + p] = (uint16_t)(v[t] >> 16);
                }
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    lds[(rc + t) * GLDK + p] =
                        (gk < K && gr + t < nrows) ? base[gk * ld + gr + t] : (uint16_t)0;
            }
        }
    }
}

template <class T, bool TA, bool TB, bool VEC>
__global__ __launch_bounds__(GThreads) void gemm_mfma_generic(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t As[GBM * GLDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[GBN * GLDK];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t tiles_n = (a.n + GBN - 1) / GBN;
    const int64_t tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    const int64_t m0 = tm * GBM, n0 = tn * GBN;

    for (int64_t b = blockIdx.y; b < a.batch; b += gridDim.y) {
        const uint16_t* A = reinterpret_cast<const uint16_t*>(a.A) + b * a.sa;
        const uint16_t* B = reinterpret_cast<const uint16_t*>(a.B) + b * a.sb;
        f32x4 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int64_t k0 = 0; k0 < a.k; k0 += GBK) {
            __syncthreads();
            stage_tile<!TA, VEC>(A, a.lda, a.m, a.k, m0, k0, As);
            stage_tile<TB, VEC>(B, a.ldb, a.n, a.k, n0, k0, Bs);
            __syncthreads();
            u32x4 af[4], bf[4];
            const int kofs = (lane >> 4) * 8;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const u32x4*>(&As[(wm * 64 + i * 16 + (lane & 15)) * GLDK + kofs]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = *reinterpret_cast<const u32x4*>(&Bs[(wn * 64 + j * 16 + (lane & 15)) * GLDK + kofs]);
            // D[n][m] = sum_k B(n,k) A(m,k): lane holds C[m = lane%16][n = 4*(lane/16) + q].
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma16<T>(bf[j], af[i], acc[i][j]);
        }

        uint16_t* C = reinterpret_cast<uint16_t*>(a.C) + b * a.sc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t gm = m0 + wm * 64 + i * 16 + (lane & 15);
            if (gm >= a.m) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t gn = n0 + wn * 64 + j * 16 + 4 * (lane >> 4);
                uint16_t* dst = C + gm * a.ldc + gn;
                if (gn + 4 <= a.n && (a.ldc & 3) == 0 &&
                    (reinterpret_cast<uintptr_t>(dst) & 7) == 0) {
                    u32x2 v;
                    v[0] = (uint32_t)narrow(T{}, acc[i][j][0]) | ((uint32_t)narrow(T{}, acc[i][j][1]) << 16);
                    v[1] = (uint32_t)narrow(T{}, acc[i][j][2]) | ((uint32_t)narrow(T{}, acc[i][j][3]) << 16);
                    *reinterpret_cast<u32x2*>(dst) = v;
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (gn + q < a.n) dst[q] = narrow(T{}, acc[i][j][q]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Large f16 / bf16 kernel: C = A . B^T with A [m,k] and B [n,k] both
// K-contiguous, m % 256 == n % 256 == 0, k % 128 == 0, 16-byte aligned.
//
// Block = 8 waves (2 x 4, two per SIMD), tile 256 x 256 x 64, each wave
// 128 x 64 with v_mfma_f32_32x32x16 (8 accumulators of 16 f32 each). Every
// thread moves 4 + 4 16-byte chunks per tile: tile kt+2 is fetched into registers (buffer
// loads) while the MFMAs run on tile kt in one LDS stage and tile kt+1 is
// written into the other stage (double-buffered, 2 x 64 KiB). In LDS a tile row is 64 halves
// = 8 chunks of 16 bytes and chunk c of row r sits at slot c ^ (r & 7), so
// the fragment reads of 32 consecutive rows spread over all banks.
// Tile order: tiles are cut into groups of 8 tile-rows (column-major inside
// a group) and each XCD takes a contiguous run of that order, so the blocks
// resident on one XCD share A and B panels in its L2.
// ---------------------------------------------------------------------------
constexpr int LBM = 256, LBN = 256, LBK = 64;
constexpr int LWM = 2, LWN = 4;              // wave grid: 2 x 4 waves of 128 x 64
constexpr int LThreads = LWM * LWN * 64;
constexpr int LTILE = LBM * LBK;             // halves per operand stage
constexpr int LROWS = LThreads / 8;          // tile rows staged per pass (8 chunks/row)
constexpr int LPASS = LBM / LROWS;           // staging passes per operand

template <class T>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (T::code == 1)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <class T>
__global__ __launch_bounds__(LThreads, 1) void gemm_mfma_large(GemmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];  // [2][A | B]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / LWN, wn = wave % LWN;
    const int64_t tiles_m = a.m / LBM, tiles_n = a.n / LBN;
    const int64_t ntiles = tiles_m * tiles_n;

    // XCD-aware grouped tile order.
    const int64_t bid = blockIdx.x;
    const int64_t per_xcd = (ntiles + 7) / 8;
    const int64_t t = (bid % 8) * per_xcd + bid / 8;
    if (t >= ntiles) return;
    constexpr int GM = 8;
    const int64_t group = t / (GM * tiles_n);
    const int64_t first_m = group * GM;
    const int64_t gsize = tiles_m - first_m < GM ? tiles_m - first_m : GM;
    const int64_t tm = first_m + (t % (GM * tiles_n)) % gsize;
    const int64_t tn = (t % (GM * tiles_n)) / gsize;
    const int64_t m0 = tm * LBM, n0 = tn * LBN;

    for (int64_t b = blockIdx.y; b < a.batch; b += gridDim.y) {
        const uint16_t* A = reinterpret_cast<const uint16_t*>(a.A) + b * a.sa + m0 * a.lda;
        const uint16_t* B = reinterpret_cast<const uint16_t*>(a.B) + b * a.sb + n0 * a.ldb;

        // Staging: thread covers chunk (tid & 7) of rows (tid >> 3) + LROWS * i.
        // Buffer loads: the tile base is a scalar resource, each lane adds one
        // 32-bit offset and the row step rides in the scalar offset.
        const int srow = tid >> 3, schunk = tid & 7;
        const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(A), (short)0, (int)(LBM * a.lda * 2), 0x00020000);
        const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(B), (short)0, (int)(LBN * a.ldb * 2), 0x00020000);
        const int voa = (srow * (int)a.lda + schunk * 8) * 2;
        const int vob = (srow * (int)a.ldb + schunk * 8) * 2;
        // Two register staging sets (R0, R1): tile kt+2 is loaded while tile kt
        // is multiplied and tile kt+1 waits in registers for its LDS stage. The
        // sets alternate by name in a loop unrolled by two (never copied).
        u32x4 ra0[LPASS], rb0[LPASS], ra1[LPASS], rb1[LPASS];
        auto gload = [&](int64_t kt, u32x4 (&ra)[LPASS], u32x4 (&rb)[LPASS]) {
            const int64_t k0 = kt * LBK;
#pragma unroll
            for (int i = 0; i < LPASS; ++i) {
                ra[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                            rsa, voa, (int)((LROWS * i * a.lda + k0) * 2), 0));
                rb[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                            rsb, vob, (int)((LROWS * i * a.ldb + k0) * 2), 0));
            }
        };
        // srow & 7 is the same for every pass, so one lane offset plus immediates.
        const int sto = srow * LBK + ((schunk ^ (srow & 7)) << 3);
        auto sstore = [&](int stage, const u32x4 (&ra)[LPASS], const u32x4 (&rb)[LPASS]) {
            uint16_t* sa = lds + stage * 2 * LTILE + sto;
            uint16_t* sb = sa + LTILE;
#pragma unroll
            for (int i = 0; i < LPASS; ++i) {
                *reinterpret_cast<u32x4*>(sa + LROWS * i * LBK) = ra[i];
                *reinterpret_cast<u32x4*>(sb + LROWS * i * LBK) = rb[i];
            }
        };
        const int lrow = lane & 31, lhi = lane >> 5, lx = lane & 7;

        f32x16 acc[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

        // Wave tile: rows wm*128 + [0,128) of A, rows wn*64 + [0,64) of B.
        auto compute = [&](int stage) {
            const uint16_t* sa = lds + stage * 2 * LTILE;
            const uint16_t* sb = sa + LTILE;
#pragma unroll
            for (int ks = 0; ks < LBK / 16; ++ks) {
                // Fragment: lane -> row (lane % 32), chunk 2*ks + lane / 32.
                const int co = (((2 * ks + lhi) ^ lx) << 3) + lrow * LBK;
                u32x4 fa[4], fb[2];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    fa[i] = *reinterpret_cast<const u32x4*>(sa + (wm * 128 + i * 32) * LBK + co);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    fb[j] = *reinterpret_cast<const u32x4*>(sb + (wn * 64 + j * 32) * LBK + co);
                // D[n][m] = sum_k B(n,k) A(m,k)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) acc[i][j] = mfma32<T>(fb[j], fa[i], acc[i][j]);
            }
        };

        // sched_barrier keeps each prefetch issued before the MFMAs it overlaps
        // (left to itself the scheduler sinks the loads next to their use).
        const int64_t nk = a.k / LBK;  // even and >= 2 on this path
        gload(0, ra0, rb0);
        gload(1, ra1, rb1);
        sstore(0, ra0, rb0);
        __syncthreads();
        for (int64_t kt = 0; kt + 2 < nk; kt += 2) {
            gload(kt + 2, ra0, rb0);
            __builtin_amdgcn_sched_barrier(0);
            compute(0);
            __builtin_amdgcn_sched_barrier(0);
            sstore(1, ra1, rb1);
            __syncthreads();
            gload(kt + 3, ra1, rb1);
            __builtin_amdgcn_sched_barrier(0);
            compute(1);
            __builtin_amdgcn_sched_barrier(0);
            sstore(0, ra0, rb0);
            __syncthreads();
        }
        compute(0);
        sstore(1, ra1, rb1);
        __syncthreads();
        compute(1);

        // Lane holds C[m = mfrag base + lane%32][n = nfrag base + (v/4)*8 + (lane/32)*4 + v%4].
        uint16_t* C = reinterpret_cast<uint16_t*>(a.C) + b * a.sc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t gm = m0 + wm * 128 + i * 32 + (lane & 31);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int64_t gn = n0 + wn * 64 + j * 32 + g * 8 + (lane >> 5) * 4;
                    u32x2 v;
                    v[0] = (uint32_t)narrow(T{}, acc[i][j][4 * g]) | ((uint32_t)narrow(T{}, acc[i][j][4 * g + 1]) << 16);
                    v[1] = (uint32_t)narrow(T{}, acc[i][j][4 * g + 2]) | ((uint32_t)narrow(T{}, acc[i][j][4 * g + 3]) << 16);
                    *reinterpret_cast<u32x2*>(C + gm * a.ldc + gn) = v;
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// f32 kernel: 64 x 64 tile, BK = 16, 256 threads x (4 x 4) outputs, FMA.
// ---------------------------------------------------------------------------
constexpr int FBM = 64, FBN = 64, FBK = 16;

template <bool TA, bool TB>
__global__ __launch_bounds__(256) void gemm_f32_fma(GemmArgs a) {
    __shared__ float As[FBK][FBM + 4];  // [k][m]
    __shared__ float Bs[FBK][FBN + 4];  // [k][n]
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int64_t tiles_n = (a.n + FBN - 1) / FBN;
    const int64_t m0 = (blockIdx.x / tiles_n) * FBM, n0 = (blockIdx.x % tiles_n) * FBN;
    for (int64_t b = blockIdx.y; b < a.batch; b += gridDim.y) {
        const float* A = reinterpret_cast<const float*>(a.A) + b * a.sa;
        const float* B = reinterpret_cast<const float*>(a.B) + b * a.sb;
        float acc[4][4] = {};
        for (int64_t k0 = 0; k0 < a.k; k0 += FBK) {
            __syncthreads();
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int q = tid + u * 256;
                // A tile element (i, p): consecutive threads walk the stored-contiguous index.
                int i, p;
                if (TA) { i = q & 63; p = q >> 6; } else { p = q & 15; i = q >> 4; }
                const int64_t gi = m0 + i, gp = k0 + p;
                As[p][i] = (gi < a.m && gp < a.k) ? A[TA ? gp * a.lda + gi : gi * a.lda + gp] : 0.f;
                int j, pb;
                if (TB) { pb = q & 15; j = q >> 4; } else { j = q & 63; pb = q >> 6; }
                const int64_t gj = n0 + j, gpb = k0 + pb;
                Bs[pb][j] = (gj < a.n && gpb < a.k) ? B[TB ? gj * a.ldb + gpb : gpb * a.ldb + gj] : 0.f;
            }
            __syncthreads();
#pragma unroll
            for (int p = 0; p < FBK; ++p) {
                float av[4], bv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) av[r] = As[p][ty * 4 + r];
#pragma unroll
                for (int c = 0; c < 4; ++c) bv[c] = Bs[p][tx * 4 + c];
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[r][c] = __builtin_fmaf(av[r], bv[c], acc[r][c]);
            }
        }
        float* C = reinterpret_cast<float*>(a.C) + b * a.sc;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t gi = m0 + ty * 4 + r;
            if (gi >= a.m) continue;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int64_t gj = n0 + tx * 4 + c;
                if (gj < a.n) C[gi * a.ldc + gj] = acc[r][c];
            }
        }
    }
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <class T>
const void* pick_mfma(bool ta, bool tb, bool vec) {
#define MM_PICK(TA_, TB_)                                                                    \
    if (ta == TA_ && tb == TB_)                                                              \
        return vec ? reinterpret_cast<const void*>(&gemm_mfma_generic<T, TA_, TB_, true>)   \
                   : reinterpret_cast<const void*>(&gemm_mfma_generic<T, TA_, TB_, false>);
    MM_PICK(false, false)
    MM_PICK(false, true)
    MM_PICK(true, false)
    MM_PICK(true, true)
#undef MM_PICK
    return nullptr;
}

const void* pick_f32(bool ta, bool tb) {
    if (!ta && !tb) return reinterpret_cast<const void*>(&gemm_f32_fma<false, false>);
    if (!ta && tb) return reinterpret_cast<const void*>(&gemm_f32_fma<false, true>);
    if (ta && !tb) return reinterpret_cast<const void*>(&gemm_f32_fma<true, false>);
    return reinterpret_cast<const void*>(&gemm_f32_fma<true, true>);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
    void* args[] = {const_cast<GemmArgs*>(&a)};
    const unsigned gy = (unsigned)(a.batch < 65535 ? a.batch : 65535);
    if (a.dtype == 0) {
        const int64_t tiles = ((a.m + FBM - 1) / FBM) * ((a.n + FBN - 1) / FBN);
        return hipLaunchKernel(pick_f32(a.ta, a.tb), dim3((unsigned)tiles, gy), dim3(256), args,
                               0, s);
    }
    const bool vec = aligned16(a.A) && aligned16(a.B) && a.lda % 8 == 0 && a.ldb % 8 == 0 &&
                     a.sa % 8 == 0 && a.sb % 8 == 0;
    const int64_t big_tiles = (a.m / LBM) * (a.n / LBN);
    if (vec && !a.ta && a.tb && a.m % LBM == 0 && a.n % LBN == 0 && a.k % (2 * LBK) == 0 &&
        big_tiles >= 512 && a.ldc % 4 == 0 && (reinterpret_cast<uintptr_t>(a.C) & 7) == 0 &&
        a.sc % 4 == 0) {
        // Large NT products: 256 x 256 tiles (enough of them to fill the chip).
        const void* fn = a.dtype == 1 ? (const void*)&gemm_mfma_large<TF16>
                                      : (const void*)&gemm_mfma_large<TBF16>;
        const unsigned grid = (unsigned)(((big_tiles + 7) / 8) * 8);
        return hipLaunchKernel(fn, dim3(grid, gy), dim3(LThreads), args,
                               (size_t)2 * 2 * LTILE * sizeof(uint16_t), s);
    }
    const int64_t tiles = ((a.m + GBM - 1) / GBM) * ((a.n + GBN - 1) / GBN);
    const void* fn = a.dtype == 1 ? pick_mfma<TF16>(a.ta, a.tb, vec) : pick_mfma<TBF16>(a.ta, a.tb, vec);
    return hipLaunchKernel(fn, dim3((unsigned)tiles, gy), dim3(GThreads), args, 0, s);
}

}  // namespace mmk
