// Expert-ID matmul (mlx-native 0.13.0 dense_matmul_id.rs): each routed row
// r = t*top_k + s multiplies the [n, k] row-major weight of expert ids[r]
// with an f32 activation row; ids outside the expert count give +0.0 rows.
//
//   id_direct  one launch over every routed row (decode / repeated ids).
//              HBM streaming like the GEMV row form; with the shared layout,
//              slots of one token that name the same expert share one pass
//              over that expert's rows (the first such slot writes them all).
//   id_map     one workgroup: per-expert counts and ascending routed-row
//              lists (deterministic: wave-local ballot ranks plus an
//              exclusive scan across waves), and zero rows for invalid ids.
//   id_grouped per (expert, tile of routed rows, tile of outputs): a gathered
//              GEMM. bf16 weights run on MFMA with each f32 activation split
//              into bf16 hi + lo parts (two MFMAs, f32 accumulate); f32/f16
//              weights run an LDS-tiled FMA kernel. The tile list is rebuilt
//              from the counts inside every block, so the host never waits.
#include "common.hpp"
#include "kernels.hpp"

namespace mmk {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// ---------------------------------------------------------------------------
// Direct route
// ---------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ void unpack_w(u32x4 v, float* f) {
    if constexpr (T::Elems16 == 8)
        unpack8(T{}, v, f);
    else
        unpack4(v, f);
}

// One pass of R weight rows [j0, j0+R) of expert e against the activation x.
// VEC: k % 8 == 0, 16-byte aligned weights (stride and base) and activations.
template <class T, int R, bool VEC>
__device__ __forceinline__ void direct_rows(const IdArgs& a, const char* We, const float* x,
                                            int64_t j0, float* acc) {
    using S = typename T::store_t;
    const int lane = threadIdx.x & (kWave - 1);
    const S* rowp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int64_t j = j0 + r < a.n ? j0 + r : a.n - 1;
        rowp[r] = reinterpret_cast<const S*>(We) + j * a.k;
        acc[r] = 0.f;
    }
    if constexpr (VEC) {
        constexpr int CH = T::Elems16;  // weights per 16-byte load
        const int64_t nch = a.k / CH;
        constexpr int U = 4;
        int64_t c = lane;
        for (; c + kWave * (U - 1) < nch; c += kWave * U) {
            u32x4 wv[R][U];
            float xf[U][CH];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int u = 0; u < U; ++u) wv[r][u] = ld16_stream(rowp[r] + (c + kWave * u) * CH);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int h = 0; h < CH / 4; ++h)
                    unpack4(ld16(x + (c + kWave * u) * CH + 4 * h), &xf[u][4 * h]);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float wf[CH];
                    unpack_w<T>(wv[r][u], wf);
#pragma unroll
                    for (int q = 0; q < CH; ++q) acc[r] = __builtin_fmaf(wf[q], xf[u][q], acc[r]);
                }
        }
        for (; c < nch; c += kWave) {
            float xf[CH];
#pragma unroll
            for (int h = 0; h < CH / 4; ++h) unpack4(ld16(x + c * CH + 4 * h), &xf[4 * h]);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float wf[CH];
                unpack_w<T>(ld16_stream(rowp[r] + c * CH), wf);
#pragma unroll
                for (int q = 0; q < CH; ++q) acc[r] = __builtin_fmaf(wf[q], xf[q], acc[r]);
            }
        }
    } else {
        for (int64_t p = lane; p < a.k; p += kWave) {
            const float xv = x[p];
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = __builtin_fmaf(widen(T{}, rowp[r][p]), xv, acc[r]);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);
}

template <class T, int R, bool VEC>
__global__ __launch_bounds__(kThreads) void id_direct(IdArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t per_block = (int64_t)kWaves * R;
    const int64_t nchunks = (a.n + per_block - 1) / per_block;
    const int64_t rows = (int64_t)a.m * a.top_k;
    for (int64_t work = blockIdx.x; work < rows * nchunks; work += gridDim.x) {
        const int64_t r = work / nchunks;
        const int64_t j0 = (work % nchunks) * per_block + (int64_t)wave * R;
        if (j0 >= a.n) continue;
        const uint32_t e = a.ids[r];
        const int64_t t = r / a.top_k, s = r % a.top_k;
        float* out_r = a.out + r * a.n;
        if (e >= a.n_experts) {  // no weight address is formed
            if (lane < R && j0 + lane < a.n) out_r[j0 + lane] = 0.f;
            continue;
        }
        const uint32_t* tok_ids = a.ids + t * a.top_k;
        if (a.dedup) {  // an earlier slot of this token owns this expert
            bool owned = false;
            for (int64_t s2 = 0; s2 < s; ++s2) owned |= tok_ids[s2] == e;
            if (owned) continue;
        }
        const char* We = reinterpret_cast<const char*>(a.W) + (uint64_t)e * a.expert_stride_bytes;
        const float* x = reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.X) +
                                                        t * a.x_tok_stride_bytes +
                                                        s * a.x_slot_stride_bytes);
        float acc[R];
        direct_rows<T, R, VEC>(a, We, x, j0, acc);
#pragma unroll
        for (int q = 0; q < R; ++q) {
            if (lane == q && j0 + q < a.n) {
                out_r[j0 + q] = acc[q];
                if (a.dedup)
                    for (int64_t s3 = s + 1; s3 < a.top_k; ++s3)
                        if (tok_ids[s3] == e) a.out[(t * a.top_k + s3) * a.n + j0 + q] = acc[q];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Map pass: one workgroup of 16 waves; LDS holds per-wave per-expert counters.
// ---------------------------------------------------------------------------
constexpr int kMapThreads = 1024;
constexpr int kMapWaves = kMapThreads / kWave;

__global__ __launch_bounds__(kMapThreads) void id_map(IdArgs a) {
    extern __shared__ uint32_t cnt[];  // [kMapWaves][n_experts]
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const uint32_t E = a.n_experts;
    const int64_t total = (int64_t)a.m * a.top_k;
    for (int64_t i = tid; i < (int64_t)kMapWaves * E; i += kMapThreads) cnt[i] = 0;
    __syncthreads();

    const int64_t seg = (total + kMapWaves - 1) / kMapWaves;
    const int64_t seg0 = wave * seg;
    const int64_t seg1 = seg0 + seg < total ? seg0 + seg : total;
    uint32_t* my = cnt + (int64_t)wave * E;
    const uint64_t lt_mask = (1ull << lane) - 1ull;

    // Phase 1: per-wave counts over the wave's contiguous segment.
    for (int64_t base = seg0; base < seg1; base += kWave) {
        const int64_t r = base + lane;
        const uint32_t v = r < seg1 ? a.ids[r] : E;
        bool pending = r < seg1 && v < E;
        uint64_t live = __ballot(pending);
        while (live) {
            const int leader = __ffsll((unsigned long long)live) - 1;
            const uint32_t val = __shfl(v, leader);
            const uint64_t mask = __ballot(pending && v == val);
            if (lane == leader) my[val] += (uint32_t)__popcll(mask);
            if (pending && v == val) pending = false;
            live &= ~mask;
        }
    }
    __syncthreads();

    // Phase 2: exclusive scan across waves per expert; counts (cut at m).
    for (uint32_t e = tid; e < E; e += kMapThreads) {
        uint32_t run = 0;
        for (int w = 0; w < kMapWaves; ++w) {
            const uint32_t c = cnt[(int64_t)w * E + e];
            cnt[(int64_t)w * E + e] = run;
            run += c;
        }
        a.counts_w[e] = run < a.m ? run : a.m;
    }
    __syncthreads();

    // Phase 3: place each row at its ascending rank; zero rows of bad ids.
    for (int64_t base = seg0; base < seg1; base += kWave) {
        const int64_t r = base + lane;
        const uint32_t v = r < seg1 ? a.ids[r] : E;
        bool pending = r < seg1 && v < E;
        uint64_t live = __ballot(pending);
        while (live) {
            const int leader = __ffsll((unsigned long long)live) - 1;
            const uint32_t val = __shfl(v, leader);
            const uint64_t mask = __ballot(pending && v == val);
            if (pending && v == val) {
                const uint32_t pos = my[val] + (uint32_t)__popcll(mask & lt_mask);
                if (pos < a.m) a.routed_rows_w[(int64_t)val * a.m + pos] = (uint32_t)r;
                pending = false;
            }
            if (lane == leader) my[val] += (uint32_t)__popcll(mask);
            live &= ~mask;
        }
        uint64_t bad = __ballot(r < seg1 && v >= E);
        while (bad) {
            const int l = __ffsll((unsigned long long)bad) - 1;
            float* row = a.out + (base + l) * (int64_t)a.n;
            for (int64_t j = lane; j < a.n; j += kWave) row[j] = 0.f;
            bad &= bad - 1;
        }
    }
}

// ---------------------------------------------------------------------------
// Grouped pass: shared tile schedule.
// ---------------------------------------------------------------------------
// Rebuild the m-tile list from the counts: tile_start[e] = sum over e' < e of
// ceil(counts[e'] / BM). Returns the total tile count. Uses s_start[E + 1].
template <int BM>
__device__ uint32_t build_schedule(const IdArgs& a, uint32_t* s_start, uint32_t* s_part) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const uint32_t E = a.n_experts;
    // Each thread sums 4 consecutive experts (E <= 1024 = 4 * kThreads).
    uint32_t local[4];
    uint32_t sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t e = tid * 4 + q;
        uint32_t c = e < E ? a.counts[e] : 0u;
        c = c < a.m ? c : a.m;
        local[q] = (c + BM - 1) / BM;
        sum += local[q];
    }
    // Inclusive scan of `sum` within the wave.
    uint32_t incl = sum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
    }
    if (lane == kWave - 1) s_part[wave] = incl;
    __syncthreads();
    uint32_t wave_base = 0;
    for (int w = 0; w < wave; ++w) wave_base += s_part[w];
    uint32_t run = wave_base + incl - sum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t e = tid * 4 + q;
        if (e < E) s_start[e] = run;
        run += local[q];
    }
    uint32_t total = 0;
    for (int w = 0; w < kWaves; ++w) total += s_part[w];
    if (tid == 0) s_start[E] = total;
    __syncthreads();
    return total;
}

// Map a block to (tile, n-tile). Blocks are handed to the 8 XCDs round-robin,
// so tile ti goes to the blocks of XCD ti % 8 and all n-tiles of one tile run
// on one XCD, sharing its L2 for the gathered activation rows.
__device__ __forceinline__ void block_to_tile(uint32_t n_tiles, uint32_t* ti, uint32_t* nt) {
    const uint32_t bid = blockIdx.x, xcd = bid % 8u, slot = bid / 8u;
    *ti = (slot / n_tiles) * 8u + xcd;
    *nt = slot % n_tiles;
}

// Expert owning tile `ti`: largest e with s_start[e] <= ti.
__device__ __forceinline__ uint32_t find_expert(const uint32_t* s_start, uint32_t E, uint32_t ti) {
    uint32_t lo = 0, hi = E;  // s_start[lo] <= ti < s_start[hi]
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) / 2;
        if (s_start[mid] <= ti) lo = mid; else hi = mid;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// Grouped pass, bf16 weights: MFMA with bf16 hi/lo activation split.
// ---------------------------------------------------------------------------
constexpr int QBM = 128, QBN = 128, QBK = 64;
constexpr int QLDK = QBK + 8;  // LDS row pitch (elements): 144 bytes

__device__ __forceinline__ uint16_t bf16_rne(float x) { return narrow(TBF16{}, x); }

template <bool VEC>
__global__ __launch_bounds__(kThreads) void id_grouped_bf16(IdArgs a) {
    __shared__ uint32_t s_start[MM_GROUPED_MAX_E + 1];
    __shared__ uint32_t s_part[kWaves];
    __shared__ uint32_t s_rows[QBM];
    __shared__ uint64_t s_xoff[QBM];
    __shared__ __attribute__((aligned(16))) uint16_t Xhi[QBM * QLDK];
    __shared__ __attribute__((aligned(16))) uint16_t Xlo[QBM * QLDK];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const uint32_t n_tiles = (a.n + QBN - 1) / QBN;
    uint32_t ti, nt;
    block_to_tile(n_tiles, &ti, &nt);
    const uint32_t T = build_schedule<QBM>(a, s_start, s_part);
    if (ti >= T) return;
    const uint32_t e = find_expert(s_start, a.n_experts, ti);
    uint32_t c = a.counts[e];
    c = c < a.m ? c : a.m;
    const uint32_t row_begin = (ti - s_start[e]) * QBM;
    const uint32_t cnt = c - row_begin < (uint32_t)QBM ? c - row_begin : (uint32_t)QBM;
    const uint64_t total = (uint64_t)a.m * a.top_k;

    if (tid < QBM) {
        uint32_t r = 0xffffffffu;
        uint64_t off = 0;
        if ((uint32_t)tid < cnt) {
            r = a.routed_rows[(uint64_t)e * a.m + row_begin + tid];
            if (r < total) {
                const uint64_t t = r / a.top_k, s = r % a.top_k;
                off = t * a.x_tok_stride_bytes + s * a.x_slot_stride_bytes;
            } else {
                r = 0xffffffffu;
            }
        }
        s_rows[tid] = r;
        s_xoff[tid] = off;
    }
    __syncthreads();

    const int64_t n0 = (int64_t)nt * QBN + wave * 32;  // this wave's 32 output columns
    const uint16_t* We = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(a.W) +
                                                           (uint64_t)e * a.expert_stride_bytes);
    const int nmf = (int)((cnt + 15) / 16);  // live 16-row fragments

    f32x4 acc[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Weight fragment loads: lane -> column n0 + nf*16 + lane%16, k offset
    // kk*32 + (lane/16)*8 within the K step.
    auto load_w = [&](int64_t k0, u32x4 (&w)[2][2]) {
#pragma unroll
        for (int nf = 0; nf < 2; ++nf) {
            const int64_t col = n0 + nf * 16 + (lane & 15);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int64_t kb = k0 + kk * 32 + (lane >> 4) * 8;
                if (VEC && col < a.n && kb + 8 <= a.k) {
                    w[nf][kk] = ld16_stream(We + col * a.k + kb);
                } else {
                    uint32_t h[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        h[q] = (col < a.n && kb + q < a.k) ? We[col * a.k + kb + q] : 0u;
                    w[nf][kk] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                      h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
                }
            }
        }
    };

    u32x4 wcur[2][2];
    load_w(0, wcur);
    for (int64_t k0 = 0; k0 < a.k; k0 += QBK) {
        // Stage the gathered activation rows for this K step as bf16 hi/lo.
        __syncthreads();
#pragma unroll
        for (int pass = 0; pass < QBM / 16; ++pass) {
            const int row = pass * 16 + (tid >> 4);
            const int kc = (tid & 15) * 4;
            float v[4] = {0.f, 0.f, 0.f, 0.f};
            if ((uint32_t)row < cnt && s_rows[row] != 0xffffffffu) {
                const float* x = reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.X) + s_xoff[row]);
                const int64_t kb = k0 + kc;
                if (VEC && kb + 4 <= a.k) {
                    unpack4(ld16(x + kb), v);
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = kb + q < a.k ? x[kb + q] : 0.f;
                }
            }
            uint16_t hi[4], lo[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                hi[q] = bf16_rne(v[q]);
                lo[q] = bf16_rne(v[q] - __uint_as_float((uint32_t)hi[q] << 16));
            }
            *reinterpret_cast<u32x2*>(&Xhi[row * QLDK + kc]) =
                u32x2{(uint32_t)hi[0] | ((uint32_t)hi[1] << 16), (uint32_t)hi[2] | ((uint32_t)hi[3] << 16)};
            *reinterpret_cast<u32x2*>(&Xlo[row * QLDK + kc]) =
                u32x2{(uint32_t)lo[0] | ((uint32_t)lo[1] << 16), (uint32_t)lo[2] | ((uint32_t)lo[3] << 16)};
        }
        __syncthreads();
        u32x4 wnext[2][2];
        if (k0 + QBK < a.k) load_w(k0 + QBK, wnext);
#pragma unroll
        for (int mf = 0; mf < 8; ++mf) {
            if (mf < nmf) {
                const int row = mf * 16 + (lane & 15);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int ko = kk * 32 + (lane >> 4) * 8;
                    const u32x4 xh = *reinterpret_cast<const u32x4*>(&Xhi[row * QLDK + ko]);
                    const u32x4 xl = *reinterpret_cast<const u32x4*>(&Xlo[row * QLDK + ko]);
#pragma unroll
                    for (int nf = 0; nf < 2; ++nf) {
                        // D[n][row] = sum_k W(n,k) X(row,k)
                        acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, wcur[nf][kk]), __builtin_bit_cast(bf16x8, xh),
                            acc[mf][nf], 0, 0, 0);
                        acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, wcur[nf][kk]), __builtin_bit_cast(bf16x8, xl),
                            acc[mf][nf], 0, 0, 0);
                    }
                }
            }
        }
        if (k0 + QBK < a.k) {
#pragma unroll
            for (int nf = 0; nf < 2; ++nf)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) wcur[nf][kk] = wnext[nf][kk];
        }
    }

    // Lane holds out[row = mf*16 + lane%16][n = n0 + nf*16 + 4*(lane/16) + q].
#pragma unroll
    for (int mf = 0; mf < 8; ++mf) {
        if (mf >= nmf) continue;
        const int row = mf * 16 + (lane & 15);
        if ((uint32_t)row >= cnt) continue;
        const uint32_t r = s_rows[row];
        if (r == 0xffffffffu) continue;
        float* dst_row = a.out + (uint64_t)r * a.n;
#pragma unroll
        for (int nf = 0; nf < 2; ++nf) {
            const int64_t col = n0 + nf * 16 + 4 * (lane >> 4);
            float* dst = dst_row + col;
            if (col + 4 <= a.n && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
                *reinterpret_cast<f32x4*>(dst) = acc[mf][nf];
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (col + q < a.n) dst[q] = acc[mf][nf][q];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Grouped pass, any weight dtype: LDS-tiled FMA (64 rows x 64 outputs).
// ---------------------------------------------------------------------------
constexpr int FBM = 64, FBN = 64, FBK = 16;

template <class T>
__global__ __launch_bounds__(kThreads) void id_grouped_fma(IdArgs a) {
    using S = typename T::store_t;
    __shared__ uint32_t s_start[MM_GROUPED_MAX_E + 1];
    __shared__ uint32_t s_part[kWaves];
    __shared__ uint32_t s_rows[FBM];
    __shared__ uint64_t s_xoff[FBM];
    __shared__ float Xs[FBK][FBM + 4];
    __shared__ float Ws[FBK][FBN + 4];

    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const uint32_t n_tiles = (a.n + FBN - 1) / FBN;
    uint32_t ti, nt;
    block_to_tile(n_tiles, &ti, &nt);
    const uint32_t T_ = build_schedule<FBM>(a, s_start, s_part);
    if (ti >= T_) return;
    const uint32_t e = find_expert(s_start, a.n_experts, ti);
    uint32_t c = a.counts[e];
    c = c < a.m ? c : a.m;
    const uint32_t row_begin = (ti - s_start[e]) * FBM;
    const uint32_t cnt = c - row_begin < (uint32_t)FBM ? c - row_begin : (uint32_t)FBM;
    const uint64_t total = (uint64_t)a.m * a.top_k;
    if (tid < FBM) {
        uint32_t r = 0xffffffffu;
        uint64_t off = 0;
        if ((uint32_t)tid < cnt) {
            r = a.routed_rows[(uint64_t)e * a.m + row_begin + tid];
            if (r < total) {
                off = (uint64_t)(r / a.top_k) * a.x_tok_stride_bytes +
                      (uint64_t)(r % a.top_k) * a.x_slot_stride_bytes;
            } else {
                r = 0xffffffffu;
            }
        }
        s_rows[tid] = r;
        s_xoff[tid] = off;
    }
    __syncthreads();
    const S* We = reinterpret_cast<const S*>(reinterpret_cast<const char*>(a.W) +
                                             (uint64_t)e * a.expert_stride_bytes);
    const int64_t n0 = (int64_t)nt * FBN;
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < a.k; k0 += FBK) {
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int q = tid + u * kThreads;
            const int p = q & 15, i = q >> 4;  // 16 consecutive k per row
            const int64_t gp = k0 + p;
            float xv = 0.f;
            if ((uint32_t)i < cnt && s_rows[i] != 0xffffffffu && gp < a.k)
                xv = reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.X) + s_xoff[i])[gp];
            Xs[p][i] = xv;
            const int64_t gj = n0 + i;
            Ws[p][i] = (gj < a.n && gp < a.k) ? widen(T{}, We[gj * a.k + gp]) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < FBK; ++p) {
            float xv[4], wv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) xv[r] = Xs[p][ty * 4 + r];
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) wv[cc] = Ws[p][tx * 4 + cc];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) acc[r][cc] = __builtin_fmaf(xv[r], wv[cc], acc[r][cc]);
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = ty * 4 + r;
        if ((uint32_t)i >= cnt || s_rows[i] == 0xffffffffu) continue;
        float* dst = a.out + (uint64_t)s_rows[i] * a.n;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const int64_t j = n0 + tx * 4 + cc;
            if (j < a.n) dst[j] = acc[r][cc];
        }
    }
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Upper bound of the m-tile count: sum_e ceil(c_e / BM) < total / BM + E.
inline uint64_t grid_for(const IdArgs& a, int bm, int bn) {
    const uint64_t total = (uint64_t)a.m * a.top_k;
    const uint64_t tmax = (total + bm - 1) / bm + a.n_experts;
    const uint64_t n_tiles = (a.n + bn - 1) / bn;
    return 8ull * n_tiles * ((tmax + 7) / 8);
}

}  // namespace

hipError_t launch_id_direct(const IdArgs& a, hipStream_t s) {
    void* args[] = {const_cast<IdArgs*>(&a)};
    constexpr int R = 2;
    const int64_t per_block = kWaves * R;
    const int64_t work = (int64_t)a.m * a.top_k * ((a.n + per_block - 1) / per_block);
    const unsigned grid = (unsigned)(work < (1ll << 30) ? work : (1ll << 30));
    const int64_t es = a.wdtype == 0 ? 4 : 2;
    const bool vec = a.k % 8 == 0 && a.expert_stride_bytes % 16 == 0 && aligned16(a.W) &&
                     aligned16(a.X) && a.x_tok_stride_bytes % 16 == 0 &&
                     a.x_slot_stride_bytes % 16 == 0 && (a.k * es) % 16 == 0;
    const void* fn = nullptr;
    switch (a.wdtype) {
        case 0: fn = vec ? (const void*)&id_direct<TF32, R, true> : (const void*)&id_direct<TF32, R, false>; break;
        case 1: fn = vec ? (const void*)&id_direct<TF16, R, true> : (const void*)&id_direct<TF16, R, false>; break;
        case 2: fn = vec ? (const void*)&id_direct<TBF16, R, true> : (const void*)&id_direct<TBF16, R, false>; break;
        default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, s);
}

hipError_t launch_id_map(const IdArgs& a, hipStream_t s) {
    void* args[] = {const_cast<IdArgs*>(&a)};
    const size_t lds = (size_t)kMapWaves * a.n_experts * sizeof(uint32_t);
    return hipLaunchKernel(reinterpret_cast<const void*>(&id_map), dim3(1), dim3(kMapThreads), args,
                           lds, s);
}

hipError_t launch_id_grouped(const IdArgs& a, hipStream_t s) {
    void* args[] = {const_cast<IdArgs*>(&a)};
    if (a.wdtype == 2) {
        const bool vec = a.k % 8 == 0 && a.expert_stride_bytes % 16 == 0 && aligned16(a.W) &&
                         aligned16(a.X) && a.x_tok_stride_bytes % 16 == 0 &&
                         a.x_slot_stride_bytes % 16 == 0;
        const uint64_t g = grid_for(a, QBM, QBN);
        const void* fn = vec ? (const void*)&id_grouped_bf16<true> : (const void*)&id_grouped_bf16<false>;
        return hipLaunchKernel(fn, dim3((unsigned)g), dim3(kThreads), args, 0, s);
    }
    const uint64_t g = grid_for(a, FBM, FBN);
    const void* fn = a.wdtype == 0 ? (const void*)&id_grouped_fma<TF32> : (const void*)&id_grouped_fma<TF16>;
    return hipLaunchKernel(fn, dim3((unsigned)g), dim3(kThreads), args, 0, s);
}

}  // namespace mmk
