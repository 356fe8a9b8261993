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
#include <mutex>
#include <type_traits>
#include <utility>

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

// Direct route, fast form: k % (Elems16 * 64 * DU) == 0, top_k <= 64,
// aligned operands. Block = (routed row r, 4 * DR output rows),
// one wave per DR rows, no barrier. The token's whole id row arrives in one
// vector load (lane i holds slot i), so the expert, "an earlier slot owns it"
// and "later slots repeat it" are a lane read and two ballots: one memory
// round trip before the weight loads are issued. The activation chunks come
// straight from L2 next to the weight chunks they multiply; the next group of
// weight chunks is in flight while the current one is reduced.
constexpr int DR = 2;  // weight rows per wave
constexpr int DU = 4;  // 16-byte chunks per lane per row in flight

template <class T, bool ONE>
__global__ __launch_bounds__(kThreads) void id_direct_fast(IdArgs a) {
    using S = typename T::store_t;
    constexpr int CH = T::Elems16;
    constexpr int G = kWave * DU;  // chunks per group
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int64_t per_block = (int64_t)kWaves * DR;
    const int64_t nchunks = (a.n + per_block - 1) / per_block;
    const int64_t rows = (int64_t)a.m * a.top_k;
    const int64_t ngroups = (int64_t)a.k / CH / G;
    for (int64_t work = blockIdx.x; work < rows * nchunks; work += gridDim.x) {
        const int64_t r = work / nchunks;
        const int64_t j0 = (work % nchunks) * per_block + (int64_t)wave * DR;
        const int64_t t = r / a.top_k;
        const int s = (int)(r % a.top_k);
        const uint32_t v = lane < a.top_k ? a.ids[t * a.top_k + lane] : 0xffffffffu;
        const uint32_t e = __builtin_amdgcn_readlane(v, s);
        float* out_r = a.out + r * a.n;
        if (e >= a.n_experts) {  // no weight address is formed
            if (lane < DR && j0 + lane < a.n) out_r[j0 + lane] = 0.f;
            continue;
        }
        // Slots of this token naming expert e (only the shared layout merges them).
        const uint64_t same = a.dedup ? (uint64_t)__ballot(v == e) : (1ull << s);
        if (same & ((1ull << s) - 1)) continue;  // an earlier slot owns this expert
        const S* We = reinterpret_cast<const S*>(reinterpret_cast<const char*>(a.W) +
                                                 (uint64_t)e * a.expert_stride_bytes);
        const S* rowp[DR];
#pragma unroll
        for (int q = 0; q < DR; ++q) {
            const int64_t j = j0 + q < a.n ? j0 + q : a.n - 1;
            rowp[q] = We + j * a.k;
        }
        u32x4 wv[DR][DU];
#pragma unroll
        for (int q = 0; q < DR; ++q)
#pragma unroll
            for (int u = 0; u < DU; ++u) wv[q][u] = ld16_stream(rowp[q] + (lane + kWave * u) * CH);
        const float* x = reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.X) +
                                                        t * a.x_tok_stride_bytes +
                                                        s * a.x_slot_stride_bytes);
        float acc[DR];
#pragma unroll
        for (int q = 0; q < DR; ++q) acc[q] = 0.f;
        for (int64_t g = 0; g < (ONE ? 1 : ngroups); ++g) {
            u32x4 nv[ONE ? 1 : DR][DU];
            const bool more = !ONE && g + 1 < ngroups;
            if constexpr (!ONE) if (more) {
#pragma unroll
                for (int q = 0; q < DR; ++q)
#pragma unroll
                    for (int u = 0; u < DU; ++u)
                        nv[q][u] = ld16_stream(rowp[q] + ((g + 1) * G + lane + kWave * u) * CH);
            }
            u32x4 xv[DU][CH / 4];
#pragma unroll
            for (int u = 0; u < DU; ++u)
#pragma unroll
                for (int h = 0; h < CH / 4; ++h) xv[u][h] = ld16(x + (g * G + lane + kWave * u) * CH + 4 * h);
#pragma unroll
            for (int u = 0; u < DU; ++u) {
                float xf[CH];
#pragma unroll
                for (int h = 0; h < CH / 4; ++h) unpack4(xv[u][h], &xf[4 * h]);
#pragma unroll
                for (int q = 0; q < DR; ++q) {
                    float wf[CH];
                    unpack_w<T>(wv[q][u], wf);
#pragma unroll
                    for (int c = 0; c < CH; ++c) acc[q] = __builtin_fmaf(wf[c], xf[c], acc[q]);
                }
            }
            if constexpr (!ONE) if (more) {
#pragma unroll
                for (int q = 0; q < DR; ++q)
#pragma unroll
                    for (int u = 0; u < DU; ++u) wv[q][u] = nv[q][u];
            }
        }
#pragma unroll
        for (int q = 0; q < DR; ++q) acc[q] = wave_sum(acc[q]);
        const uint64_t later = same & ~((2ull << s) - 1);  // s < 64
#pragma unroll
        for (int q = 0; q < DR; ++q) {
            if (lane == q && j0 + q < a.n) {
                out_r[j0 + q] = acc[q];
                for (uint64_t mk = later; mk; mk &= mk - 1) {
                    const int64_t s3 = __builtin_ctzll(mk);
                    a.out[(t * a.top_k + s3) * a.n + j0 + q] = acc[q];
                }
            }
        }
    }
}

// Direct route, staged form: the same block shape (the REUSE form: one weight
// row per wave) and weight stream as id_direct_fast, with the activation row
// of the block's (token, slot) staged
// in LDS once per block (k * 4 bytes, k = 1024 * XPT with XPT in {1, 2, 4, 8}).
// Its loads are issued next to the id load, before the expert is known, and
// each wave then reads its activation chunks from LDS instead of from L2.
//   REUSE (slotted layout, one weight group per row): the first slot of a
//   token naming expert e keeps its weight chunks in registers and also
//   computes every later slot naming e, staging that slot's activation row
//   in turn, so a repeated expert is streamed once.
template <class T, bool ONE, bool REUSE, int XPT>  // XPT = k / 4 / kThreads exactly
__global__ __launch_bounds__(kThreads) void id_direct_staged(IdArgs a) {
    using S = typename T::store_t;
    constexpr int CH = T::Elems16;
    constexpr int G = kWave * DU;  // chunks per group
    // Weight rows per wave: one when slots reuse a repeated expert (measured
    // faster for that form), DR otherwise.
    constexpr int R = REUSE ? 1 : DR;
    extern __shared__ __attribute__((aligned(16))) float xs[];  // k floats
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int64_t per_block = (int64_t)kWaves * R;
    const int64_t nchunks = (a.n + per_block - 1) / per_block;
    const int64_t rows = (int64_t)a.m * a.top_k;
    const int64_t ngroups = (int64_t)a.k / CH / G;
    for (int64_t work = blockIdx.x; work < rows * nchunks; work += gridDim.x) {
        // Everything up to the barriers below is uniform across the block
        // (r, t, s, e depend on the work item only), so every wave reaches
        // the same barriers.
        const int64_t r = work / nchunks;
        const int64_t j0 = (work % nchunks) * per_block + (int64_t)wave * R;
        const int64_t t = r / a.top_k;
        const int s = (int)(r % a.top_k);
        const uint32_t v = lane < a.top_k ? a.ids[t * a.top_k + lane] : 0xffffffffu;
        auto xrow = [&](int slot) {
            return reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.X) +
                                                  t * a.x_tok_stride_bytes +
                                                  slot * a.x_slot_stride_bytes);
        };
        // Activation chunks of this slot (XPT per thread), in flight beside
        // the id load.
        u32x4 xv[XPT];
        {
            const float* x = xrow(s);
#pragma unroll
            for (int i = 0; i < XPT; ++i) xv[i] = ld16(x + 4 * (tid + i * kThreads));
        }
        const uint32_t e = __builtin_amdgcn_readlane(v, s);
        float* out_r = a.out + r * a.n;
        if (e >= a.n_experts) {  // no weight address is formed
            if (lane < R && j0 + lane < a.n) out_r[j0 + lane] = 0.f;
            continue;
        }
        // Slots of this token naming expert e: the shared layout writes one
        // result to all of them; REUSE computes each with its own row.
        const uint64_t same = (a.dedup || REUSE) ? (uint64_t)__ballot(v == e) : (1ull << s);
        if (same & ((1ull << s) - 1)) continue;  // an earlier slot owns this expert
        const S* We = reinterpret_cast<const S*>(reinterpret_cast<const char*>(a.W) +
                                                 (uint64_t)e * a.expert_stride_bytes);
        const S* rowp[R];
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const int64_t j = j0 + q < a.n ? j0 + q : a.n - 1;
            rowp[q] = We + j * a.k;
        }
        u32x4 wv[R][DU];
#pragma unroll
        for (int q = 0; q < R; ++q)
#pragma unroll
            for (int u = 0; u < DU; ++u) wv[q][u] = ld16_stream(rowp[q] + (lane + kWave * u) * CH);
        __syncthreads();  // the previous work item's readers are done with xs
#pragma unroll
        for (int i = 0; i < XPT; ++i) *reinterpret_cast<u32x4*>(&xs[4 * (tid + i * kThreads)]) = xv[i];
        __syncthreads();

        // acc[q] = W rows . staged activation row
        auto dot = [&](float (&acc)[R]) {
#pragma unroll
            for (int q = 0; q < R; ++q) acc[q] = 0.f;
            for (int64_t g = 0; g < (ONE ? 1 : ngroups); ++g) {
                u32x4 nv[ONE ? 1 : R][DU];
                const bool more = !ONE && g + 1 < ngroups;
                if constexpr (!ONE) if (more) {
#pragma unroll
                    for (int q = 0; q < R; ++q)
#pragma unroll
                        for (int u = 0; u < DU; ++u)
                            nv[q][u] = ld16_stream(rowp[q] + ((g + 1) * G + lane + kWave * u) * CH);
                }
#pragma unroll
                for (int u = 0; u < DU; ++u) {
                    const float* xl = &xs[(g * G + lane + kWave * u) * CH];
                    float xf[CH];
#pragma unroll
                    for (int h = 0; h < CH / 4; ++h)
                        unpack4(*reinterpret_cast<const u32x4*>(xl + 4 * h), &xf[4 * h]);
#pragma unroll
                    for (int q = 0; q < R; ++q) {
                        float wf[CH];
                        unpack_w<T>(wv[q][u], wf);
#pragma unroll
                        for (int c = 0; c < CH; ++c) acc[q] = __builtin_fmaf(wf[c], xf[c], acc[q]);
                    }
                }
                if constexpr (!ONE) if (more) {
#pragma unroll
                    for (int q = 0; q < R; ++q)
#pragma unroll
                        for (int u = 0; u < DU; ++u) wv[q][u] = nv[q][u];
                }
            }
#pragma unroll
            for (int q = 0; q < R; ++q) acc[q] = wave_sum(acc[q]);
        };
        float acc[R];
        dot(acc);
        const uint64_t later = same & ~((2ull << s) - 1);  // s < 64
#pragma unroll
        for (int q = 0; q < R; ++q) {
            if (lane == q && j0 + q < a.n) {
                out_r[j0 + q] = acc[q];
                if constexpr (!REUSE)
                    for (uint64_t mk = later; mk; mk &= mk - 1) {
                        const int64_t s3 = __builtin_ctzll(mk);
                        a.out[(t * a.top_k + s3) * a.n + j0 + q] = acc[q];
                    }
            }
        }
        if constexpr (REUSE) {
            static_assert(ONE, "slot reuse keeps one weight group in registers");
            for (uint64_t mk = later; mk; mk &= mk - 1) {
                const int s3 = __builtin_ctzll(mk);
                const float* x3 = xrow(s3);
#pragma unroll
                for (int i = 0; i < XPT; ++i) xv[i] = ld16(x3 + 4 * (tid + i * kThreads));
                __syncthreads();  // every wave is done reading the previous row
#pragma unroll
                for (int i = 0; i < XPT; ++i)
                    *reinterpret_cast<u32x4*>(&xs[4 * (tid + i * kThreads)]) = xv[i];
                __syncthreads();
                dot(acc);
#pragma unroll
                for (int q = 0; q < R; ++q)
                    if (lane == q && j0 + q < a.n) a.out[(t * a.top_k + s3) * a.n + j0 + q] = acc[q];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Map pass: one workgroup of W waves (W chosen by the host so the LDS tables
// fit). Wave w owns a contiguous segment of routed rows; LDS holds its
// per-expert counters cnt[w][e] and 64-bit lane masks msk[w][e].
//   1. counts: every lane adds 1 to cnt[w][ids[r]] (LDS atomics: the totals
//      do not depend on the order of the adds).
//   2. an exclusive scan over waves turns cnt[.][e] into each wave's first
//      slot in expert e's list; counts[e] is the total (cut at m).
//   3. per 64-row chunk, each lane ORs its lane bit into msk[w][v]; its slot
//      is the wave's running base for v plus the number of lower lanes in
//      the mask. Lists therefore come out in ascending r, independent of
//      timing. Rows of out-of-range ids are zeroed.
// ---------------------------------------------------------------------------
constexpr int kMapMaxWaves = 16;
constexpr int kMapBatch = 4;  // 64-row chunks per batch of id loads

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__global__ __launch_bounds__(kMapMaxWaves * kWave) void id_map(IdArgs a) {
    extern __shared__ uint64_t map_lds[];  // msk[W][E] (u64), then cnt[W][E] (u32)
    const int nthreads = blockDim.x, nwaves = nthreads / kWave;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const uint32_t E = a.n_experts;
    uint64_t* msk_all = map_lds;
    uint32_t* cnt = reinterpret_cast<uint32_t*>(map_lds + (int64_t)nwaves * E);
    const int64_t total = (int64_t)a.m * a.top_k;
    for (int64_t i = tid; i < (int64_t)nwaves * E; i += nthreads) {
        cnt[i] = 0;
        msk_all[i] = 0;
    }
    __syncthreads();

    const int64_t seg = (total + nwaves - 1) / nwaves;
    const int64_t seg0 = wave * seg;
    const int64_t seg1 = seg0 + seg < total ? seg0 + seg : total;
    uint32_t* my = cnt + (int64_t)wave * E;
    uint64_t* msk = msk_all + (int64_t)wave * E;
    const uint64_t below = (1ull << lane) - 1ull;

    // Ids are read in batches of kMapBatch chunks, all loads issued before use.
    for (int64_t b0 = seg0; b0 < seg1; b0 += (int64_t)kWave * kMapBatch) {
        uint32_t v[kMapBatch];
#pragma unroll
        for (int q = 0; q < kMapBatch; ++q) {
            const int64_t r = b0 + q * kWave + lane;
            v[q] = a.ids[r < seg1 ? r : seg0];
            if (r >= seg1) v[q] = E;
        }
#pragma unroll
        for (int q = 0; q < kMapBatch; ++q)
            if (v[q] < E) atomicAdd(&my[v[q]], 1u);
    }
    __syncthreads();

    for (uint32_t e = tid; e < E; e += nthreads) {
        uint32_t run = 0;
        for (int w = 0; w < nwaves; ++w) {
            const uint32_t c = cnt[(int64_t)w * E + e];
            cnt[(int64_t)w * E + e] = run;
            run += c;
        }
        a.counts_w[e] = run < a.m ? run : a.m;
    }
    __syncthreads();

    for (int64_t b0 = seg0; b0 < seg1; b0 += (int64_t)kWave * kMapBatch) {
        uint32_t vb[kMapBatch];
#pragma unroll
        for (int q = 0; q < kMapBatch; ++q) {
            const int64_t r = b0 + q * kWave + lane;
            vb[q] = a.ids[r < seg1 ? r : seg0];
        }
#pragma unroll
        for (int q = 0; q < kMapBatch; ++q) {
            const int64_t base = b0 + q * kWave;
            if (base >= seg1) break;
            const int64_t r = base + lane;
            const bool in = r < seg1;
            const uint32_t v = in ? vb[q] : E;
            const bool valid = in && v < E;
            // In program order within the wave: read the base, publish the lane
            // bit, read the chunk's mask, then one lane per expert advances the
            // base and clears the mask.
            const uint32_t first = valid ? my[v] : 0u;
            if (valid) atomicOr(reinterpret_cast<unsigned long long*>(&msk[v]), 1ull << lane);
            const uint64_t mask = valid ? msk[v] : 0ull;
            const uint32_t rank = lanes_below(mask);
            if (valid) {
                const uint32_t pos = first + rank;
                if (pos < a.m) a.routed_rows_w[(int64_t)v * a.m + pos] = (uint32_t)r;
                if ((mask & below) == 0) {
                    my[v] = first + (uint32_t)__popcll(mask);
                    msk[v] = 0ull;
                }
            }
            uint64_t bad = __ballot(in && v >= E);
            while (bad) {
                const int l = __ffsll((unsigned long long)bad) - 1;
                float* row = a.out + (base + l) * (int64_t)a.n;
                for (int64_t j = lane; j < a.n; j += kWave) row[j] = 0.f;
                bad &= bad - 1;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Grouped pass: shared tile schedule.
// ---------------------------------------------------------------------------
// Rebuild the m-tile list from the counts: tile_start[e] = sum over e' < e of
// ceil(counts[e'] / BM). Returns the total tile count. Uses s_start[E + 1].
template <int BM, int WAVES = kWaves>
__device__ __forceinline__ uint32_t build_schedule(const IdArgs& a, uint32_t* s_start, uint32_t* s_part) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const uint32_t E = a.n_experts;
    // Each thread sums EPT consecutive experts (E <= 1024 = EPT * threads).
    constexpr int EPT = MM_GROUPED_MAX_E / (WAVES * kWave);
    uint32_t local[EPT];
    uint32_t sum = 0;
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const uint32_t e = tid * EPT + q;
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
    for (int q = 0; q < EPT; ++q) {
        const uint32_t e = tid * EPT + q;
        if (e < E) s_start[e] = run;
        run += local[q];
    }
    uint32_t total = 0;
    for (int w = 0; w < WAVES; ++w) total += s_part[w];
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
//
// Tile = (expert e, up to 128 routed rows, `bn` outputs); the host picks bn
// (a multiple of 16, at most GW*GF*16) so that the tile count is close to the
// CU count: every CU streams one contiguous slab of W_e once. Block = GW
// waves; 16-output fragment f of the tile belongs to wave f % GW. Per 64-wide
// K step:
//   W  (read once from HBM) goes straight to registers in MFMA fragment
//      layout, issued two K steps ahead (three register buffers);
//   X  (the gathered f32 activation rows) is loaded two steps ahead, split
//      into bf16 hi = rne(x) and lo = rne(x - hi) with the packed hardware
//      convert, and written to a double-buffered LDS stage that all waves
//      of the block share;
//   MFMA v_mfma_f32_16x16x32_bf16: D[n][row] += W.hi + W.lo.
// One barrier per K step. W is exact in bf16 and x - hi - lo is below
// 2^-16 |x|, so the result is f32-accurate.
// ---------------------------------------------------------------------------
constexpr int QBM = 128, QBK = 64;
constexpr int QLDK = QBK + 8;  // LDS row pitch (elements): 144 bytes
constexpr int QXS = QBM * QLDK;  // elements per hi (or lo) stage
constexpr int GW = 8, GF = 3;    // waves per block, fragments per wave
constexpr int GMAXBN = GW * GF * 16;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// VEC: k % 8 == 0 and 16-byte aligned operands (16-byte weight and
// activation loads); otherwise element loads with edge masks.
template <bool VEC>
__global__ __launch_bounds__(GW * kWave, 1) void id_grouped_bf16(IdArgs a, uint32_t bn) {
    constexpr int NT = GW * kWave;       // threads
    constexpr int XRP = NT / 16;         // activation rows per staging pass
    constexpr int XP = QBM / XRP;        // staging passes
    __shared__ uint32_t s_start[MM_GROUPED_MAX_E + 1];
    __shared__ uint32_t s_part[GW];
    __shared__ uint32_t s_rows[QBM];
    __shared__ uint64_t s_xoff[QBM];
    __shared__ __attribute__((aligned(16))) uint16_t Xs[2][2][QXS];  // [stage][hi/lo]

    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform: scalar branches
    const uint32_t n_tiles = (a.n + bn - 1) / bn;
    uint32_t ti, nt;
    block_to_tile(n_tiles, &ti, &nt);
    const uint32_t T = build_schedule<QBM, GW>(a, s_start, s_part);
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

    const int64_t tile_n0 = (int64_t)nt * bn;
    const int64_t tile_n1 = tile_n0 + bn < a.n ? tile_n0 + bn : a.n;
    const int nfr = (int)((tile_n1 - tile_n0 + 15) / 16);          // fragments in this tile
    const int nf_live = nfr > wave ? (nfr - wave + GW - 1) / GW : 0;  // this wave's
    const uint16_t* We = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(a.W) +
                                                           (uint64_t)e * a.expert_stride_bytes);
    const int nmf = (int)((cnt + 15) / 16);  // live 16-row fragments
    const int64_t nk = (a.k + QBK - 1) / QBK;

    // Columns of this wave's fragments (lane -> column of fragment j).
    int64_t wcol[GF];
#pragma unroll
    for (int j = 0; j < GF; ++j) {
        const int64_t col = tile_n0 + (int64_t)(wave + GW * j) * 16 + (lane & 15);
        wcol[j] = col < tile_n1 ? col : tile_n1 - 1;
    }

    // Activation staging: thread covers 4 consecutive k of rows p*XRP + tid/16.
    const int xr0 = tid >> 4, xk = (tid & 15) * 4;
    const char* xrow[XP];
    bool xlive[XP];
#pragma unroll
    for (int p = 0; p < XP; ++p) {
        const int row = p * XRP + xr0;
        xlive[p] = (uint32_t)row < cnt && s_rows[row] != 0xffffffffu;
        const uint64_t off = xlive[p] ? s_xoff[row] : s_xoff[cnt - 1];
        xrow[p] = reinterpret_cast<const char*>(a.X) + off;
    }
    auto load_x = [&](int64_t k0, f32x4 (&xv)[XP]) {
#pragma unroll
        for (int p = 0; p < XP; ++p) {
            xv[p] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (xlive[p]) {
                const float* x = reinterpret_cast<const float*>(xrow[p]);
                const int64_t kb = k0 + xk;
                if (VEC && kb + 4 <= a.k) {
                    xv[p] = *reinterpret_cast<const f32x4*>(x + kb);
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) xv[p][q] = kb + q < a.k ? x[kb + q] : 0.f;
                }
            }
        }
    };
    auto store_x = [&](const f32x4 (&xv)[XP], int stage) {
#pragma unroll
        for (int p = 0; p < XP; ++p) {
            if (p * XRP >= (int)cnt) continue;  // no live row in this pass
            const uint32_t h01 = cvt_pk_bf16(xv[p][0], xv[p][1]);
            const uint32_t h23 = cvt_pk_bf16(xv[p][2], xv[p][3]);
            const uint32_t l01 = cvt_pk_bf16(xv[p][0] - __uint_as_float(h01 << 16),
                                             xv[p][1] - __uint_as_float(h01 & 0xffff0000u));
            const uint32_t l23 = cvt_pk_bf16(xv[p][2] - __uint_as_float(h23 << 16),
                                             xv[p][3] - __uint_as_float(h23 & 0xffff0000u));
            const int o = (p * XRP + xr0) * QLDK + xk;
            *reinterpret_cast<u32x2*>(&Xs[stage][0][o]) = u32x2{h01, h23};
            *reinterpret_cast<u32x2*>(&Xs[stage][1][o]) = u32x2{l01, l23};
        }
    };
    // Weight fragments: lane -> column wcol[j], k offset kk*32 + (lane/16)*8.
    auto load_w = [&](int64_t k0, u32x4 (&w)[GF][2]) {
#pragma unroll
        for (int j = 0; j < GF; ++j) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int64_t kb = k0 + kk * 32 + (lane >> 4) * 8;
                if (VEC && kb + 8 <= a.k) {
                    w[j][kk] = ld16_stream(We + wcol[j] * a.k + kb);
                } else {
                    uint32_t h[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q) h[q] = kb + q < a.k ? We[wcol[j] * a.k + kb + q] : 0u;
                    w[j][kk] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                     h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
                }
            }
        }
    };

    f32x4 acc[8][GF];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < GF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Register buffers rotate by name, never by copy: a copy would wait for
    // loads that were just issued. W uses three buffers (two K steps ahead),
    // X two (A/B alternate); the K loop is unrolled by 6 to close both cycles.
    u32x4 w0[GF][2], w1[GF][2], w2[GF][2];
    f32x4 xA[XP], xB[XP];
    auto compute = [&](int64_t it, const u32x4 (&wc)[GF][2]) {
        const int st = (int)(it & 1);
        // Per 32-wide half kk: the hi products of every live (row, output)
        // fragment, then the lo products, so the two MFMAs that update one
        // accumulator are never issued back to back.
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int part = 0; part < 2; ++part) {
#pragma unroll
                for (int mf = 0; mf < 8; ++mf) {
                    if (mf < nmf) {
                        const int ko = (mf * 16 + (lane & 15)) * QLDK + kk * 32 + (lane >> 4) * 8;
                        const u32x4 xv = *reinterpret_cast<const u32x4*>(&Xs[st][part][ko]);
#pragma unroll
                        for (int j = 0; j < GF; ++j) {
                            if (j < nf_live)
                                acc[mf][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    __builtin_bit_cast(bf16x8, wc[j][kk]),
                                    __builtin_bit_cast(bf16x8, xv), acc[mf][j], 0, 0, 0);
                        }
                    }
                }
            }
        }
    };
    // One K step: W(it+2) -> wf, MFMAs on W(it) = wc and stage it%2, X(it+1)
    // (held in xbuf) -> stage (it+1)%2, then X(it+3) -> xbuf.
    auto step = [&](int64_t it, const u32x4 (&wc)[GF][2], u32x4 (&wf)[GF][2], f32x4 (&xbuf)[XP]) {
        if (it + 2 < nk) load_w((it + 2) * QBK, wf);
        compute(it, wc);
        if (it + 1 < nk) store_x(xbuf, (int)((it + 1) & 1));
        if (it + 3 < nk) load_x((it + 3) * QBK, xbuf);
        __syncthreads();
    };

    load_w(0, w0);
    if (nk > 1) load_w(QBK, w1);
    load_x(0, xA);
    store_x(xA, 0);
    if (nk > 1) load_x(QBK, xA);
    if (nk > 2) load_x(2 * QBK, xB);
    __syncthreads();
    for (int64_t it = 0; it < nk; it += 6) {
        step(it, w0, w2, xA);
        if (it + 1 < nk) step(it + 1, w1, w0, xB);
        if (it + 2 < nk) step(it + 2, w2, w1, xA);
        if (it + 3 < nk) step(it + 3, w0, w2, xB);
        if (it + 4 < nk) step(it + 4, w1, w0, xA);
        if (it + 5 < nk) step(it + 5, w2, w1, xB);
    }

    // Lane holds out[row = mf*16 + lane%16][n = frag column base + 4*(lane/16) + q].
#pragma unroll
    for (int mf = 0; mf < 8; ++mf) {
        if (mf >= nmf) continue;
        const int row = mf * 16 + (lane & 15);
        if ((uint32_t)row >= cnt) continue;
        const uint32_t r = s_rows[row];
        if (r == 0xffffffffu) continue;
        float* dst_row = a.out + (uint64_t)r * a.n;
#pragma unroll
        for (int j = 0; j < GF; ++j) {
            if (j >= nf_live) continue;
            const int64_t col = tile_n0 + (int64_t)(wave + GW * j) * 16 + 4 * (lane >> 4);
            float* dst = dst_row + col;
            if (col + 4 <= tile_n1 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
                *reinterpret_cast<f32x4*>(dst) = acc[mf][j];
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (col + q < tile_n1) dst[q] = acc[mf][j][q];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Grouped pass, pipelined form for every weight dtype (k % 128 == 0, aligned
// operands, input and one expert below 2 GiB).
//
// Block = NW waves. NW = 4, one per SIMD: each wave has the whole register
// file, the accumulators of up to 8 row groups x DF output fragments of
// 16 x 16 sit in AGPRs, DF = 2, 4 or 6 picked by the host as the fewest slots
// that cover the tile. NW = 8, two per SIMD, DF = 3 (2-byte weights when a
// 4-wave block would need 5 or 6 slots): half the accumulators per wave, and
// twice the waves per CU keep more weight loads in flight (measured 3-4%
// faster on the 64-expert prefill, 1408-wide experts). Tile = (expert, up to
// 128 routed rows, bn <= 384 outputs); the host sizes bn so that the tile
// count is close to the CU count. Per K step
// of 32 (four LDS stages, step kt in stage kt % 4):
//   X  the gathered f32 activation rows go from global memory straight into
//      LDS (buffer_load ... lds; each lane fetches the 16-byte chunk that
//      belongs at its LDS slot: rows of 8 chunks, chunk c of row r at slot
//      c ^ ((r ^ (r >> 3)) & 7), so the fragment reads of 16 rows, one chunk
//      index, hit distinct 16-byte bank groups both per 8 consecutive lanes
//      in a 128-byte window and over all 16 lanes in a 256-byte window),
//      three steps ahead;
//   W  each wave's fragments (16 rows x 64 bytes per 16-byte lane load) go
//      to registers three steps ahead, four buffers rotating by name;
//   MFMA per row group, two 16-byte LDS reads give 8 floats that are split
//      in registers into bf16 hi = rne(x) and lo = rne(x - hi), then
//      v_mfma_f32_16x16x32_bf16 with W.hi and W.lo for every fragment.
// Each step opens with one wait and one barrier. Loads complete in issue
// order and a step's activations are issued just before its weights, so the
// wait covers this wave's DMA for step kt; after the barrier every wave's DMA
// for kt has landed and stage (kt - 1) % 4 is free for step kt + 3. The live
// row-group count is a template constant, so each step is straight-line code
// with a fixed number of loads.
// ---------------------------------------------------------------------------
constexpr int DW = 4;               // waves per block of the one-wave-per-SIMD form
constexpr int DQM = 128;            // routed rows per tile
constexpr int DBK = 32;             // K step
constexpr int DST = 4;              // LDS stages = weight register buffers
constexpr int DLA = DST - 1;        // steps fetched ahead
constexpr int DSTAGE = DQM * DBK;   // floats per stage

// s_waitcnt immediate: vmcnt <= n, lgkmcnt and expcnt untouched.
constexpr int dwait_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

#define MM_LDSP(p) ((__attribute__((address_space(3))) void*)(p))

// LDS slot swizzle of an activation row (8 chunks of 16 bytes per row).
__device__ __forceinline__ int xswz(int row) { return (row ^ (row >> 3)) & 7; }

struct DTile {
    const uint32_t* rows;  // routed row of each tile row (0xffffffff: none)
    const uint64_t* xoff;  // activation byte offset of each tile row
    float* xs[DST];        // LDS stages [DQM][DBK], each its own array
    uint32_t cnt;          // live rows
    int64_t tile_n0, tile_n1;
    int nf_live;           // live fragments of this wave
    int wave, lane;
    const char* W;         // expert base
};

template <int... I, class F>
__device__ __forceinline__ void dstatic_for(std::integer_sequence<int, I...>, F&& f) {
    (f(std::integral_constant<int, I>{}), ...);
}

// f16 weight fragment (8 values) -> exact bf16 pair: hi = rne(w), lo = w - hi.
// w has at most 11 significant bits and hi keeps 8, so w - hi has at most 3
// and is a bf16 value; both stay in range because bf16 shares f32's exponents.
__device__ __forceinline__ void split_f16_bf16(u32x4 w, u32x4& hi, u32x4& lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = widen(TF16{}, (uint16_t)(w[i] & 0xffffu));
        const float b = widen(TF16{}, (uint16_t)(w[i] >> 16));
        hi[i] = cvt_pk_bf16(a, b);
        lo[i] = cvt_pk_bf16(a - __uint_as_float(hi[i] << 16), b - __uint_as_float(hi[i] & 0xffff0000u));
    }
}

// WT: TBF16 (W used as stored: two MFMAs, W.x_hi + W.x_lo), TF16 (W split
// exactly into bf16 hi + lo: three MFMAs, W_hi.x_hi + W_hi.x_lo + W_lo.x_hi;
// the dropped W_lo.x_lo is below 2^-18 |w| |x|) or TF32 (f32 MFMA 16x16x4 on
// the values as stored: a fragment is two 16-byte loads per lane, 8 k values,
// and MFMA q of a step takes value q of every lane for both operands).
template <int NMF, class WT, int DF, int NW>
__device__ __attribute__((always_inline)) void grouped_dma_body(const IdArgs& a, const DTile& t) {
    constexpr int NROW = NMF * 16;                  // LDS rows in use
    constexpr int DPW = (NROW / 8 + NW - 1) / NW;   // DMA instructions per wave per step
    constexpr int WL = WT::code == 0 ? 2 : 1;       // 16-byte loads per weight fragment
    constexpr int NWR = DF * WL;                    // weight loads per wave per step
    constexpr int ES = WT::code == 0 ? 4 : 2;       // weight element bytes
    constexpr int LPS = DPW + NWR;                  // loads per wave per step
    const int lane = t.lane, wave = t.wave;
    const int64_t nk = a.k / DBK;                   // a multiple of DST
    static_assert(DLA * LPS <= 63, "loads in flight exceed vmcnt");
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.X), (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(t.W), (short)0, (int)(a.n * a.k * ES), 0x00020000);

    // DMA: instruction d of this wave fills LDS rows r0 .. r0 + 7 with
    // r0 = 8 * min(wave * DPW + d, NROW / 8 - 1) (a repeated instruction
    // rewrites identical data); lane -> row r0 + lane/8, slot lane%8.
    int xvo[DPW];
    int xr0[DPW];
#pragma unroll
    for (int d = 0; d < DPW; ++d) {
        int ins = wave * DPW + d;
        ins = ins < NROW / 8 ? ins : NROW / 8 - 1;
        xr0[d] = 8 * ins;
        const int row = 8 * ins + lane / 8;
        const bool live = (uint32_t)row < t.cnt && t.rows[row] != 0xffffffffu;
        const uint64_t off = live ? t.xoff[row] : t.xoff[t.cnt - 1];
        xvo[d] = (int)off + (((lane & 7) ^ xswz(row)) * 16);
    }
    // Stages are separate LDS arrays picked by a compile-time index: when the
    // compiler cannot tell a DMA target from the stage being read, it waits
    // for every outstanding DMA before each LDS read.
    auto dma_x = [&](int64_t kt, auto STG) {
        float* st = t.xs[decltype(STG)::value];
#pragma unroll
        for (int d = 0; d < DPW; ++d)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, MM_LDSP(st + xr0[d] * DBK), 16, xvo[d],
                                                     (int)(kt * DBK * 4), 0, 0);
    };
    // Weight fragment j: lane -> output column, k chunk (lane/16)*8 of the step.
    int wvo[DF];
#pragma unroll
    for (int j = 0; j < DF; ++j) {
        int64_t col = t.tile_n0 + (int64_t)(wave + NW * j) * 16 + (lane & 15);
        col = col < t.tile_n1 ? col : t.tile_n1 - 1;
        wvo[j] = (int)((col * a.k + (lane >> 4) * 8) * ES);
    }
    auto load_w = [&](int64_t kt, u32x4 (&w)[NWR]) {
#pragma unroll
        for (int j = 0; j < DF; ++j)
#pragma unroll
            for (int h = 0; h < WL; ++h)
                w[j * WL + h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                    wrs, wvo[j] + 16 * h, (int)(kt * DBK * ES), 0));
    };

    f32x4 acc[NMF][DF];
#pragma unroll
    for (int i = 0; i < NMF; ++i)
#pragma unroll
        for (int j = 0; j < DF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Activation fragment of row group mf: lane -> row mf*16 + lane%16,
    // floats 8*(lane/16) .. +8 (chunks 2q, 2q+1 at their swizzled slots).
    const int frow = lane & 15, fq = lane >> 4;
    auto compute = [&](auto STG, const u32x4 (&wc)[NWR]) {
        const float* st = t.xs[decltype(STG)::value];
        if constexpr (WT::code == 0) {
            // f32: row groups in chunks of four; value q of the lane's 8
            // activations and weights is contraction slot q of MFMA q.
            constexpr int NCH = (NMF + 3) / 4;
            dstatic_for(std::make_integer_sequence<int, NCH>{}, [&](auto C_) {
                constexpr int m0 = 4 * decltype(C_)::value;
                constexpr int mn = NMF - m0 < 4 ? NMF - m0 : 4;
                f32x4 x0[mn], x1[mn];
#pragma unroll
                for (int i = 0; i < mn; ++i) {
                    const int row = (m0 + i) * 16 + frow;
                    const int sw = xswz(row);
                    x0[i] = *reinterpret_cast<const f32x4*>(st + row * DBK + (((2 * fq) ^ sw) << 2));
                    x1[i] = *reinterpret_cast<const f32x4*>(st + row * DBK + (((2 * fq + 1) ^ sw) << 2));
                }
#pragma unroll
                for (int q = 0; q < 8; ++q)
#pragma unroll
                    for (int i = 0; i < mn; ++i)
#pragma unroll
                        for (int j = 0; j < DF; ++j)
                            acc[m0 + i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                __uint_as_float(wc[j * 2 + q / 4][q % 4]),
                                q < 4 ? x0[i][q % 4] : x1[i][q % 4], acc[m0 + i][j], 0, 0, 0);
            });
            return;
        }
        auto mma = [&](u32x4 w, u32x4 x, f32x4 c) __attribute__((always_inline)) {
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w),
                                                           __builtin_bit_cast(bf16x8, x), c, 0, 0, 0);
        };
        // f16 weights: the exact bf16 halves of every fragment, once per step.
        u32x4 wh[DF], wl[DF];
        if constexpr (WT::code == 1) {
#pragma unroll
            for (int j = 0; j < DF; ++j) split_f16_bf16(wc[j], wh[j], wl[j]);
        }
        // Row groups in chunks of up to four (bounded register use): the
        // chunk's rows are read and split first, then its hi products of every
        // (row group, fragment) pair, then the lo products, so the updates of
        // one accumulator are at least 4 * DF MFMAs apart when the chunk is
        // full.
        constexpr int NCH = (NMF + 3) / 4;
        dstatic_for(std::make_integer_sequence<int, NCH>{}, [&](auto C_) {
            constexpr int m0 = 4 * decltype(C_)::value;
            constexpr int mn = NMF - m0 < 4 ? NMF - m0 : 4;
            u32x4 xh[mn], xl[mn];
#pragma unroll
            for (int i = 0; i < mn; ++i) {
                const int row = (m0 + i) * 16 + frow;
                const int sw = xswz(row);
                const f32x4 x0 = *reinterpret_cast<const f32x4*>(st + row * DBK + (((2 * fq) ^ sw) << 2));
                const f32x4 x1 = *reinterpret_cast<const f32x4*>(st + row * DBK + (((2 * fq + 1) ^ sw) << 2));
                xh[i][0] = cvt_pk_bf16(x0[0], x0[1]);
                xh[i][1] = cvt_pk_bf16(x0[2], x0[3]);
                xh[i][2] = cvt_pk_bf16(x1[0], x1[1]);
                xh[i][3] = cvt_pk_bf16(x1[2], x1[3]);
                xl[i][0] = cvt_pk_bf16(x0[0] - __uint_as_float(xh[i][0] << 16), x0[1] - __uint_as_float(xh[i][0] & 0xffff0000u));
                xl[i][1] = cvt_pk_bf16(x0[2] - __uint_as_float(xh[i][1] << 16), x0[3] - __uint_as_float(xh[i][1] & 0xffff0000u));
                xl[i][2] = cvt_pk_bf16(x1[0] - __uint_as_float(xh[i][2] << 16), x1[1] - __uint_as_float(xh[i][2] & 0xffff0000u));
                xl[i][3] = cvt_pk_bf16(x1[2] - __uint_as_float(xh[i][3] << 16), x1[3] - __uint_as_float(xh[i][3] & 0xffff0000u));
            }
            // Every fragment slot is computed: a wave's dead slots read a
            // clamped, valid column and are never stored.
            if constexpr (WT::code == 2) {
#pragma unroll
                for (int i = 0; i < mn; ++i)
#pragma unroll
                    for (int j = 0; j < DF; ++j) acc[m0 + i][j] = mma(wc[j], xh[i], acc[m0 + i][j]);
#pragma unroll
                for (int i = 0; i < mn; ++i)
#pragma unroll
                    for (int j = 0; j < DF; ++j) acc[m0 + i][j] = mma(wc[j], xl[i], acc[m0 + i][j]);
            } else {
#pragma unroll
                for (int i = 0; i < mn; ++i)
#pragma unroll
                    for (int j = 0; j < DF; ++j) acc[m0 + i][j] = mma(wh[j], xh[i], acc[m0 + i][j]);
#pragma unroll
                for (int i = 0; i < mn; ++i)
#pragma unroll
                    for (int j = 0; j < DF; ++j) acc[m0 + i][j] = mma(wh[j], xl[i], acc[m0 + i][j]);
#pragma unroll
                for (int i = 0; i < mn; ++i)
#pragma unroll
                    for (int j = 0; j < DF; ++j) acc[m0 + i][j] = mma(wl[j], xh[i], acc[m0 + i][j]);
            }
        });
    };

    // Step kt: wait until this wave's X(kt) DMA is done (AHEAD: the loads of
    // that many later steps may stay in flight behind W(kt)), barrier, issue
    // step kt + DLA into the buffer step kt - 1 used, multiply.
    u32x4 wb[DST][NWR];
    // Step kt = kt0 + S (kt0 a multiple of DST, so stage S): S_ carries S.
    auto step = [&](auto AHEAD, auto LOAD, auto S_, int64_t kt, const u32x4 (&wc)[NWR],
                    u32x4 (&wf)[NWR]) {
        constexpr int S = decltype(S_)::value;
        __builtin_amdgcn_s_waitcnt(dwait_vm(NWR + decltype(AHEAD)::value * LPS));
        __builtin_amdgcn_s_barrier();
        if constexpr (decltype(LOAD)::value) {
            dma_x(kt + DLA, std::integral_constant<int, (S + DLA) % DST>{});
            load_w(kt + DLA, wf);
        }
        compute(S_, wc);
    };
    dstatic_for(std::make_integer_sequence<int, DLA>{}, [&](auto S_) {
        constexpr int s = decltype(S_)::value;
        dma_x(s, S_);
        load_w(s, wb[s]);
    });
    int64_t kt = 0;
    for (; kt + DST < nk; kt += DST) {
        dstatic_for(std::make_integer_sequence<int, DST>{}, [&](auto S_) {
            constexpr int s = decltype(S_)::value;
            step(std::integral_constant<int, DLA - 1>{}, std::integral_constant<bool, true>{}, S_,
                 kt + s, wb[s], wb[(s + DLA) % DST]);
        });
    }
    // Last DST steps: only step kt + DLA remains to be fetched (at s = 0).
    dstatic_for(std::make_integer_sequence<int, DST>{}, [&](auto S_) {
        constexpr int s = decltype(S_)::value;
        constexpr int ahead = (DST - 1 - s) < (DLA - 1) ? (DST - 1 - s) : (DLA - 1);
        step(std::integral_constant<int, ahead>{}, std::integral_constant<bool, s == 0>{}, S_,
             kt + s, wb[s], wb[(s + DLA) % DST]);
    });

    // Lane holds out[row = mf*16 + lane%16][n = fragment base + 4*(lane/16) + q].
#pragma unroll
    for (int mf = 0; mf < NMF; ++mf) {
        const int row = mf * 16 + frow;
        if ((uint32_t)row >= t.cnt) continue;
        const uint32_t r = t.rows[row];
        if (r == 0xffffffffu) continue;
        float* dst_row = a.out + (uint64_t)r * a.n;
#pragma unroll
        for (int j = 0; j < DF; ++j) {
            if (j >= t.nf_live) continue;
            const int64_t col = t.tile_n0 + (int64_t)(wave + NW * j) * 16 + 4 * fq;
            float* dst = dst_row + col;
            if (col + 4 <= t.tile_n1 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
                *reinterpret_cast<f32x4*>(dst) = acc[mf][j];
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (col + q < t.tile_n1) dst[q] = acc[mf][j][q];
            }
        }
    }
}
#undef MM_LDSP

template <class WT, int DF, int NW>
__global__ __launch_bounds__(NW * kWave, 1) void id_grouped_dma(IdArgs a, uint32_t bn) {
    __shared__ uint32_t s_start[MM_GROUPED_MAX_E + 1];
    __shared__ uint32_t s_part[NW];
    __shared__ uint32_t s_rows[DQM];
    __shared__ uint64_t s_xoff[DQM];
    __shared__ __attribute__((aligned(1024))) float Xs0[DSTAGE], Xs1[DSTAGE], Xs2[DSTAGE],
        Xs3[DSTAGE];
    static_assert(DST == 4, "one LDS array per stage");

    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const uint32_t n_tiles = (a.n + bn - 1) / bn;
    uint32_t ti, nt;
    block_to_tile(n_tiles, &ti, &nt);
    const uint32_t T = build_schedule<DQM, NW>(a, s_start, s_part);
    if (ti >= T) return;
    const uint32_t e = find_expert(s_start, a.n_experts, ti);
    uint32_t c = a.counts[e];
    c = c < a.m ? c : a.m;
    const uint32_t row_begin = (ti - s_start[e]) * DQM;
    const uint32_t cnt = c - row_begin < (uint32_t)DQM ? c - row_begin : (uint32_t)DQM;
    const uint64_t total = (uint64_t)a.m * a.top_k;
    if (tid < DQM) {
        uint32_t r = 0xffffffffu;
        uint64_t off = 0;
        if ((uint32_t)tid < cnt) {
            r = a.routed_rows[(uint64_t)e * a.m + row_begin + tid];
            if (r < total) {
                const uint64_t tk = r / a.top_k, sl = r % a.top_k;
                off = tk * a.x_tok_stride_bytes + sl * a.x_slot_stride_bytes;
            } else {
                r = 0xffffffffu;
            }
        }
        s_rows[tid] = r;
        s_xoff[tid] = off;
    }
    __syncthreads();

    DTile t;
    t.rows = s_rows;
    t.xoff = s_xoff;
    t.xs[0] = Xs0; t.xs[1] = Xs1; t.xs[2] = Xs2; t.xs[3] = Xs3;
    t.cnt = cnt;
    t.tile_n0 = (int64_t)nt * bn;
    t.tile_n1 = t.tile_n0 + bn < a.n ? t.tile_n0 + bn : a.n;
    const int nfr = (int)((t.tile_n1 - t.tile_n0 + 15) / 16);
    t.nf_live = nfr > wave ? (nfr - wave + NW - 1) / NW : 0;
    t.wave = wave;
    t.lane = lane;
    t.W = reinterpret_cast<const char*>(a.W) + (uint64_t)e * a.expert_stride_bytes;
    switch ((cnt + 15) / 16) {
        case 1: grouped_dma_body<1, WT, DF, NW>(a, t); break;
        case 2: grouped_dma_body<2, WT, DF, NW>(a, t); break;
        case 3: grouped_dma_body<3, WT, DF, NW>(a, t); break;
        case 4: grouped_dma_body<4, WT, DF, NW>(a, t); break;
        case 5: grouped_dma_body<5, WT, DF, NW>(a, t); break;
        case 6: grouped_dma_body<6, WT, DF, NW>(a, t); break;
        case 7: grouped_dma_body<7, WT, DF, NW>(a, t); break;
        default: grouped_dma_body<8, WT, DF, NW>(a, t); break;
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
// Upper bound on the tile count: every expert in use adds at most one
// partial row tile, and at most min(E, routed rows) experts are in use.
inline uint64_t grid_for(const IdArgs& a, int bm, int bn) {
    const uint64_t total = (uint64_t)a.m * a.top_k;
    const uint64_t used = total < a.n_experts ? total : a.n_experts;
    const uint64_t tmax = (total + bm - 1) / bm + used;
    const uint64_t n_tiles = (a.n + bn - 1) / bn;
    return 8ull * n_tiles * ((tmax + 7) / 8);
}

}  // namespace

hipError_t launch_id_direct(const IdArgs& a, hipStream_t s, Launched* L) {
    void* args[] = {const_cast<IdArgs*>(&a)};
    const int64_t es = a.wdtype == 0 ? 4 : 2;
    const int64_t ch = 16 / es;  // weights per 16-byte load
    const bool aligned = a.expert_stride_bytes % 16 == 0 && aligned16(a.W) && aligned16(a.X) &&
                         a.x_tok_stride_bytes % 16 == 0 && a.x_slot_stride_bytes % 16 == 0;
    if (aligned && a.k % (ch * kWave * DU) == 0 && a.top_k <= kWave) {
        const bool one = a.k == ch * kWave * DU;
        const int64_t xpt = a.k / 4 / kThreads;  // k is a multiple of 1024 here
        const bool staged = xpt == 1 || xpt == 2 || xpt == 4 || xpt == 8;
        // Activation row staged in LDS; the slotted layout with one weight
        // group per row reuses a repeated expert's weights across slots (one
        // weight row per wave). One weight group is k = 2048 (2-byte weights,
        // XPT 2) or k = 1024 (f32, XPT 1).
        const bool reuse = staged && a.layout == 1 && one;
        const int64_t per_block = kWaves * (reuse ? 1 : DR);
        const int64_t work = (int64_t)a.m * a.top_k * ((a.n + per_block - 1) / per_block);
        const unsigned grid = (unsigned)(work < (1ll << 30) ? work : (1ll << 30));
        L->kernel = MM_KERNEL_ID_DIRECT_FAST;
        if (staged) {
            L->variant = reuse ? 2 : 1;
            const void* fn = nullptr;
            if (one) {
                if (a.wdtype == 0)
                    fn = reuse ? (const void*)&id_direct_staged<TF32, true, true, 1>
                               : (const void*)&id_direct_staged<TF32, true, false, 1>;
                else if (a.wdtype == 1)
                    fn = reuse ? (const void*)&id_direct_staged<TF16, true, true, 2>
                               : (const void*)&id_direct_staged<TF16, true, false, 2>;
                else
                    fn = reuse ? (const void*)&id_direct_staged<TBF16, true, true, 2>
                               : (const void*)&id_direct_staged<TBF16, true, false, 2>;
            } else {
#define MM_DS(T) (xpt == 1 ? (const void*)&id_direct_staged<T, false, false, 1>   \
                  : xpt == 2 ? (const void*)&id_direct_staged<T, false, false, 2> \
                  : xpt == 4 ? (const void*)&id_direct_staged<T, false, false, 4> \
                             : (const void*)&id_direct_staged<T, false, false, 8>)
                fn = a.wdtype == 0 ? MM_DS(TF32) : a.wdtype == 1 ? MM_DS(TF16) : MM_DS(TBF16);
#undef MM_DS
            }
            return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, (size_t)a.k * 4, s);
        }
#define MM_DF(T) (one ? (const void*)&id_direct_fast<T, true> : (const void*)&id_direct_fast<T, false>)
        const void* fn = a.wdtype == 0 ? MM_DF(TF32) : a.wdtype == 1 ? MM_DF(TF16) : MM_DF(TBF16);
#undef MM_DF
        return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, s);
    }
    L->kernel = MM_KERNEL_ID_DIRECT;
    constexpr int R = 2;
    const int64_t per_block = kWaves * R;
    const int64_t work = (int64_t)a.m * a.top_k * ((a.n + per_block - 1) / per_block);
    const unsigned grid = (unsigned)(work < (1ll << 30) ? work : (1ll << 30));
    const bool vec = a.k % 8 == 0 && aligned;
    const void* fn = nullptr;
    switch (a.wdtype) {
        case 0: fn = vec ? (const void*)&id_direct<TF32, R, true> : (const void*)&id_direct<TF32, R, false>; break;
        case 1: fn = vec ? (const void*)&id_direct<TF16, R, true> : (const void*)&id_direct<TF16, R, false>; break;
        case 2: fn = vec ? (const void*)&id_direct<TBF16, R, true> : (const void*)&id_direct<TBF16, R, false>; break;
        default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, s);
}

hipError_t launch_id_map(const IdArgs& a, hipStream_t s, Launched* L) {
    L->kernel = MM_KERNEL_ID_MAP;
    void* args[] = {const_cast<IdArgs*>(&a)};
    // 12 bytes of LDS per (wave, expert); keep the tables within 64 KiB.
    int waves = (int)(65536 / (12ull * a.n_experts));
    waves = waves < 1 ? 1 : (waves > kMapMaxWaves ? kMapMaxWaves : waves);
    const size_t lds = (size_t)waves * a.n_experts * 12;
    return hipLaunchKernel(reinterpret_cast<const void*>(&id_map), dim3(1), dim3(waves * kWave),
                           args, lds, s);
}

hipError_t launch_id_grouped(const IdArgs& a, hipStream_t s, Launched* L) {
    // Output tile width: as few tiles as cover n at the widest tile each,
    // raised until (experts that can be in use) x tiles reaches the CU count,
    // so every CU streams one W slab even when few tokens touch few experts.
    // f32 weight fragments take twice the registers: at most four per wave.
    const uint32_t maxbn = a.wdtype == 0 ? (uint32_t)(DW * 4 * 16) : (uint32_t)GMAXBN;
    const uint32_t frags = (a.n + 15) / 16;
    uint32_t split = (a.n + maxbn - 1) / maxbn;
    const uint64_t rows = (uint64_t)a.m * a.top_k;
    const uint32_t used = (uint32_t)(rows < a.n_experts ? rows : a.n_experts);
    const uint32_t want = (256 + used - 1) / used;
    // At least one live 16-output fragment per wave of a block.
    const uint32_t most = frags / 4 > 1 ? frags / 4 : 1;
    if (split < want) split = want < most ? want : most;
    if (split < 1) split = 1;
    uint32_t bn = ((frags + split - 1) / split) * 16;
    void* args[] = {const_cast<IdArgs*>(&a), &bn};
    const uint64_t es = a.wdtype == 0 ? 4 : 2;
    const bool vec = a.k % 8 == 0 && a.expert_stride_bytes % 16 == 0 && aligned16(a.W) &&
                     aligned16(a.X) && a.x_tok_stride_bytes % 16 == 0 &&
                     a.x_slot_stride_bytes % 16 == 0;
    const uint64_t in_rows = a.layout == 0 ? a.m : (uint64_t)a.m * a.top_k;
    const bool fast = vec && a.k % (DST * DBK) == 0 && in_rows * a.k * 4 < (1ull << 31) &&
                      (uint64_t)a.n * a.k * es < (1ull << 31);
    if (fast) {
        L->kernel = MM_KERNEL_ID_GROUPED_MFMA;
        // Fragment slots per wave: the fewest of 2, 4, 6 that cover the tile.
        const uint32_t per_wave = (bn / 16 + DW - 1) / DW;
        const int df = per_wave <= 2 ? 2 : per_wave <= 4 ? 4 : 6;
        // 2-byte weight tiles that need 5 or 6 slots on 4 waves take 3 slots
        // on 8 (f32 tiles stop at 4 slots).
        if (df == 6) {
            L->variant = 3 | (8 << 8);
            const void* fn8 = a.wdtype == 2 ? (const void*)&id_grouped_dma<TBF16, 3, 8>
                                            : (const void*)&id_grouped_dma<TF16, 3, 8>;
            return hipLaunchKernel(fn8, dim3((unsigned)grid_for(a, DQM, bn)), dim3(8 * kWave), args, 0, s);
        }
        L->variant = df;
#define MM_GD(T) (df == 2 ? (const void*)&id_grouped_dma<T, 2, DW> : (const void*)&id_grouped_dma<T, 4, DW>)
        const void* fn = a.wdtype == 2 ? MM_GD(TBF16) : a.wdtype == 1 ? MM_GD(TF16) : MM_GD(TF32);
#undef MM_GD
        return hipLaunchKernel(fn, dim3((unsigned)grid_for(a, DQM, bn)), dim3(DW * kWave), args, 0, s);
    }
    if (a.wdtype == 2) {
        L->kernel = MM_KERNEL_ID_GROUPED_MFMA;
        const uint64_t g = grid_for(a, QBM, bn);
        const void* fn = vec ? (const void*)&id_grouped_bf16<true>
                             : (const void*)&id_grouped_bf16<false>;
        return hipLaunchKernel(fn, dim3((unsigned)g), dim3(GW * kWave), args, 0, s);
    }
    void* fargs[] = {const_cast<IdArgs*>(&a)};
    const uint64_t g = grid_for(a, FBM, FBN);
    L->kernel = MM_KERNEL_ID_GROUPED_FMA;
    const void* fn = a.wdtype == 0 ? (const void*)&id_grouped_fma<TF32> : (const void*)&id_grouped_fma<TF16>;
    return hipLaunchKernel(fn, dim3((unsigned)g), dim3(kThreads), fargs, 0, s);
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free prefill entry point: counts[E] followed (at
// the next 256-byte boundary) by routed_rows[E * m], u32. Each GPU holds its
// own copy of the array until the process ends; every call on one GPU shares
// it, so calls that overlap on one GPU race. Nothing in it needs clearing:
// the map pass writes every count and every list entry the grouped pass reads.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint32_t scratch[kStaticScratchBytes / 4];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of `scratch` on the GPU that runs `s` (the current device
// for the null stream). The first call for a GPU looks the address up with
// that GPU current and keeps it; host code never passes the array's own name
// (a host-side stand-in) to a kernel or a copy.
hipError_t static_scratch(hipStream_t s, void** out) {
    int dev = -1;
    hipError_t err = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        if ((err = hipGetDevice(&cur)) != hipSuccess) return err;
        if (cur != dev && (err = hipSetDevice(dev)) != hipSuccess) return err;
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (err == hipSuccess) err = back;
        }
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace mmk
