// Skinny route: C = A . B^T with only a few (2..64) rows on one side, both
// operands stored with rows along the contraction (tract-metal 0.23.6
// mlx_gemm/mod.rs, `gemv_wide_config` and `dispatch_metal_mlx_gemv_wide`: a
// padded GEMM tile would waste most of its rows, so the weight block is
// streamed once for all activation rows).
//
// Roles: W is the operand with many rows (streamed from HBM once), X the one
// with at most 64 rows (re-read from L2). out(x_row, w_row) lands at
// out[x_row * out_sx + w_row * out_sw], which covers both C = X . W^T
// (X = A) and C = W . X^T (W = A).
//
// One block computes NXF (1 to 4) 16 x 16 MFMA fragments: 16 weight rows
// against all activation rows, 16 per fragment (padded rows read zeros
// without a memory access and their results are never stored; weight rows
// past the end repeat the last row, also never stored). Each weight fragment read from LDS feeds NXF MFMAs.
// The weight rows stream through a ring of SST LDS stages, each 16 rows x 1 KB:
// one DMA instruction (buffer_load ... lds) moves 1 KB of one row, so HBM
// sees whole contiguous row pieces as in the GEMV row form. Lane i of that
// instruction fetches chunk i ^ row so that, later, the 16 lanes reading one
// chunk index of 16 different rows hit 16 different bank groups. A stage holds
// 16 contraction steps of four 16-byte chunks; wave w multiplies steps
// 4w .. 4w + 3 of every stage: it reads the weight fragment (lane l: row l % 16,
// chunk 4 * step + l / 16) from LDS and the matching activation fragment,
// prefetched into registers with the stage's DMA, and issues one MFMA per
// activation fragment (f16/bf16: 16x16x32; f32: four 16x16x4, component q of
// every lane's chunk being contraction slot q for both operands). Each stage
// opens with one wait and one barrier; the stage computed two steps earlier
// is then free for the next DMA. The four waves' partial fragments are
// summed in a fixed order through LDS. HBM-bound: about 2 * rows FLOP per
// weight byte.
#include <utility>

#include "common.hpp"
#include "kernels.hpp"

namespace mmk {

namespace {

constexpr int SThreads = 256;
constexpr int SWaves = SThreads / kWave;
constexpr int SST = 3;             // LDS stages
constexpr int SROW = 1024;         // bytes of one weight row per stage
constexpr int SCH = SROW / 16;     // 16-byte chunks of one row per stage
// Loads per wave per stage: 4 row pieces + 4 activation chunks per fragment.
constexpr int sops(int nxf) { return 4 + 4 * nxf; }
static_assert(SWaves * 4 == 16 && SCH == 4 * 4 * SWaves, "one fragment, four steps per wave");

// s_waitcnt immediate: vmcnt <= n; lgkmcnt and expcnt untouched.
constexpr int swait_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

#define MM_LDSP(p) ((__attribute__((address_space(3))) void*)(p))

template <int... I, class F>
__device__ __forceinline__ void sk_for(std::integer_sequence<int, I...>, F&& f) {
    (f(std::integral_constant<int, I>{}), ...);
}

template <class T>
__device__ __forceinline__ f32x4 frag_mma(u32x4 w, u32x4 x, f32x4 acc) {
    if constexpr (T::code == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w[q]), __uint_as_float(x[q]),
                                                       acc, 0, 0, 0);
        return acc;
    } else if constexpr (T::code == 1) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, w),
                                                      __builtin_bit_cast(f16x8, x), acc, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w),
                                                       __builtin_bit_cast(bf16x8, x), acc, 0, 0, 0);
    }
}

// Requires k, ldw, ldx and the batch strides to be multiples of Elems16,
// 16-byte aligned W and X, and each batch's W and X extents below 2 GiB:
// every 16-byte chunk is then wholly inside a row or wholly past its end.
// Chunks past the end are fetched through an offset beyond the buffer
// resource's range, which yields zeros without touching memory; weight
// chunks past the end are also zeroed after the LDS read.
template <class T, int NXF>
__global__ __launch_bounds__(SThreads) void gemv_wide(SkinnyArgs a) {
    using S = typename T::store_t;
    constexpr int CH = T::Elems16;
    constexpr uint32_t kOff = 0x80000000u;  // past every resource range
    __shared__ __attribute__((aligned(1024))) uint8_t ring0[16 * SROW], ring1[16 * SROW],
        ring2[16 * SROW];
    static_assert(SST == 3, "one LDS array per stage");
    uint8_t* const ring[SST] = {ring0, ring1, ring2};
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int r = lane & 15, g = lane >> 4;
    const int64_t w0 = (int64_t)blockIdx.x * 16;
    const int64_t nch = a.k / CH;               // chunks per row
    const int64_t nst = (nch + SCH - 1) / SCH;  // stages
    // DMA rows of this wave: 4 * wave + d.
    uint32_t dbyte[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int64_t gr = w0 + 4 * wave + d < a.nw ? w0 + 4 * wave + d : a.nw - 1;
        dbyte[d] = (uint32_t)(gr * a.ldw * (int64_t)sizeof(S));
    }
    constexpr int SOPS = sops(NXF);
    // Activation row of fragment f for this lane; padded rows (past nx) read
    // zeros through an offset beyond the resource range, without a memory access.
    uint32_t xbyte[NXF];
    bool xlive[NXF];
#pragma unroll
    for (int f = 0; f < NXF; ++f) {
        xlive[f] = 16 * f + r < a.nx;
        const int64_t xrow = xlive[f] ? 16 * f + r : 0;
        xbyte[f] = (uint32_t)(xrow * a.ldx * (int64_t)sizeof(S));
    }

    for (int64_t b = blockIdx.y; b < a.batch; b += gridDim.y) {
        const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<S*>(static_cast<const S*>(a.W) + b * a.sw), (short)0, (int)a.w_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<S*>(static_cast<const S*>(a.X) + b * a.sx), (short)0, (int)a.x_bytes, 0x00020000);
        // Stage st into ring slot SLOT: this wave's four row pieces and the
        // activation chunks of its four steps.
        auto issue = [&](int64_t st, auto SLOT, u32x4 (&xv)[NXF][4]) {
            uint8_t* base = ring[decltype(SLOT)::value];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int row = 4 * wave + d;
                const int64_t c = st * SCH + (lane ^ row);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    wrs, MM_LDSP(base + row * SROW), 16,
                    c < nch ? dbyte[d] + (uint32_t)(c * 16) : kOff, 0, 0, 0);
            }
#pragma unroll
            for (int f = 0; f < NXF; ++f)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t c = st * SCH + 4 * (4 * wave + j) + g;
                    xv[f][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                   xrs, xlive[f] && c < nch ? xbyte[f] + (uint32_t)(c * 16) : kOff, 0, 0));
                }
        };
        f32x4 acc[NXF];
#pragma unroll
        for (int f = 0; f < NXF; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto compute = [&](int64_t st, auto SLOT, const u32x4 (&xv)[NXF][4]) {
            const uint8_t* base = ring[decltype(SLOT)::value];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int cl = 4 * (4 * wave + j) + g;
                u32x4 wv = *reinterpret_cast<const u32x4*>(base + r * SROW + ((cl ^ r) << 4));
                if (st * SCH + cl >= nch) wv = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int f = 0; f < NXF; ++f) acc[f] = frag_mma<T>(wv, xv[f][j], acc[f]);
            }
        };
        u32x4 xb[SST][NXF][4];
        sk_for(std::make_integer_sequence<int, SST - 1>{}, [&](auto P) {
            if (decltype(P)::value < nst) issue(decltype(P)::value, P, xb[decltype(P)::value]);
        });
        // Stage st sits in slot st % SST; after its wait and barrier, stage
        // st + SST - 1 goes into the slot stage st - 1 used. Rounds in which
        // every such stage exists run without conditions (so the compiler's
        // own waits stay exact); the last few stages take the checked form.
        int64_t st0 = 0;
        for (; st0 + 2 * SST - 2 < nst; st0 += SST) {
            sk_for(std::make_integer_sequence<int, SST>{}, [&](auto Q) {
                constexpr int q = decltype(Q)::value;
                constexpr int nq = (q + SST - 1) % SST;
                __builtin_amdgcn_s_waitcnt(swait_vm(SOPS * (SST - 2)));
                __builtin_amdgcn_s_barrier();
                issue(st0 + q + SST - 1, std::integral_constant<int, nq>{}, xb[nq]);
                compute(st0 + q, Q, xb[q]);
            });
        }
        for (; st0 < nst; st0 += SST) {
            sk_for(std::make_integer_sequence<int, SST>{}, [&](auto Q) {
                constexpr int q = decltype(Q)::value;
                const int64_t st = st0 + q;
                if (st < nst) {
                    if (nst - 1 - st >= SST - 2)
                        __builtin_amdgcn_s_waitcnt(swait_vm(SOPS * (SST - 2)));
                    else
                        __builtin_amdgcn_s_waitcnt(swait_vm(0));
                    __builtin_amdgcn_s_barrier();
                    constexpr int nq = (q + SST - 1) % SST;
                    if (st + SST - 1 < nst) issue(st + SST - 1, std::integral_constant<int, nq>{}, xb[nq]);
                    compute(st, Q, xb[q]);
                }
            });
        }
        __syncthreads();
        f32x4* part = reinterpret_cast<f32x4*>(ring0);  // NXF * 3 KiB of the 16 KiB stage
        static_assert(NXF * (SWaves - 1) * kWave * 16 <= 16 * SROW, "partials fit one stage");
        if (wave > 0) {
#pragma unroll
            for (int f = 0; f < NXF; ++f) part[(f * (SWaves - 1) + wave - 1) * kWave + lane] = acc[f];
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int f = 0; f < NXF; ++f) {
                f32x4 sum = acc[f];
#pragma unroll
                for (int w = 0; w < SWaves - 1; ++w) sum += part[(f * (SWaves - 1) + w) * kWave + lane];
                // Lane holds out(x_row = 16 f + lane % 16, w_row = w0 + 4 * (lane / 16) + q).
                const int xr = 16 * f + r;
                if (xr < a.nx) {
                    S* o = static_cast<S*>(a.out) + b * a.so + (int64_t)xr * a.out_sx;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int64_t ow = w0 + 4 * g + q;
                        if (ow < a.nw) o[ow * a.out_sw] = axpby<T>(sum[q], a.alpha, a.beta, o + ow * a.out_sw);
                    }
                }
            }
        }
        __syncthreads();
    }
}
#undef MM_LDSP

}  // namespace

hipError_t launch_gemv_wide(const SkinnyArgs& a, hipStream_t s, Launched* L) {
    void* args[] = {const_cast<SkinnyArgs*>(&a)};
    const dim3 grid((unsigned)((a.nw + 15) / 16), (unsigned)(a.batch < 65535 ? a.batch : 65535));
    // One activation fragment per 16 rows (up to four: 64 rows).
    const int nxf = (int)((a.nx + 15) / 16);
#define MM_SW(T) (nxf == 1 ? reinterpret_cast<const void*>(&gemv_wide<T, 1>)   \
                  : nxf == 2 ? reinterpret_cast<const void*>(&gemv_wide<T, 2>) \
                  : nxf == 3 ? reinterpret_cast<const void*>(&gemv_wide<T, 3>) \
                             : reinterpret_cast<const void*>(&gemv_wide<T, 4>))
    const void* fn = a.dtype == 0 ? MM_SW(TF32) : a.dtype == 1 ? MM_SW(TF16) : MM_SW(TBF16);
#undef MM_SW
    L->kernel = MM_KERNEL_GEMV_WIDE;
    L->variant = nxf;
    return hipLaunchKernel(fn, grid, dim3(SThreads), args, 0, s);
}

}  // namespace mmk
