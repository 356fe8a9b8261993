// Skinny route: C = A . B^T with only a few (2..16) rows on one side, both
// operands stored with rows along the contraction (tract-metal 0.23.6
// mlx_gemm/mod.rs, `gemv_wide_config` and `dispatch_metal_mlx_gemv_wide`: a
// padded GEMM tile would waste most of its rows, so the weight block is
// streamed once for all activation rows).
//
// Roles: W is the operand with many rows (streamed from HBM once), X the one
// with at most 16 rows (re-read from L2). out(x_row, w_row) lands at
// out[x_row * out_sx + w_row * out_sw], which covers both C = X . W^T
// (X = A) and C = W . X^T (W = A).
//
// One block computes one 16 x 16 MFMA fragment: 16 weight rows against all
// activation rows (padded to 16 by repeating the last one; padded results
// are never stored; rows past the end repeat the last row the same way). Per contraction step of four 16-byte chunks, lane l
// loads chunk (l / 16) of weight row l % 16 and of activation row l % 16 and
// feeds them to one MFMA (f16/bf16: 16x16x32; f32: four 16x16x4, component q
// of every lane's chunk being contraction slot q for both operands). The
// four waves take steps w, w + 4, w + 8, ..., so at any moment a block reads
// 256 contiguous bytes of each of its 16 rows; each wave keeps SD steps in
// flight. The four partial fragments are summed in a fixed order through LDS.
// HBM-bound: ~M FLOP per weight byte, far below the MFMA ridge.
#include "common.hpp"
#include "kernels.hpp"

namespace mmk {

namespace {

constexpr int SThreads = 256;
constexpr int SWaves = SThreads / kWave;
constexpr int SD = 8;  // steps in flight per wave

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
// every 16-byte chunk is then wholly inside a row or wholly past its end, and
// a chunk that must not contribute is read through an offset past the buffer
// resource's range, which returns zeros without touching memory.
template <class T>
__global__ __launch_bounds__(SThreads) void gemv_wide(SkinnyArgs a) {
    using S = typename T::store_t;
    constexpr int CH = T::Elems16;
    constexpr uint32_t kOff = 0x80000000u;  // past every resource range
    __shared__ f32x4 part[SWaves - 1][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int r = lane & 15, g = lane >> 4;
    const int64_t w0 = (int64_t)blockIdx.x * 16;
    const int64_t wrow = w0 + r < a.nw ? w0 + r : a.nw - 1;
    const int64_t xrow = r < a.nx ? r : a.nx - 1;
    const int64_t nch = a.k / CH;           // 16-byte chunks per row
    const int64_t ns = (nch + 3) / 4;       // contraction steps
    const int64_t mine = ns > wave ? (ns - wave + SWaves - 1) / SWaves : 0;
    const uint32_t wbyte = (uint32_t)(wrow * a.ldw * (int64_t)sizeof(S));
    const uint32_t xbyte = (uint32_t)(xrow * a.ldx * (int64_t)sizeof(S));
    for (int64_t b = blockIdx.y; b < a.batch; b += gridDim.y) {
        const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<S*>(static_cast<const S*>(a.W) + b * a.sw), (short)0, (int)a.w_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<S*>(static_cast<const S*>(a.X) + b * a.sx), (short)0, (int)a.x_bytes, 0x00020000);
        // The i-th step of this wave: lane chunk 4 s + g, zeros when past the
        // row end or past this wave's steps.
        auto load = [&](int64_t i, u32x4& wv, u32x4& xv) {
            const int64_t c = 4 * (wave + (int64_t)SWaves * i) + g;
            const bool live = i < mine && c < nch;
            const uint32_t cb = (uint32_t)(c * 16);
            wv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     wrs, live ? wbyte + cb : kOff, 0, 0));
            xv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     xrs, live ? xbyte + cb : kOff, 0, 0));
        };
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        u32x4 wv[SD], xv[SD];
#pragma unroll
        for (int j = 0; j < SD; ++j) load(j, wv[j], xv[j]);
        for (int64_t i0 = 0; i0 < mine; i0 += SD) {
#pragma unroll
            for (int j = 0; j < SD; ++j) {
                acc = frag_mma<T>(wv[j], xv[j], acc);
                load(i0 + j + SD, wv[j], xv[j]);
            }
        }
        if (wave > 0) part[wave - 1][lane] = acc;
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int w = 0; w < SWaves - 1; ++w) acc += part[w][lane];
            // Lane holds out(x_row = lane % 16, w_row = w0 + 4 * (lane / 16) + q).
            if (r < a.nx) {
                S* o = static_cast<S*>(a.out) + b * a.so + (int64_t)r * a.out_sx;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t ow = w0 + 4 * g + q;
                    if (ow < a.nw) o[ow * a.out_sw] = narrow(T{}, acc[q]);
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_gemv_wide(const SkinnyArgs& a, hipStream_t s, int* kernel) {
    void* args[] = {const_cast<SkinnyArgs*>(&a)};
    const dim3 grid((unsigned)((a.nw + 15) / 16), (unsigned)(a.batch < 65535 ? a.batch : 65535));
    const void* fn = a.dtype == 0   ? reinterpret_cast<const void*>(&gemv_wide<TF32>)
                     : a.dtype == 1 ? reinterpret_cast<const void*>(&gemv_wide<TF16>)
                                    : reinterpret_cast<const void*>(&gemv_wide<TBF16>);
    *kernel = MM_KERNEL_GEMV_WIDE;
    return hipLaunchKernel(fn, grid, dim3(SThreads), args, 0, s);
}

}  // namespace mmk
