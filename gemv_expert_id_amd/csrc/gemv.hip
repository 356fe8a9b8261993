// GEMV route: out = M . v, the m == 1 or n == 1 case of C = op(A).op(B)
// (tract-metal 0.23.6 mlx_gemm/mod.rs, `dispatch_metal_mlx_gemv`: the
// matrix operand is B when n != 1 and A otherwise; the "transposed" kernel
// handles a matrix whose outputs are contiguous).
//
// HBM-bound: every matrix byte is read once. Row form (outputs along rows that
// are contiguous in the contraction index): each wave owns one row, lanes pull
// it as non-temporal 16-byte chunks with eight loads in flight, and a
// wave-wide shuffle reduction finishes the row.
// Column form (outputs contiguous): lanes own 16-byte runs of outputs, the
// four waves of a block split the contraction, and LDS sums their partials in
// a fixed order. No MFMA: the arithmetic intensity is ~1 FLOP/byte.
#include "common.hpp"
#include "kernels.hpp"

namespace mmk {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <class T>
__device__ __forceinline__ void unpack(u32x4 v, float* f) {
    if constexpr (T::Elems16 == 8)
        unpack8(T{}, v, f);
    else
        unpack4(v, f);
}

template <class T>
__device__ __forceinline__ void store_out(const GemvArgs& a, int64_t idx, float v) {
    using S = typename T::store_t;
    S* o = reinterpret_cast<S*>(a.out) + idx;
    *o = axpby<T>(v, a.alpha, a.beta, o);
}

// Row form with 16-byte loads. Requires k % Elems16 == 0, ld and the batch
// strides multiples of Elems16, 16-byte aligned bases and vec_inc == 1.
// Each lane issues U independent 16-byte loads per row before using any;
// the remainder of the row is walked with 4, 2 and then 1 loads in flight.
template <class T, int R, int UU>
__device__ __forceinline__ void rows_chunk(const typename T::store_t* const* rowp,
                                           const typename T::store_t* vec, int64_t c,
                                           float* acc) {
    constexpr int CH = T::Elems16;
    u32x4 xv[UU], wv[R][UU];
#pragma unroll
    for (int u = 0; u < UU; ++u) xv[u] = ld16(vec + (c + kWave * u) * CH);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int u = 0; u < UU; ++u) wv[r][u] = ld16_stream(rowp[r] + (c + kWave * u) * CH);
#pragma unroll
    for (int u = 0; u < UU; ++u) {
        float xf[CH];
        unpack<T>(xv[u], xf);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float wf[CH];
            unpack<T>(wv[r][u], wf);
#pragma unroll
            for (int q = 0; q < CH; ++q) acc[r] = __builtin_fmaf(wf[q], xf[q], acc[r]);
        }
    }
}

template <class T, int R, int U>
__global__ __launch_bounds__(kThreads) void gemv_rows_vec(GemvArgs a) {
    using S = typename T::store_t;
    constexpr int CH = T::Elems16;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t o0 = ((int64_t)blockIdx.x * kWaves + wave) * R;
    if (o0 >= a.rows) return;
    const int64_t nch = a.k / CH;
    for (int64_t b = blockIdx.y; b < a.batch; b += gridDim.y) {
        const S* mat = reinterpret_cast<const S*>(a.mat) + b * a.mat_bstride;
        const S* vec = reinterpret_cast<const S*>(a.vec) + b * a.vec_bstride;
        const S* rowp[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int64_t o = o0 + r < a.rows ? o0 + r : a.rows - 1;
            rowp[r] = mat + o * a.ld;
        }
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.f;

        int64_t c = lane;
        for (; c + kWave * (U - 1) < nch; c += kWave * U) rows_chunk<T, R, U>(rowp, vec, c, acc);
        if (U > 4 && c + kWave * 3 < nch) {
            rows_chunk<T, R, 4>(rowp, vec, c, acc);
            c += kWave * 4;
        }
        if (U > 2 && c + kWave < nch) {
            rows_chunk<T, R, 2>(rowp, vec, c, acc);
            c += kWave * 2;
        }
        for (; c < nch; c += kWave) rows_chunk<T, R, 1>(rowp, vec, c, acc);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (lane == r && o0 + r < a.rows)
                store_out<T>(a, b * a.out_bstride + (o0 + r) * a.out_inc, acc[r]);
    }
}

// Row form, element loads: any k, ld, alignment and vector increment.
template <class T, int R>
__global__ __launch_bounds__(kThreads) void gemv_rows_scalar(GemvArgs a) {
    using S = typename T::store_t;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t o0 = ((int64_t)blockIdx.x * kWaves + wave) * R;
    if (o0 >= a.rows) return;
    for (int64_t b = blockIdx.y; b < a.batch; b += gridDim.y) {
        const S* mat = reinterpret_cast<const S*>(a.mat) + b * a.mat_bstride;
        const S* vec = reinterpret_cast<const S*>(a.vec) + b * a.vec_bstride;
        const S* rowp[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int64_t o = o0 + r < a.rows ? o0 + r : a.rows - 1;
            rowp[r] = mat + o * a.ld;
        }
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.f;
        for (int64_t p = lane; p < a.k; p += kWave) {
            float x = widen(T{}, vec[p * a.vec_inc]);
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = __builtin_fmaf(widen(T{}, rowp[r][p]), x, acc[r]);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (lane == r && o0 + r < a.rows)
                store_out<T>(a, b * a.out_bstride + (o0 + r) * a.out_inc, acc[r]);
    }
}

// Column form: M(o, p) = mat[p * ld + o]. Lanes own VW consecutive outputs
// (VW = Elems16 with 16-byte loads, or 1); wave w sums the w-th quarter of
// the contraction; the four partials are added in wave order through LDS.
template <class T, int VW>
__global__ __launch_bounds__(kThreads) void gemv_cols(GemvArgs a) {
    using S = typename T::store_t;
    __shared__ float part[kWaves][kWave * VW];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t o0 = (int64_t)blockIdx.x * kWave * VW + (int64_t)lane * VW;
    const int64_t kq = (a.k + kWaves - 1) / kWaves;
    const int64_t p_begin = wave * kq;
    const int64_t p_end = p_begin + kq < a.k ? p_begin + kq : a.k;
    for (int64_t b = blockIdx.y; b < a.batch; b += gridDim.y) {
        const S* mat = reinterpret_cast<const S*>(a.mat) + b * a.mat_bstride;
        const S* vec = reinterpret_cast<const S*>(a.vec) + b * a.vec_bstride;
        float acc[VW];
#pragma unroll
        for (int q = 0; q < VW; ++q) acc[q] = 0.f;
        if (o0 < a.rows) {
            const bool full = VW > 1 && o0 + VW <= a.rows;
#pragma unroll 4
            for (int64_t p = p_begin; p < p_end; ++p) {
                const float x = widen(T{}, vec[p * a.vec_inc]);
                const S* src = mat + p * a.ld + o0;
                if constexpr (VW > 1) {
                    if (full) {
                        float wf[VW];
                        unpack<T>(ld16(src), wf);
#pragma unroll
                        for (int q = 0; q < VW; ++q) acc[q] = __builtin_fmaf(wf[q], x, acc[q]);
                        continue;
                    }
                }
#pragma unroll
                for (int q = 0; q < VW; ++q)
                    if (o0 + q < a.rows) acc[q] = __builtin_fmaf(widen(T{}, src[q]), x, acc[q]);
            }
        }
#pragma unroll
        for (int q = 0; q < VW; ++q) part[wave][lane * VW + q] = acc[q];
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int q = 0; q < VW; ++q) {
                const int idx = lane * VW + q;
                float s = part[0][idx];
#pragma unroll
                for (int w = 1; w < kWaves; ++w) s += part[w][idx];
                if (o0 + q < a.rows) store_out<T>(a, b * a.out_bstride + (o0 + q) * a.out_inc, s);
            }
        }
        __syncthreads();
    }
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <class T>
hipError_t launch_typed(const GemvArgs& a, hipStream_t s, Launched* L) {
    constexpr int CH = T::Elems16;
    const unsigned gy = (unsigned)(a.batch < 65535 ? a.batch : 65535);
    void* args[] = {const_cast<GemvArgs*>(&a)};
    if (!a.col_form) {
        const bool vec = a.k % CH == 0 && a.ld % CH == 0 && a.vec_inc == 1 &&
                         a.mat_bstride % CH == 0 && a.vec_bstride % CH == 0 &&
                         aligned16(a.mat) && aligned16(a.vec);
        constexpr int R = 1;  // one row per wave, eight 16-byte loads in flight per lane
        dim3 grid((unsigned)((a.rows + kWaves * R - 1) / (kWaves * R)), gy);
        const void* fn = vec ? reinterpret_cast<const void*>(&gemv_rows_vec<T, R, 8>)
                             : reinterpret_cast<const void*>(&gemv_rows_scalar<T, R>);
        L->kernel = vec ? MM_KERNEL_GEMV_ROWS : MM_KERNEL_GEMV_ROWS_ELEM;
        return hipLaunchKernel(fn, grid, dim3(kThreads), args, 0, s);
    }
    const bool vec = a.ld % CH == 0 && a.mat_bstride % CH == 0 && aligned16(a.mat);
    L->kernel = MM_KERNEL_GEMV_COLS;
    if (vec) {
        dim3 grid((unsigned)((a.rows + kWave * CH - 1) / (kWave * CH)), gy);
        return hipLaunchKernel(reinterpret_cast<const void*>(&gemv_cols<T, CH>), grid,
                               dim3(kThreads), args, 0, s);
    }
    dim3 grid((unsigned)((a.rows + kWave - 1) / kWave), gy);
    return hipLaunchKernel(reinterpret_cast<const void*>(&gemv_cols<T, 1>), grid, dim3(kThreads),
                           args, 0, s);
}

}  // namespace

hipError_t launch_gemv(const GemvArgs& a, hipStream_t s, Launched* L) {
    switch (a.dtype) {
        case 0: return launch_typed<TF32>(a, s, L);
        case 1: return launch_typed<TF16>(a, s, L);
        case 2: return launch_typed<TBF16>(a, s, L);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mmk
