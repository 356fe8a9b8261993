// Device-side helpers shared by the gfx950 kernels: storage types, exact
// widening, nearest-even narrowing, 16-byte global loads and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// Storage tags. `Elems16` is how many elements one 16-byte load carries.
struct TF32 {
    using store_t = float;
    static constexpr int code = 0;
    static constexpr int Elems16 = 4;
};
struct TF16 {
    using store_t = uint16_t;
    static constexpr int code = 1;
    static constexpr int Elems16 = 8;
};
struct TBF16 {
    using store_t = uint16_t;
    static constexpr int code = 2;
    static constexpr int Elems16 = 8;
};

// ---- exact widening --------------------------------------------------------
__device__ __forceinline__ float widen(TF32, float x) { return x; }
__device__ __forceinline__ float widen(TF16, uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ float widen(TBF16, uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

// ---- nearest-even narrowing of an f32 result ------------------------------
__device__ __forceinline__ float narrow(TF32, float x) { return x; }
__device__ __forceinline__ uint16_t narrow(TF16, float x) {
    // v_cvt_f16_f32 rounds with the MODE register's default: nearest even.
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ __forceinline__ uint16_t narrow(TBF16, float x) {
    // v_cvt_pk_bf16_f32 (gfx950) rounds to nearest even as well; NaN stays NaN.
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// ---- output epilogue: alpha * acc + beta * C_old, rounded once ---------------
// beta == 0 never reads the old value (its contents, NaN included, do not
// matter); alpha == 1, beta == 0 returns exactly narrow(acc).
template <class T>
__device__ __forceinline__ typename T::store_t axpby(float acc, float alpha, float beta,
                                                     const typename T::store_t* old) {
    const float v = beta != 0.f ? __builtin_fmaf(alpha, acc, beta * widen(T{}, *old)) : alpha * acc;
    return narrow(T{}, v);
}

// ---- unpack a 16-byte chunk into f32 ---------------------------------------
// 8 x 16-bit elements -> 8 floats (exact).
__device__ __forceinline__ void unpack8(TF16, u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = widen(TF16{}, (uint16_t)(v[i] & 0xffffu));
        f[2 * i + 1] = widen(TF16{}, (uint16_t)(v[i] >> 16));
    }
}
__device__ __forceinline__ void unpack8(TBF16, u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(v[i] << 16);
        f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
}
// 4 x f32
__device__ __forceinline__ void unpack4(u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
}

// ---- loads -------------------------------------------------------------------
__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// ---- wave reductions -----------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Element load through a storage tag (scalar paths).
template <class T>
__device__ __forceinline__ float load_elem(const typename T::store_t* p, int64_t i) {
    return widen(T{}, p[i]);
}

}  // namespace mmk
