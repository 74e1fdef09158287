// common.hpp -- device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

typedef uint16_t bf16_t;  // bf16 storage (upper half of a float32)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// float32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// Two floats -> two bf16 packed in one dword (low half = a), one instruction.
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

// Scalar load/store of a storage dtype as float.
template <typename T> struct IO;
template <> struct IO<float> {
    static __device__ __forceinline__ float ld(const float *p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void st(float *p, int64_t i, float v) { p[i] = v; }
    // four consecutive values
    static __device__ __forceinline__ float4 ld4(const float *p, int64_t i) {
        return *reinterpret_cast<const float4 *>(p + i);
    }
};
template <> struct IO<bf16_t> {
    static __device__ __forceinline__ float ld(const bf16_t *p, int64_t i) {
        return bf16_to_f32(p[i]);
    }
    static __device__ __forceinline__ void st(bf16_t *p, int64_t i, float v) {
        p[i] = f32_to_bf16(v);
    }
    static __device__ __forceinline__ float4 ld4(const bf16_t *p, int64_t i) {
        const u16x4 v = *reinterpret_cast<const u16x4 *>(p + i);
        return make_float4(bf16_to_f32(v[0]), bf16_to_f32(v[1]), bf16_to_f32(v[2]),
                           bf16_to_f32(v[3]));
    }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

}  // namespace ssm
