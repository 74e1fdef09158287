// ssd_common.hpp -- shapes, LDS strides and the MFMA tile primitive shared by
// the chunked forward and backward kernels (headdim 64, dstate 128).
//
// MFMA operand convention ("NT" tiles): both operands are row-major [16 x K]
// bf16 tiles in LDS with K contiguous.  Lane l supplies row l%16, elements
// 8*(l/16) .. 8*(l/16)+7 of each 32-wide K step; the accumulator lane holds
// D[m = 4*(l/16) + v][n = l%16] for v = 0..3, where D = A_tile * B_tile^T.
#pragma once

#include "common.hpp"

namespace ssm {

constexpr int kP = 64;          // value channels per head
constexpr int kN = 128;         // state coordinates
constexpr int kLs = 64;         // tokens per block
constexpr int kS128 = kN + 8;   // LDS row stride (elements) of 128-wide rows
constexpr int kS64 = kLs + 8;   // LDS row stride (elements) of 64-wide rows

__device__ __forceinline__ f32x4 mma16(const bf16_t *a, const bf16_t *b, f32x4 acc) {
    const bf16x8 av = *reinterpret_cast<const bf16x8 *>(a);
    const bf16x8 bv = *reinterpret_cast<const bf16x8 *>(b);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
}

// Dispatch places workgroup i on XCD i % 8; hand each XCD a contiguous range
// of logical ids so that neighbouring ids (the heads of one group, the blocks
// of one chunk) share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int i, int n) {
    if ((n & 7) != 0) return i;
    return (i & 7) * (n >> 3) + (i >> 3);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_prefix_sum(float v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    return v;
}

__device__ __forceinline__ u16x4 pack4(float a, float b, float c, float d) {
    u16x4 v;
    v[0] = f32_to_bf16(a);
    v[1] = f32_to_bf16(b);
    v[2] = f32_to_bf16(c);
    v[3] = f32_to_bf16(d);
    return v;
}

}  // namespace ssm
