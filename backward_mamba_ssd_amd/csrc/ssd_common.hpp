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
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 w = {pack2_bf16(a, b), pack2_bf16(c, d)};
    return __builtin_bit_cast(u16x4, w);
}

// Staging thread maps (256 threads).  Transposed LDS writes are the bank-hot
// accesses; these maps spread one wave's lanes over all 64 banks.
//  [tok][p] source rows -> [p][tok] tile: thread covers 2 tokens x 8 channels,
//  lanes of a wave vary the token pair (32 pairs) and 2 channel blocks.
__device__ __forceinline__ int map64_tok(int tid) { return 2 * (tid & 31); }
__device__ __forceinline__ int map64_col(int tid) { return 8 * ((tid >> 5) & 1) + 16 * (tid >> 6); }
//  [tok][n] source rows -> [n][tok] tile: thread covers 4 tokens x 8 coords,
//  lanes vary the token quad (16 quads) and 4 coordinate blocks.
__device__ __forceinline__ int map128_tok(int tid) { return 4 * (tid & 15); }
__device__ __forceinline__ int map128_col(int tid) { return 8 * ((tid >> 4) & 3) + 32 * (tid >> 6); }

}  // namespace ssm
