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

// Argument blocks of the chunked MFMA path (bf16 operands, P = 64, N = 128,
// chunk % 64 == 0).
struct SsdFwdArgs {
    int64_t Bsz, T;
    int H, G;
    int64_t L, nchunks;
    const void *x, *B, *C;
    const float *dt, *A, *D, *h0;
    void *y;
    float *h_final, *chunk_states;
};

struct SsdBwdArgs {
    int64_t Bsz, T;
    int H, G;
    int64_t L, nchunks;
    const void *x, *B, *C, *dy;
    const float *dt, *A, *D, *chunk_states, *dh_final;
    void *dx;
    float *dB, *dC, *ddt, *dA, *dD, *dh0;
    // workspace
    bf16_t *dstates;  // [Bsz, H, nchunks, 64 x 128]: gradient on the state leaving chunk c, in bf16,
                      // in pairs of 16 x 16 tiles in accumulator lane order (dstate_pair)
    double *pA, *pD;  // [Bsz, H, nchunks, chunk/64] per-block partials of dA, dD
};

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

// Fragment of a row-major [16 x K] operand tile: 8 consecutive K of row l%16.
__device__ __forceinline__ bf16x8 frag_row(const bf16_t *rowk) {
    return *reinterpret_cast<const bf16x8 *>(rowk);
}

// Fragment of the operand A[r][k] = T[k][r] read from a row-major [K][R] LDS
// tile T (row stride ld elements) with gfx950's transposing LDS read: within a
// 16-lane group, lane i receives element i%4 of the 8-byte chunks addressed by
// lanes i/4, i/4+4, i/4+8, i/4+12.  Lane j of group g therefore addresses row
// k0 + 8g + j/4, columns r0 + 4(j%4) .. +3, and lane i gets T[k0+8g+m][r0+i],
// m = 0..3; a second read 4 rows further down supplies m = 4..7.
__device__ __forceinline__ bf16x8 frag_tr(const bf16_t *T, int ld, int r0, int k0, int lane) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const int g = lane >> 4, j = lane & 15;
    const bf16_t *p = T + (k0 + 8 * g + (j >> 2)) * ld + r0 + 4 * (j & 3);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)p);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p + 4 * ld));
    const v4i16 both[2] = {lo, hi};
    return *reinterpret_cast<const bf16x8 *>(both);
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// Dispatch places workgroup i on XCD i % 8; hand each XCD a contiguous range
// of logical ids so that neighbouring ids (the heads of one group, the blocks
// of one chunk) share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int i, int n) {
    if ((n & 7) != 0) return i;
    return (i & 7) * (n >> 3) + (i >> 3);
}

// Raw buffer access over one chunk's rows.  The hardware range-checks the per-lane
// byte offset against `bytes`: reads at or past it return zero and writes there are
// dropped, so ragged tails need no branches.  The scalar offset is always 0 (it is
// not part of the check).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ u16x8 buf_ld_16b(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u16x4 buf_ld_8b(rsrc_t r, uint32_t off) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(u16x4, __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0)));
}
__device__ __forceinline__ float buf_ld_f32(rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void buf_st_8b(rsrc_t r, uint32_t off, u16x4 v) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, 0);
}
__device__ __forceinline__ void buf_st_16b(rsrc_t r, uint32_t off, u16x8 v) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
}
__device__ __forceinline__ void buf_st_f32(rsrc_t r, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}

__device__ __forceinline__ u16x4 pack4(float a, float b, float c, float d) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 w = {pack2_bf16(a, b), pack2_bf16(c, d)};
    return __builtin_bit_cast(u16x4, w);
}

}  // namespace ssm
