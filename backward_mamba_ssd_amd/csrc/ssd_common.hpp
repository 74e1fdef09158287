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

// ---------------------------------------------------------------------------
// Unpadded LDS tiles with permuted 16-byte pieces.  Row r of a 64 x W bf16 tile keeps
// its piece c (columns 8c .. 8c + 7) at piece c ^ (r % 16) when W = 128 and at
// c ^ ((r / 2) % 8) when W = 64.  Measured on gfx950 (256 workgroups of 8 waves issuing
// back to back), per wave instruction: the 128-bit row-fragment reads (16 rows x 4
// pieces) take 4.7 cycles, against 8.9 with rows padded by one piece; the transposing
// reads stay at their 5-cycle floor; 8-byte accesses down 16 rows of one column share
// banks two ways, as with the padded rows (no piece permutation does better there).
//
// Every access form reduces to a per-lane byte offset combined with constants: the
// fragment index enters by XOR (it only moves pieces within a row) and the row block by
// addition.  SwzLane holds the per-lane offsets for lane l (lr = l % 16, l4 = l / 16;
// frag_tr's map: lane (g, j) = (l / 16, l % 16) reads row 8g + j/4, column 4 (j % 4)).
struct SwzLane {
    uint32_t row64, row128;  // frag_row: row lr, piece l4
    uint32_t tr64, tr128;    // frag_tr, tile 0, k0 = 0, first of its two reads
    uint32_t pc64, pc128;    // 8-byte piece: row lr, columns 4 l4 .. 4 l4 + 3
};
__device__ __forceinline__ SwzLane swz_lane(int lane) {
    const uint32_t lr = lane & 15, l4 = lane >> 4, j = lane & 15, g = lane >> 4;
    const uint32_t b1 = (j >> 1) & 1, trow = 8 * g + (j >> 2);
    SwzLane s;
    s.row64 = lr * 128 + ((l4 ^ (lr >> 1)) << 4);
    s.row128 = lr * 256 + ((l4 ^ lr) << 4);
    s.tr64 = trow * 128 + ((b1 ^ ((trow >> 1) & 7)) << 4) + (j & 1) * 8;
    s.tr128 = trow * 256 + ((b1 ^ (trow & 15)) << 4) + (j & 1) * 8;
    s.pc64 = lr * 128 + (((l4 >> 1) ^ (lr >> 1)) << 4) + (l4 & 1) * 8;
    s.pc128 = lr * 256 + (((l4 >> 1) ^ lr) << 4) + (l4 & 1) * 8;
    return s;
}
// byte offsets within a swizzled tile
// frag_row of rows 16 t .. 16 t + 15, K columns 32 kk .. 32 kk + 31
__device__ __forceinline__ uint32_t swz_row64(const SwzLane &s, int t, int kk) { return t * 2048 + (s.row64 ^ (kk << 6)); }
__device__ __forceinline__ uint32_t swz_row128(const SwzLane &s, int t, int kk) { return t * 4096 + (s.row128 ^ (kk << 6)); }
// 8-byte piece of rows 16 t .. 16 t + 15, columns 16 w .. 16 w + 15
__device__ __forceinline__ uint32_t swz_pc64(const SwzLane &s, int t, int w) { return t * 2048 + (s.pc64 ^ (w << 5)); }
__device__ __forceinline__ uint32_t swz_pc128(const SwzLane &s, int t, int w) { return t * 4096 + (s.pc128 ^ (w << 5)); }
// the row-staging piece: row r, piece c (c < W / 8)
__device__ __forceinline__ uint32_t swz_stage64(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }
__device__ __forceinline__ uint32_t swz_stage128(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }

__device__ __forceinline__ bf16x8 lds_frag(const bf16_t *tile, uint32_t off) {
    return *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const char *>(tile) + off);
}
__device__ __forceinline__ bf16x8 lds_frag_tr(const bf16_t *tile, uint32_t lo, uint32_t hi) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const char *b = reinterpret_cast<const char *>(tile);
    const v4i16 l = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(b + lo));
    const v4i16 h = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(b + hi));
    const v4i16 both[2] = {l, h};
    return *reinterpret_cast<const bf16x8 *>(both);
}
// frag_tr of a swizzled tile: operand rows 16 tile .. 16 tile + 15 (tile columns), K rows
// 32 kk .. 32 kk + 31 (the second read, 4 rows down, moves the lane's piece by 2 within a
// 64-wide row and by 4 within a 128-wide one)
__device__ __forceinline__ bf16x8 frag_tr64(const bf16_t *T, const SwzLane &s, int tile, int kk) {
    return lds_frag_tr(T, kk * 4096 + (s.tr64 ^ (tile << 5)), kk * 4096 + 512 + (s.tr64 ^ ((tile ^ 1) << 5)));
}
__device__ __forceinline__ bf16x8 frag_tr128(const bf16_t *T, const SwzLane &s, int tile, int kk) {
    return lds_frag_tr(T, kk * 8192 + (s.tr128 ^ (tile << 5)), kk * 8192 + 1024 + (s.tr128 ^ ((tile ^ 2) << 5)));
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
