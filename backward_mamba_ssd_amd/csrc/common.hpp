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

// Streaming (nontemporal) 16-byte access for data touched once per call, such as a
// state streamed through HBM: the load does not allocate in L2, which measured ~9%
// more HBM bandwidth for the in-place decode update than ordinary loads.
__device__ __forceinline__ float4 nt_ld4(const float *p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void nt_st4(float *p, const float4 &v) {
    __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4 *>(p));
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

// Cross-lane sums without lane-address registers.  A 64-lane wave is four rows of
// 16 lanes.  Within a row, DPP swaps neighbours (quad_perm 1,0,3,2 and 2,3,0,1), then
// mirrors half-rows and rows; across rows, the gfx950 permlane swaps pair row r with
// r^1 and the half-waves with each other.  Each helper returns the sum in every lane
// it covers; the order of additions is fixed, so results are deterministic.
#define SSM_DPP(v, ctrl) \
    __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, (v)), (ctrl), 0xf, 0xf, false))
// sum over the 16 lanes of the row
__device__ __forceinline__ float row16_sum(float v) {
    v += SSM_DPP(v, 0xB1);   // quad_perm [1,0,3,2]
    v += SSM_DPP(v, 0x4E);   // quad_perm [2,3,0,1]
    v += SSM_DPP(v, 0x141);  // row_half_mirror
    v += SSM_DPP(v, 0x140);  // row_mirror
    return v;
}
// sum over lanes l, l^16, l^32, l^48.  A swap given the same value in both operands
// returns rows (0,0,2,2)/(1,1,3,3) for the 16-lane form and halves (lo,lo)/(hi,hi)
// for the 32-lane form, so the sum of its two results is the pair sum.  The results
// are read with __uint_as_float: __builtin_bit_cast of a subscript of the returned
// pair reads element 0 for both.
__device__ __forceinline__ float swap_pair_sum16(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_pair_sum32(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float rows4_sum(float v) { return swap_pair_sum32(swap_pair_sum16(v)); }
// rows4_sum of two values in one pass: the total of a in rows 0 and 2, of b in rows 1 and
// 3.  The 16-lane swap of (a, b) gives rows (a0, b0, a2, b2) and (a1, b1, a3, b3), whose
// sum pairs the rows of each value; the 32-lane pair sum then adds the halves.
__device__ __forceinline__ float rows4_sum2(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return swap_pair_sum32(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_total(float v) { return rows4_sum(row16_sum(v)); }
#undef SSM_DPP

// Inclusive prefix sum over the wave (lane 0 first) with DPP: row_shr 1, 2, 4, 8
// scan each row of 16 (lanes shifted in from outside the row add zero), then
// row_bcast15 adds row r's total into row r+1 (rows 1, 3) and row_bcast31 adds the
// first half's total into rows 2, 3.
#define SSM_DPP0(v, ctrl, rmask) \
    __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, (v)), (ctrl), (rmask), 0xf, true))
__device__ __forceinline__ float wave_prefix_sum(float v) {
    v += SSM_DPP0(v, 0x111, 0xf);  // row_shr:1
    v += SSM_DPP0(v, 0x112, 0xf);  // row_shr:2
    v += SSM_DPP0(v, 0x114, 0xf);  // row_shr:4
    v += SSM_DPP0(v, 0x118, 0xf);  // row_shr:8
    v += SSM_DPP0(v, 0x142, 0xa);  // row_bcast:15 into rows 1 and 3
    v += SSM_DPP0(v, 0x143, 0xc);  // row_bcast:31 into rows 2 and 3
    return v;
}
#undef SSM_DPP0
// inclusive suffix sum over the wave (lane 63 first): the prefix sum of the
// lane-reversed values, reversed back (row_mirror within rows, then the two
// permlane swaps exchange rows r and 3-r).
__device__ __forceinline__ float lane_reverse(float v) {
    v = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xf, 0xf, false));
    uint32_t u = __float_as_uint(v);
    const auto r32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);  // (lo,lo) / (hi,hi)
    // lane l < 32 takes the upper half, lane l >= 32 the lower half
    const bool lo = (__lane_id() < 32);
    u = lo ? r32[1] : r32[0];
    const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);  // rows (0,0,2,2) / (1,1,3,3)
    const bool even = ((__lane_id() >> 4) & 1) == 0;
    u = even ? r16[1] : r16[0];
    return __uint_as_float(u);
}
__device__ __forceinline__ float wave_suffix_sum(float v) {
    return lane_reverse(wave_prefix_sum(lane_reverse(v)));
}

// Sum / max over aligned groups of W lanes (W = 2, 4, 8, 16, 32, 64); every lane of a
// group gets the group's result, in a fixed order.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
template <int W, bool MAX>
__device__ __forceinline__ float lane_group_reduce(float v) {
    auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
    static_assert(W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "group width");
    v = op(v, dpp_mov<0xB1>(v));                              // quad_perm [1,0,3,2]
    if constexpr (W >= 4) v = op(v, dpp_mov<0x4E>(v));        // quad_perm [2,3,0,1]
    if constexpr (W >= 8) v = op(v, dpp_mov<0x141>(v));       // row_half_mirror
    if constexpr (W >= 16) v = op(v, dpp_mov<0x140>(v));      // row_mirror
    if constexpr (W >= 32) {
        const uint32_t u = __float_as_uint(v);
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        v = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    if constexpr (W >= 64) {
        const uint32_t u = __float_as_uint(v);
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        v = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    return v;
}

}  // namespace ssm
