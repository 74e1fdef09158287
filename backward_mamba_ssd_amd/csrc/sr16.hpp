// sr16.hpp -- device side of the FP16 stochastic rounding used by the checkpoint
// kernel and by the decode step with an FP16 state cache.
//
// Rule ("Nemotron 3 Ultra: replaying a rounded state", section "Stochastic
// rounding and the mean state"): between two binary16 neighbours the value goes
// to the upper one exactly when the entropy residue is smaller than the discarded
// remainder.  The remainder is read off the float32 bit fields: the float32
// significand, shifted onto the binary16 grid of its binade, splits into the kept
// integer k and the discarded bits; R = discarded bits scaled to 32 bits (floor),
// and k+1 is taken iff u < R.
//
// The entropy word u is keyed by (seed, key, element): for element e, the high (e even)
// or low (e odd) 32 bits of output floor(e / 2) of a SplitMix64 stream (Steele, Lea &
// Flood 2014) whose seed is output `key` of the stream seeded with `seed`; output k of
// a stream seeded with s is mix64(s + (k+1)*gamma) with SplitMix64's published
// finaliser and gamma.
#pragma once

#include "common.hpp"

namespace ssm {

typedef _Float16 h16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

// The same rule in the binary16 normal range, 2^-14 <= |v| < 65536 (float32 biased
// exponent 113..142), on the float32 bit pattern directly.  There the kept integer and
// the 13 discarded bits d are the top and bottom of the magnitude's bits, R = d << 19,
// and u < R holds exactly when (u >> 19) < d, that is when adding 8191 - (u >> 19) to
// the magnitude carries out of the 13 discarded bits.  So the result is
// sign | (((mag + 8191 - (u >> 19)) >> 13) - (112 << 10)): the exponent is rebiased by
// the subtraction, and a carry moves to the next binade by itself, from the top binade
// to 0x7C00 (infinity), as in sr16_bits.  Bit for bit equal to sr16_bits on that range.
__host__ __device__ __forceinline__ bool sr16_in_normal_range(float v) {
    return ((__builtin_bit_cast(uint32_t, v) & 0x7FFFFFFFu) - 0x38800000u) < 0x0F000000u;
}
__host__ __device__ __forceinline__ uint16_t sr16_bits_normal(float v, uint32_t u) {
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    const uint32_t mag = b & 0x7FFFFFFFu;
    const uint32_t r = ((mag + (8191u - (u >> 19))) >> 13) - (112u << 10);
    return static_cast<uint16_t>(((b >> 16) & 0x8000u) | r);
}

// The rule for any float32: the short form in the binary16 normal range (almost every
// value of a state), the general one for the rest (a wave skips either branch when none
// of its lanes needs it).
__host__ __device__ __forceinline__ uint16_t sr16_bits_general(float v, uint32_t u);
__host__ __device__ __forceinline__ uint16_t sr16_bits(float v, uint32_t u) {
    if (sr16_in_normal_range(v)) return sr16_bits_normal(v, u);
    return sr16_bits_general(v, u);
}

__host__ __device__ __forceinline__ uint16_t sr16_bits_general(float v, uint32_t u) {
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    const uint32_t sign = (b >> 16) & 0x8000u;
    const uint32_t mag = b & 0x7FFFFFFFu;
    if (mag > 0x7F800000u) return static_cast<uint16_t>(sign | 0x7E00u);  // NaN
    if (mag >= 0x47800000u) return static_cast<uint16_t>(sign | 0x7C00u); // >= 65536, Inf
    // One form for both binary16 ranges.  The float32 significand (24 bits) is shifted
    // onto the binary16 grid of its binade: by 13 bits in the normal range (biased
    // float32 exponent e >= 113) and by 126 - e bits below it (spacing 2^-24).  k is
    // the kept integer, R the discarded bits scaled to 32 bits (floor; 0 once the shift
    // reaches 56, i.e. remainder < 2^-32, and for zeros and float32 subnormals, e = 0);
    // k + 1 is taken iff u < R.  The result is the exponent field (e - 113 in the
    // normal range, 0 below) shifted by 10 plus k, so that k = 2048 carries into the
    // next binade and into infinity at the top, and k = 1024 below the normal range is
    // the smallest normal's bit pattern.  (The rare cases stay branches: a wave skips
    // them when none of its lanes needs them.)
    const uint32_t e = mag >> 23;
    const uint32_t sig = (mag & 0x7FFFFFu) | 0x800000u;
    const bool normal = e >= 113u;
    const uint32_t es = normal ? e - 113u : 0u;
    const uint32_t sh = normal ? 13u : 126u - e;
    const uint32_t k = sh >= 32u ? 0u : (sig >> sh);
    const uint32_t R = sh >= 56u ? 0u : (sh <= 32u ? (sig << (32u - sh)) : (sig >> (sh - 32u)));
    return static_cast<uint16_t>(sign | ((es << 10) + k + (u < R ? 1u : 0u)));
}

// Entropy words: output k of the sub-stream sub = sr16_stream(seed, key) serves the two
// elements 2k (its high 32 bits) and 2k + 1 (its low 32 bits), so one 64-bit finaliser
// (six 32-bit multiplies at a quarter of the vector rate) covers two elements.
__device__ __forceinline__ uint64_t sr16_stream(uint64_t seed, uint64_t key) {
    return sm64_mix(seed + (key + 1ull) * kGamma);
}
__device__ __forceinline__ uint32_t sr16_entropy(uint64_t sub, uint64_t e) {
    const uint64_t r = sm64_mix(sub + ((e >> 1) + 1ull) * kGamma);
    return (e & 1ull) ? static_cast<uint32_t>(r) : static_cast<uint32_t>(r >> 32);
}
// u for the K consecutive elements e .. e+K-1 (K even): the stream counter advances by
// one gamma per output, so only the first needs a 64-bit multiply.  e is even wherever
// the kernels call this with a whole run (rows of an even state width); an odd e takes
// the general path.
template <int K>
__device__ __forceinline__ void sr16_entropy_run(uint64_t sub, uint64_t e, uint32_t (&u)[K]) {
    static_assert(K % 2 == 0, "runs of whole outputs");
    if ((e & 1ull) == 0) {
        uint64_t z = sub + ((e >> 1) + 1ull) * kGamma;
#pragma unroll
        for (int j = 0; j < K; j += 2) {
            const uint64_t r = sm64_mix(z);
            u[j] = static_cast<uint32_t>(r >> 32);
            u[j + 1] = static_cast<uint32_t>(r);
            z += kGamma;
        }
    } else {
#pragma unroll
        for (int j = 0; j < K; ++j) u[j] = sr16_entropy(sub, e + j);
    }
}

}  // namespace ssm
