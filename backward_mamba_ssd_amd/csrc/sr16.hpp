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
// The entropy word u is keyed by (seed, key, element): u = high 32 bits of output e
// of a SplitMix64 stream (Steele, Lea & Flood 2014) whose seed is output `key` of
// the stream seeded with `seed`; output k of a stream seeded with s is
// mix64(s + (k+1)*gamma) with SplitMix64's published finaliser and gamma.
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

__device__ __forceinline__ uint16_t sr16_bits(float v, uint32_t u) {
    const uint32_t b = __float_as_uint(v);
    const uint32_t sign = (b >> 16) & 0x8000u;
    const uint32_t mag = b & 0x7FFFFFFFu;
    if (mag > 0x7F800000u) return static_cast<uint16_t>(sign | 0x7E00u);  // NaN
    if (mag >= 0x47800000u) return static_cast<uint16_t>(sign | 0x7C00u); // >= 65536, Inf
    const uint32_t e = mag >> 23;             // biased float32 exponent
    if (e == 0) return static_cast<uint16_t>(sign);  // zero / float32 subnormal: R = 0
    const uint32_t sig = (mag & 0x7FFFFFu) | 0x800000u;  // 24-bit significand
    uint32_t k, R;
    if (e >= 113) {
        // binary16 normal binade: spacing 2^(e-127-10); 13 discarded bits
        k = sig >> 13;
        R = (sig & 0x1FFFu) << 19;
        k += (u < R) ? 1u : 0u;
        // exponent field (e-112) and mantissa (k-1024); k == 2048 carries into
        // the next binade and into infinity (0x7C00) at the top.
        return static_cast<uint16_t>(sign | (((e - 112u) << 10) + (k - 1024u)));
    }
    // binary16 subnormal range: spacing 2^-24; shift = 126 - e >= 14
    const uint32_t sh = 126u - e;
    if (sh >= 56u) return static_cast<uint16_t>(sign);  // remainder < 2^-32: never up
    k = (sh >= 32u) ? 0u : (sig >> sh);
    uint64_t rem = static_cast<uint64_t>(sig) & ((1ull << sh) - 1ull);
    R = static_cast<uint32_t>(sh <= 32u ? (rem << (32u - sh)) : (rem >> (sh - 32u)));
    k += (u < R) ? 1u : 0u;  // k <= 1024: 1024 is the smallest normal's bit pattern
    return static_cast<uint16_t>(sign | k);
}

// u for element e under (seed, key): sub = sr16_stream(seed, key) once per call
__device__ __forceinline__ uint64_t sr16_stream(uint64_t seed, uint64_t key) {
    return sm64_mix(seed + (key + 1ull) * kGamma);
}
__device__ __forceinline__ uint32_t sr16_entropy(uint64_t sub, uint64_t e) {
    return static_cast<uint32_t>(sm64_mix(sub + (e + 1ull) * kGamma) >> 32);
}

}  // namespace ssm
