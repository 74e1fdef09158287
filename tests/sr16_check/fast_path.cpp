// Host check that the binary16-normal-range shortcut of the SR16 rounding
// (sr16_bits_normal in csrc/sr16.hpp) gives the bits of the general rule (sr16_bits_general)
// wherever it is used (2^-14 <= |v| < 65536).  In that range the result depends on
// the sign, the top 10 significand bits with the exponent (which set where a carry
// goes), the 13 discarded bits d and the top 13 bits of u; the check is exhaustive in
// (d, u >> 19) for both signs at every exponent's first and last significand value
// (the binade carries, including the one into infinity), with the low 19 bits of u at
// both extremes, and random over the whole range otherwise.  Exit status 0 when all
// agree.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "sr16.hpp"

namespace {

float from_bits(uint32_t b) {
    float f;
    std::memcpy(&f, &b, 4);
    return f;
}

uint64_t state = 0x243F6A8885A308D3ull;
uint32_t next32() {  // xorshift64*, a test-side draw only
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return static_cast<uint32_t>((state * 0x2545F4914F6CDD1Dull) >> 32);
}

}  // namespace

int main() {
    long long checked = 0, bad = 0;
    auto check = [&](uint32_t bits, uint32_t u) {
        const float v = from_bits(bits);
        if (!ssm::sr16_in_normal_range(v)) {
            ++bad;
            std::printf("not in range: %08x\n", bits);
            return;
        }
        ++checked;
        const uint16_t a = ssm::sr16_bits_general(v, u), b = ssm::sr16_bits_normal(v, u);
        if (a != b && bad++ < 10) std::printf("bits %08x u %08x: general %04x short %04x\n", bits, u, a, b);
    };
    for (uint32_t e = 113; e <= 142; ++e)
        for (uint32_t m10 : {0u, 1023u})
            for (uint32_t sign : {0u, 0x80000000u})
                for (uint32_t d = 0; d < 8192; ++d)
                    for (uint32_t uh = 0; uh < 8192; uh += (e == 113 || e == 127 || e == 142) ? 1 : 61)
                        for (uint32_t ul : {0u, 0x7FFFFu})
                            check(sign | (e << 23) | (m10 << 13) | d, (uh << 19) | ul);
    for (int i = 0; i < 50000000; ++i) {
        const uint32_t mag = 0x38800000u + next32() % 0x0F000000u;
        check((next32() & 0x80000000u) | mag, next32());
    }
    std::printf("%s: %lld values compared, %lld mismatches\n", bad ? "FAIL" : "OK", checked, bad);
    return bad ? 1 : 0;
}
