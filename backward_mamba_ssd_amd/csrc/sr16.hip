// sr16.hip -- FP16 stochastically rounded checkpoint of a float32 state (the
// rounding rule and the keyed entropy are in sr16.hpp).
//
// HBM-bound elementwise kernel: 4 B read + 2 B written per element; each thread
// handles 8 consecutive elements (two 16-byte loads, one 16-byte store).
#include "common.hpp"
#include "launch.hpp"
#include "sr16.hpp"

namespace ssm {

__global__ void __launch_bounds__(256) sr16_kernel(Sr16Args a) {
    const uint64_t sub = sr16_stream(a.seed, a.ckpt);
    const uint64_t i0 = (static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 8ull;
    if (i0 >= a.n) return;
    if (i0 + 8 <= a.n && (reinterpret_cast<uintptr_t>(a.in + i0) & 15u) == 0 &&
        (reinterpret_cast<uintptr_t>(a.out + i0) & 15u) == 0) {
        const float4 v0 = nt_ld4(a.in + i0);
        const float4 v1 = nt_ld4(a.in + i0 + 4);
        const float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        u16x8 o;
        uint32_t u[8];
        sr16_entropy_run<8>(sub, a.offset + i0, u);
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = sr16_bits(vv[j], u[j]);
        __builtin_nontemporal_store(o, reinterpret_cast<u16x8 *>(a.out + i0));
    } else {
        for (uint64_t i = i0; i < a.n && i < i0 + 8; ++i) {
            const uint64_t e = a.offset + i;
            a.out[i] = sr16_bits(a.in[i], sr16_entropy(sub, e));
        }
    }
}

hipError_t launch_sr16(const Sr16Args &a, hipStream_t s) {
    if (a.n == 0) return hipSuccess;
    const uint64_t threads = (a.n + 7) / 8;
    const uint64_t blocks = (threads + 255) / 256;
    sr16_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace ssm
