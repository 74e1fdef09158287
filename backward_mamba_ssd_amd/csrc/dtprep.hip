// dtprep.hip -- preparation of the time step and the per-head rate, and the
// chain rule back through it.
//
// "Nemotron Kernels: From Inference To Backpropagation", section "From
// Classical State Space To A Selective Mamba State": the raw time-step stream
// passes through softplus and is clamped to a configured interval; its local
// derivative is the sigmoid inside the interval and zero where the clamp
// saturates, and the boundary needs a declared convention.  "Nemotron 3 Ultra:
// replaying a rounded state", section "The Mamba state update": the time step
// is built from the raw value and a per-head bias, and the rate is
// A = -exp(logA).
//
//   forward   dt[r,h] = clamp(softplus(raw[r,h] + bias[h]), lo, hi),  A[h] = -exp(logA[h])
//   backward  d_raw[r,h] = ddt[r,h] * sigmoid(raw[r,h] + bias[h]) * [lo <= softplus <= hi]
//             d_bias[h]  = sum over r of d_raw[r,h]        (fp64, fixed order)
//             d_logA[h]  = dA[h] * A[h]
// The interval is closed: a softplus equal to either end keeps its gradient.
// The inside test is taken on the float32 softplus that dt stores.
//
// Both directions are HBM-bound elementwise passes over [rows, H] float32
// (8 B per element forward, 12 B backward).  The bias sum is deterministic:
// each workgroup of the backward owns a tile of rows x 64 heads, sums its rows
// per head in fp64 in a fixed order and writes one partial per head; a second
// pass adds the partials of a head in ascending tile order.
#include "common.hpp"
#include "launch.hpp"

namespace ssm {
namespace {

constexpr int kRowsPerTile = 64;  // rows of one backward workgroup
constexpr int kHeadsPerTile = 64; // heads of one backward workgroup (one per lane)

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(e^-|v|); no overflow for any v.
__device__ __forceinline__ float softplus32(float v) {
    return fmaxf(v, 0.f) + log1pf(expf(-fabsf(v)));
}

// sigmoid(v) = 1 / (1 + e^-v), evaluated on the side where the exponential is <= 1.
__device__ __forceinline__ float sigmoid32(float v) {
    const float e = expf(-fabsf(v));
    return v >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
}

__global__ void __launch_bounds__(256) dt_prep_kernel(DtPrepArgs a) {
    const int64_t n = a.rows * a.H;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        const int h = static_cast<int>(i % a.H);
        const float sp = softplus32(a.raw[i] + a.bias[h]);
        a.dt[i] = fminf(fmaxf(sp, a.lo), a.hi);
    }
    if (blockIdx.x == 0)
        for (int h = threadIdx.x; h < a.H; h += blockDim.x) a.A[h] = -expf(a.logA[h]);
}

// Tile (row tile rt, head tile ht): wave w takes rows rt*64 + w, +4, ...; lane l
// takes head ht*64 + l.  The four waves' fp64 sums meet in LDS in wave order.
__global__ void __launch_bounds__(256) dt_prep_bwd_kernel(DtPrepArgs a) {
    __shared__ double part[4][kHeadsPerTile];
    const int rt = blockIdx.x, ht = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int h = ht * kHeadsPerTile + lane;
    double acc = 0.0;
    if (h < a.H) {
        const float bh = a.bias[h];
        const int64_t r0 = static_cast<int64_t>(rt) * kRowsPerTile;
        const int64_t r1 = r0 + kRowsPerTile < a.rows ? r0 + kRowsPerTile : a.rows;
        for (int64_t r = r0 + wave; r < r1; r += 4) {
            const int64_t i = r * a.H + h;
            const float v = a.raw[i] + bh;
            const float sp = softplus32(v);
            const bool inside = sp >= a.lo && sp <= a.hi;
            const float g = inside ? a.ddt[i] * sigmoid32(v) : 0.f;
            a.d_raw[i] = g;
            acc += static_cast<double>(g);
        }
    }
    part[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && h < a.H)
        a.part[static_cast<int64_t>(rt) * a.H + h] = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
}

__global__ void __launch_bounds__(256) dt_prep_bwd_heads_kernel(DtPrepArgs a, int ntiles) {
    const int h = blockIdx.x * blockDim.x + threadIdx.x;
    if (h >= a.H) return;
    double s = 0.0;
    for (int t = 0; t < ntiles; ++t) s += a.part[static_cast<int64_t>(t) * a.H + h];
    a.d_bias[h] = static_cast<float>(s);
    a.d_logA[h] = a.dA[h] * -expf(a.logA[h]);
}

}  // namespace

int64_t dt_prep_row_tiles(int64_t rows) { return (rows + kRowsPerTile - 1) / kRowsPerTile; }

hipError_t launch_dt_prep(const DtPrepArgs &a, hipStream_t s) {
    const int64_t n = a.rows * a.H;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;  // grid-stride beyond this
    if (blocks < 1) blocks = 1;          // A is written even with no rows
    dt_prep_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_dt_prep_bwd(const DtPrepArgs &a, hipStream_t s) {
    const int64_t nt = dt_prep_row_tiles(a.rows);
    if (nt > 0) {
        const dim3 grid(static_cast<unsigned>(nt), static_cast<unsigned>((a.H + kHeadsPerTile - 1) / kHeadsPerTile));
        dt_prep_bwd_kernel<<<grid, 256, 0, s>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    dt_prep_bwd_heads_kernel<<<static_cast<unsigned>((a.H + 255) / 256), 256, 0, s>>>(a, static_cast<int>(nt));
    return hipGetLastError();
}

}  // namespace ssm
