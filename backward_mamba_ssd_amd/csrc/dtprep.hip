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
// each workgroup of the backward owns a tile of 16 rows x 256 heads, sums its
// rows per head in fp64 in row order and writes one partial per head; a second
// pass adds a head's partials in a fixed order (strided lane sums, then lanes in
// order).
#include "common.hpp"
#include "launch.hpp"

namespace ssm {
namespace {

constexpr int kRowsPerTile = kDtPrepRowsPerTile;  // rows of one workgroup (loads in flight together)
constexpr int kHeadsPerTile = 256; // heads of one workgroup (one per thread)

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(e^-|v|); no overflow for any v.
__device__ __forceinline__ float softplus32(float v) {
    return fmaxf(v, 0.f) + log1pf(expf(-fabsf(v)));
}

// sigmoid(v) = 1 / (1 + e^-v), evaluated on the side where the exponential is <= 1.
__device__ __forceinline__ float sigmoid32(float v) {
    const float e = expf(-fabsf(v));
    return v >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
}

// Tile (row tile rt, head tile ht): thread t takes head ht*256 + t and the tile's
// rows; a wave reads 64 consecutive heads of one row (256 contiguous bytes).
__global__ void __launch_bounds__(256) dt_prep_kernel(DtPrepArgs a) {
    const int h = blockIdx.y * kHeadsPerTile + threadIdx.x;
    if (blockIdx.x == 0 && h < a.H) a.A[h] = -expf(a.logA[h]);
    if (h >= a.H) return;
    const float bh = a.bias[h];
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kRowsPerTile;
    const int nr = a.rows - r0 < kRowsPerTile ? static_cast<int>(a.rows - r0) : kRowsPerTile;
    float v[kRowsPerTile];
#pragma unroll
    for (int r = 0; r < kRowsPerTile; ++r)
        if (r < nr) v[r] = a.raw[(r0 + r) * a.H + h];
#pragma unroll
    for (int r = 0; r < kRowsPerTile; ++r)
        if (r < nr) a.dt[(r0 + r) * a.H + h] = fminf(fmaxf(softplus32(v[r] + bh), a.lo), a.hi);
}

// Same tiling; each thread sums its head's d_raw over the tile's rows in fp64, in
// row order, and writes one partial per (row tile, head).
__global__ void __launch_bounds__(256) dt_prep_bwd_kernel(DtPrepArgs a) {
    const int h = blockIdx.y * kHeadsPerTile + threadIdx.x;
    if (h >= a.H) return;
    const float bh = a.bias[h];
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kRowsPerTile;
    const int nr = a.rows - r0 < kRowsPerTile ? static_cast<int>(a.rows - r0) : kRowsPerTile;
    float v[kRowsPerTile], gi[kRowsPerTile];
#pragma unroll
    for (int r = 0; r < kRowsPerTile; ++r)
        if (r < nr) {
            v[r] = a.raw[(r0 + r) * a.H + h];
            gi[r] = a.ddt[(r0 + r) * a.H + h];
        }
    double acc = 0.0;
#pragma unroll
    for (int r = 0; r < kRowsPerTile; ++r)
        if (r < nr) {
            const float u = v[r] + bh;
            const float sp = softplus32(u);
            const bool inside = sp >= a.lo && sp <= a.hi;
            const float g = inside ? gi[r] * sigmoid32(u) : 0.f;
            a.d_raw[(r0 + r) * a.H + h] = g;
            acc += static_cast<double>(g);
        }
    a.part[static_cast<int64_t>(blockIdx.x) * a.H + h] = acc;
}

// One 64-lane workgroup per head: lane l adds the partials of tiles l, l+64, ... in
// order, then lane 0 adds the 64 lane sums in lane order (a fixed order).
__global__ void __launch_bounds__(64) dt_prep_bwd_heads_kernel(DtPrepArgs a, int64_t ntiles) {
    __shared__ double red[64];
    const int h = blockIdx.x, lane = threadIdx.x;
    double s = 0.0;
    for (int64_t t = lane; t < ntiles; t += 64) s += a.part[t * a.H + h];
    red[lane] = s;
    __syncthreads();
    if (lane == 0) {
        double tot = 0.0;
        for (int l = 0; l < 64; ++l) tot += red[l];
        a.d_bias[h] = static_cast<float>(tot);
        a.d_logA[h] = a.dA[h] * -expf(a.logA[h]);
    }
}

}  // namespace


hipError_t launch_dt_prep(const DtPrepArgs &a, hipStream_t s) {
    int64_t nt = dt_prep_row_tiles(a.rows);
    if (nt < 1) nt = 1;  // A is written even with no rows
    const dim3 grid(static_cast<unsigned>(nt), static_cast<unsigned>((a.H + kHeadsPerTile - 1) / kHeadsPerTile));
    dt_prep_kernel<<<grid, 256, 0, s>>>(a);
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
    dt_prep_bwd_heads_kernel<<<static_cast<unsigned>(a.H), 64, 0, s>>>(a, nt);
    return hipGetLastError();
}

}  // namespace ssm
