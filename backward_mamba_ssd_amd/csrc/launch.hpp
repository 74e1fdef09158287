// launch.hpp -- argument blocks and host launchers of the gfx950 kernels
// (internal to the library; the public surface is include/ssm.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "ssd_common.hpp"

namespace ssm {

// Compute units of the current device, queried once per device (the chunked launchers
// size their workgroups by how deep the grid fills the chip).
inline hipError_t device_cu_count(int *out) {
    static std::atomic<int> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int v = (dev >= 0 && dev < 64) ? cache[dev].load() : 0;
    if (v == 0) {
        if ((e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        if (dev >= 0 && dev < 64) cache[dev].store(v);
    }
    *out = v;
    return hipSuccess;
}

struct DecodeArgs {
    int64_t Bsz;
    int H, P, N, G;
    float *state;         // float state, or nullptr when state16 is used
    uint16_t *state16;    // binary16 state cache (stochastically rounded on store)
    uint64_t seed, key;   // SR entropy key of this step (state16 only)
    const void *x, *B, *C;
    const float *dt, *A, *D;
    void *y;
};

struct ScanArgs {
    int64_t Bsz, T;      // T: token stride of x/B/C/dt/y (the full sequence length)
    int H, P, N, G;
    int64_t t0, r;       // tokens t0 .. t0+r-1
    int64_t L, nchunks;  // chunk_states cadence (relative to t0)
    const void *ckpt;    // initial state (float or binary16 bits) or nullptr = zero
    const float *live;   // lockstep live copy or nullptr
    float *state_out;
    const void *x, *B, *C;
    const float *dt, *A, *D;
    void *y;
    float *chunk_states;
    float *part_max, *part_sum;  // [r][Bsz*H*4] per-wave drift partials
    float *snap;                 // nullptr, or a snapshot stack: slot k+1 <- state after token t0+k
    int64_t snap_stride;         // floats between slots
};

// Rollback: state_out[b] <- snapshots[accepted[b]][b]
struct RollbackArgs {
    int64_t Bsz, per_seq;  // per_seq: floats per sequence (H*P*N), a multiple of 4
    int64_t ndraft;        // slots 0..ndraft
    const float *snap;
    const int32_t *accepted;
    float *state_out;
    int32_t *err;          // nullptr, or set to 1 when an accepted count is out of range
};

struct ScanBwdArgs {
    int64_t Bsz, T;
    int H, P, N, G;
    int64_t L, nchunks;
    const void *x, *B, *C, *dy;
    const float *dt, *A, *D, *chunk_states, *dh_final;
    void *dx;
    float *dB, *dC, *ddt, *dA, *dD, *dh0;
    // workspace
    float *slab;            // [Bsz*H][slab_stride]: states of one chunk per head
    int64_t slab_stride;    // (min(L, T) + 1) * P * N
    float *dB_part, *dC_part;  // [Bsz, T, H, N]
    double *dA_part, *dD_part;  // [Bsz*H]
};

struct Sr16Args {
    const float *in;
    uint16_t *out;
    uint64_t n, seed, ckpt, offset;
};

// SsdFwdArgs, SsdBwdArgs (the chunked MFMA path) are in ssd_common.hpp.

// Time-step and rate preparation (forward and backward share one block).
struct DtPrepArgs {
    int64_t rows;  // batch * seqlen
    int H;
    float lo, hi;  // closed clamp interval of the softplus
    const float *raw, *bias, *logA;
    float *dt, *A;                          // forward outputs
    const float *ddt, *dA;                  // backward inputs
    float *d_raw, *d_bias, *d_logA;         // backward outputs
    double *part;                           // [row tiles][H] fp64 bias partials
};

// Causal depthwise convolution + SiLU (forward and backward share one block).
struct ConvArgs {
    int64_t Bsz, T, C;
    int K;                    // taps, 1..8
    int64_t ntiles;           // backward token tiles per sequence
    const void *u, *init;     // [Bsz][T][C], [Bsz][K-1][C] or nullptr (storage dtype)
    const float *w, *bias;    // [C][K], [C]
    void *out, *final_state;  // [Bsz][T][C], [Bsz][K-1][C] or nullptr
    const void *dout;         // backward: [Bsz][T][C]
    void *du, *dinit;         // [Bsz][T][C], [Bsz][K-1][C] or nullptr
    float *dw, *dbias;        // [C][K], [C]
    double *part;             // [Bsz*ntiles][K+1][C] fp64 partials
};

// SiLU-gated group RMSNorm.
struct NormArgs {
    int64_t rows, C, G;
    float eps;
    const void *y, *z;   // [rows][C] (storage dtype)
    const float *w;      // [C]
    void *out;           // [rows][C]
    const void *dout;    // backward
    void *dy, *dz;
    float *dw;
    double *part;        // [row tiles][C] fp64 partials
};

// Tile sizes that fix the shapes of the fp64 partial-sum workspaces (host and kernels agree
// on them through these definitions).
constexpr int kDtPrepRowsPerTile = 16;  // time-step preparation: rows per workgroup
constexpr int kConvBwdTile = 256;       // conv backward: tokens per partial-sum tile
constexpr int kNormRows = 32;           // norm backward: rows per partial-sum tile
inline int64_t dt_prep_row_tiles(int64_t rows) { return (rows + kDtPrepRowsPerTile - 1) / kDtPrepRowsPerTile; }
inline int64_t conv_bwd_tiles(int64_t T) { return (T + kConvBwdTile - 1) / kConvBwdTile; }
inline int64_t norm_row_tiles(int64_t rows) { return (rows + kNormRows - 1) / kNormRows; }

// Scratch of ssm_bwd_noalloc: one 4096-token sequence at 256 heads x 64 x 128 with chunk 256
// (64 MiB of chunk-exit state gradients in bf16, 256 KiB of fp64 partials), rounded up.
constexpr size_t kNoAllocScratchBytes = size_t{65} << 20;
// The device address of the current device's scratch (looked up once per device).
hipError_t noalloc_scratch(void **ptr);

hipError_t launch_fill(float *p, int64_t n, float v, hipStream_t s);
hipError_t launch_copy(float *dst, const float *src, int64_t n, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, bool bf16, hipStream_t s);  // state or state16
hipError_t launch_scan(const ScanArgs &a, bool bf16, bool ckpt_f16, hipStream_t s);
hipError_t launch_drift_reduce(const float *pm, const float *ps, int64_t nwaves, int64_t r,
                               double inv_count, float *dmax, float *dmean, hipStream_t s);
hipError_t launch_rollback(const RollbackArgs &a, hipStream_t s);
hipError_t launch_scan_bwd(const ScanBwdArgs &a, bool bf16, hipStream_t s);
hipError_t launch_sr16(const Sr16Args &a, hipStream_t s);
hipError_t launch_ssd_fwd(const SsdFwdArgs &a, hipStream_t s);
// ev_begin / ev_end: NULL, or events recorded on s around the per-block kernel
hipError_t launch_ssd_bwd(const SsdBwdArgs &a, hipEvent_t ev_begin, hipEvent_t ev_end, hipStream_t s);
hipError_t launch_conv(const ConvArgs &a, bool bf16, bool bwd, hipStream_t s);
hipError_t launch_norm(const NormArgs &a, bool bf16, bool bwd, hipStream_t s);
hipError_t launch_dt_prep(const DtPrepArgs &a, hipStream_t s);
hipError_t launch_dt_prep_bwd(const DtPrepArgs &a, hipStream_t s);

}  // namespace ssm
