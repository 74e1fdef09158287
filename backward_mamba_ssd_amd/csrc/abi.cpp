// abi.cpp -- the extern "C" surface declared in include/ssm.h: argument
// validation (all of it before the first enqueue), workspace carving, and
// dispatch to the gfx950 kernels.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <climits>
#include <cmath>
#include <cstring>
#include <initializer_list>

#include "../../include/ssm.h"
#include "launch.hpp"

using namespace ssm;

namespace {

constexpr size_t kAlign = 256;
static_assert(kNoAllocScratchBytes == SSM_NOALLOC_SCRATCH_BYTES, "ssm.h states the scratch size");
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
size_t esize(ssm_dtype t) { return t == SSM_F32 ? 4 : 2; }

// Alignment contract: state-shaped float arrays are read as float4 (16 B);
// B and C rows are read 4 elements at a time (4 * element size); on the MFMA
// path x, y, dy, dx rows are read 16 B at a time; everything else is scalar.
bool check_align(std::initializer_list<const void *> vec16, std::initializer_list<const void *> bc,
                 std::initializer_list<const void *> rows, std::initializer_list<const void *> scal,
                 ssm_dtype t, bool mfma) {
    for (const void *p : vec16)
        if (p && !aligned(p, 16)) return false;
    for (const void *p : bc)
        if (p && !aligned(p, mfma ? 16 : 4 * esize(t))) return false;
    for (const void *p : rows)
        if (p && !aligned(p, mfma ? 16 : esize(t))) return false;
    for (const void *p : scal)
        if (p && !aligned(p, 4)) return false;
    return true;
}

bool valid_dtype(ssm_dtype t) { return t == SSM_F32 || t == SSM_BF16; }

// Dims every call shares.  seqlen/batch may be zero (no tokens / no sequences).
ssm_status check_dims(const ssm_dims *d, bool need_chunk) {
    if (d == nullptr) return SSM_ERR_NULL;
    if (d->batch < 0 || d->seqlen < 0 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 ||
        d->ngroups < 1)
        return SSM_ERR_DIMS;
    if (d->nheads % d->ngroups != 0) return SSM_ERR_DIMS;
    if (need_chunk && d->chunk < 1) return SSM_ERR_DIMS;
    if (d->batch * d->nheads > (int64_t(1) << 31) - 1) return SSM_ERR_DIMS;
    if (d->nheads > 65535 || d->headdim > 65535) return SSM_ERR_DIMS;
    return SSM_OK;
}

// Token-serial kernels: dstate in {16,32,64,128,256}; a 256-thread workgroup
// holds 8 rows per thread, i.e. headdim <= 8 * 256 / (dstate / 4).
bool serial_supported(const ssm_dims *d) {
    const int64_t N = d->dstate;
    if (N != 16 && N != 32 && N != 64 && N != 128 && N != 256) return false;
    return d->headdim <= 8 * 256 / (N / 4);
}

bool mfma_shape(const ssm_dims *d, ssm_dtype t) {
    return t == SSM_BF16 && d->headdim == 64 && d->dstate == 128 && d->chunk % 64 == 0;
}

bool mfma_fwd_path(const ssm_dims *d, ssm_dtype t) { return mfma_shape(d, t); }

bool mfma_bwd_path(const ssm_dims *d, ssm_dtype t) {
    return mfma_shape(d, t) && d->chunk <= 256 && d->nheads / d->ngroups <= 64;
}

bool mfma_path(const ssm_dims *d, ssm_dtype t) { return mfma_fwd_path(d, t) && mfma_bwd_path(d, t); }

int64_t nchunks_of(const ssm_dims *d) { return (d->seqlen + d->chunk - 1) / d->chunk; }

struct Carve {
    char *base;
    size_t off = 0;
    template <typename T> T *take(size_t count) {
        T *p = reinterpret_cast<T *>(base + off);
        off += round_up(count * sizeof(T));
        return p;
    }
};

size_t bwd_ws_bytes(const ssm_dims *d, ssm_dtype t) {
    const size_t B = d->batch, T = d->seqlen, H = d->nheads, P = d->headdim, N = d->dstate;
    const size_t nc = nchunks_of(d);
    if (mfma_bwd_path(d, t)) {
        const size_t nb = d->chunk / 64;
        return round_up(B * H * nc * P * N * sizeof(uint16_t)) +
               2 * round_up(B * H * nc * nb * sizeof(double));
    }
    const size_t L = d->chunk < d->seqlen ? d->chunk : (d->seqlen > 0 ? d->seqlen : 1);
    return round_up(B * H * (L + 1) * P * N * sizeof(float)) +
           2 * round_up(B * T * H * N * sizeof(float)) + 2 * round_up(B * H * sizeof(double));
}

size_t replay_ws_bytes(const ssm_dims *d, int64_t r) {
    return 2 * round_up(static_cast<size_t>(r) * d->batch * d->nheads * 4 * sizeof(float));
}

// The preparation reads batch, seqlen and nheads only.
ssm_status check_dt_prep_dims(const ssm_dims *d, float lo, float hi) {
    if (d == nullptr) return SSM_ERR_NULL;
    if (d->batch < 0 || d->seqlen < 0 || d->nheads < 1 || d->nheads > 65535) return SSM_ERR_DIMS;
    if (d->seqlen > 0 && d->batch > (int64_t(1) << 62) / d->seqlen) return SSM_ERR_DIMS;
    if (d->batch * d->seqlen > (int64_t(1) << 34)) return SSM_ERR_DIMS;  // 16-row tiles fit the grid
    if (!(lo <= hi)) return SSM_ERR_DIMS;  // also rejects NaN bounds
    return SSM_OK;
}

size_t dt_prep_ws_bytes(const ssm_dims *d) {
    return round_up(static_cast<size_t>(dt_prep_row_tiles(d->batch * d->seqlen)) * d->nheads * sizeof(double));
}

bool conv_sizes_ok(int64_t batch, int64_t seqlen, int64_t channels, int64_t width) {
    return batch >= 0 && batch <= 65535 && seqlen >= 0 && seqlen <= (int64_t(1) << 36) &&
           channels >= 4 && channels % 4 == 0 && channels <= (int64_t(1) << 32) && width >= 1 &&
           width <= 8;
}

size_t conv_ws_bytes(int64_t batch, int64_t seqlen, int64_t channels, int64_t width) {
    return round_up(static_cast<size_t>(batch) * conv_bwd_tiles(seqlen) * (width + 1) * channels *
                    sizeof(double));
}

bool norm_sizes_ok(int64_t rows, int64_t channels, int64_t ngroups) {
    if (rows < 0 || rows > INT32_MAX || channels < 1 || ngroups < 1 || ngroups > 65535) return false;
    if (channels % ngroups != 0) return false;
    const int64_t S = channels / ngroups;
    return S % 8 == 0 && S <= 8192;
}

size_t norm_ws_bytes(int64_t rows, int64_t channels) {
    return round_up(static_cast<size_t>(norm_row_tiles(rows)) * channels * sizeof(double));
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b) return false;
    const char *x = static_cast<const char *>(a), *y = static_cast<const char *>(b);
    return x < y + nb && y < x + na;
}

hipError_t fill(float *p, int64_t n, hipStream_t s) { return launch_fill(p, n, 0.f, s); }

}  // namespace

extern "C" {

const char *ssm_status_string(ssm_status s) {
    switch (s) {
        case SSM_OK: return "SSM_OK";
        case SSM_ERR_NULL: return "SSM_ERR_NULL: a required pointer is NULL";
        case SSM_ERR_DIMS: return "SSM_ERR_DIMS: invalid dimensions";
        case SSM_ERR_UNSUPPORTED: return "SSM_ERR_UNSUPPORTED: no kernel for these dimensions";
        case SSM_ERR_DTYPE: return "SSM_ERR_DTYPE: unknown dtype";
        case SSM_ERR_ALIGN: return "SSM_ERR_ALIGN: pointer not aligned as required";
        case SSM_ERR_WORKSPACE: return "SSM_ERR_WORKSPACE: workspace missing or too small";
        case SSM_ERR_HIP: return "SSM_ERR_HIP: HIP launch failed";
    }
    return "unknown ssm_status";
}

int ssm_uses_mfma_path(const ssm_dims *d, ssm_dtype dtype) {
    if (check_dims(d, true) != SSM_OK) return 0;
    return mfma_path(d, dtype) ? 1 : 0;
}

size_t ssm_workspace_bytes(const ssm_dims *d, ssm_dtype dtype, int which, int64_t r) {
    if (!valid_dtype(dtype)) return static_cast<size_t>(-1);
    if (which == SSM_WS_FWD) {
        if (check_dims(d, true) != SSM_OK) return static_cast<size_t>(-1);
        if (!mfma_fwd_path(d, dtype) && !serial_supported(d)) return static_cast<size_t>(-1);
        return 0;
    }
    if (which == SSM_WS_BWD) {
        if (check_dims(d, true) != SSM_OK) return static_cast<size_t>(-1);
        if (!mfma_bwd_path(d, dtype) && !serial_supported(d)) return static_cast<size_t>(-1);
        return bwd_ws_bytes(d, dtype);
    }
    if (which == SSM_WS_DT_PREP_BWD) {
        if (check_dt_prep_dims(d, 0.f, 0.f) != SSM_OK) return static_cast<size_t>(-1);
        return dt_prep_ws_bytes(d);
    }
    if (which == SSM_WS_REPLAY) {
        if (check_dims(d, false) != SSM_OK || r < 0 || !serial_supported(d))
            return static_cast<size_t>(-1);
        return replay_ws_bytes(d, r);
    }
    return static_cast<size_t>(-1);
}

ssm_status ssm_fwd_chunked(const ssm_dims *d, ssm_dtype dtype, const void *x, const void *B,
                           const void *C, const float *dt, const float *A, const float *D,
                           const float *h0, void *y, float *h_final, float *chunk_states,
                           void *workspace, size_t ws_bytes, ssm_stream stream) {
    ssm_status st = check_dims(d, true);
    if (st != SSM_OK) return st;
    if (!valid_dtype(dtype)) return SSM_ERR_DTYPE;
    const bool mfma = mfma_fwd_path(d, dtype);
    if (!mfma && !serial_supported(d)) return SSM_ERR_UNSUPPORTED;
    const bool tokens = d->batch > 0 && d->seqlen > 0;
    if (tokens && (!x || !B || !C || !dt || !y)) return SSM_ERR_NULL;
    if (!A || !D) return SSM_ERR_NULL;
    if (!check_align({h0, h_final, chunk_states}, {B, C}, {x, y}, {dt, A, D}, dtype, mfma))
        return SSM_ERR_ALIGN;
    (void)workspace;
    (void)ws_bytes;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (d->batch == 0) return SSM_OK;
    const int64_t PN = d->headdim * d->dstate;
    if (d->seqlen == 0) {  // no tokens: the final state is the initial state
        if (h_final) {
            hipError_t e = h0 ? launch_copy(h_final, h0, d->batch * d->nheads * PN, s)
                              : fill(h_final, d->batch * d->nheads * PN, s);
            if (e != hipSuccess) return SSM_ERR_HIP;
        }
        return SSM_OK;
    }
    hipError_t e;
    if (mfma) {
        SsdFwdArgs a{};
        a.Bsz = d->batch; a.T = d->seqlen; a.H = static_cast<int>(d->nheads);
        a.G = static_cast<int>(d->ngroups); a.L = d->chunk; a.nchunks = nchunks_of(d);
        a.x = x; a.B = B; a.C = C; a.dt = dt; a.A = A; a.D = D; a.h0 = h0; a.y = y;
        a.h_final = h_final; a.chunk_states = chunk_states;
        e = launch_ssd_fwd(a, s);
    } else {
        ScanArgs a{};
        a.Bsz = d->batch; a.T = d->seqlen; a.H = static_cast<int>(d->nheads);
        a.P = static_cast<int>(d->headdim); a.N = static_cast<int>(d->dstate);
        a.G = static_cast<int>(d->ngroups); a.t0 = 0; a.r = d->seqlen; a.L = d->chunk;
        a.nchunks = nchunks_of(d); a.ckpt = h0; a.live = nullptr; a.state_out = h_final;
        a.x = x; a.B = B; a.C = C; a.dt = dt; a.A = A; a.D = D; a.y = y;
        a.chunk_states = chunk_states;
        e = launch_scan(a, dtype == SSM_BF16, false, s);
    }
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // extern "C"

namespace {

// ssm_bwd and ssm_bwd_timed: `ev` is NULL or two caller events recorded around the
// per-block kernel of the chunked path.
ssm_status bwd_impl(const ssm_dims *d, ssm_dtype dtype, const void *x, const void *B,
                    const void *C, const float *dt, const float *A, const float *D,
                    const float *chunk_states, const void *dy, const float *dh_final, void *dx,
                    float *dB, float *dC, float *ddt, float *dA, float *dD, float *dh0,
                    void *workspace, size_t ws_bytes, void *const *ev, hipStream_t s) {
    ssm_status st = check_dims(d, true);
    if (st != SSM_OK) return st;
    if (!valid_dtype(dtype)) return SSM_ERR_DTYPE;
    const bool mfma = mfma_bwd_path(d, dtype);
    if (!mfma && !serial_supported(d)) return SSM_ERR_UNSUPPORTED;
    const bool tokens = d->batch > 0 && d->seqlen > 0;
    if (tokens && (!x || !B || !C || !dt || !chunk_states || !dy || !dx || !dB || !dC || !ddt))
        return SSM_ERR_NULL;
    if (!A || !D || !dA || !dD) return SSM_ERR_NULL;
    if (!check_align({chunk_states, dh_final, dh0, workspace}, {B, C, dB, dC}, {x, dy, dx},
                     {dt, A, D, ddt, dA, dD}, dtype, mfma))
        return SSM_ERR_ALIGN;
    const size_t need = tokens ? bwd_ws_bytes(d, dtype) : 0;
    if (need > 0 && (workspace == nullptr || ws_bytes < need)) return SSM_ERR_WORKSPACE;
    hipEvent_t ev_begin = nullptr, ev_end = nullptr;
    if (ev != nullptr) {
        ev_begin = static_cast<hipEvent_t>(ev[0]);
        ev_end = static_cast<hipEvent_t>(ev[1]);
        if (ev_begin == nullptr || ev_end == nullptr) return SSM_ERR_NULL;
        // a first record of both events: an unusable event fails here, before any work
        if (hipEventRecord(ev_begin, s) != hipSuccess || hipEventRecord(ev_end, s) != hipSuccess)
            return SSM_ERR_HIP;
    }
    const int64_t PN = d->headdim * d->dstate;
    if (!tokens) {  // no tokens: zero parameter gradients, dh0 = dh_final
        if (fill(dA, d->nheads, s) != hipSuccess || fill(dD, d->nheads, s) != hipSuccess)
            return SSM_ERR_HIP;
        if (dh0 && d->batch > 0) {
            hipError_t e = dh_final ? launch_copy(dh0, dh_final, d->batch * d->nheads * PN, s)
                                    : fill(dh0, d->batch * d->nheads * PN, s);
            if (e != hipSuccess) return SSM_ERR_HIP;
        }
        return SSM_OK;
    }
    Carve cv{static_cast<char *>(workspace)};
    hipError_t e;
    const int64_t nc = nchunks_of(d);
    if (mfma) {
        SsdBwdArgs a{};
        a.Bsz = d->batch; a.T = d->seqlen; a.H = static_cast<int>(d->nheads);
        a.G = static_cast<int>(d->ngroups); a.L = d->chunk; a.nchunks = nc;
        a.x = x; a.B = B; a.C = C; a.dy = dy; a.dt = dt; a.A = A; a.D = D;
        a.chunk_states = chunk_states; a.dh_final = dh_final; a.dx = dx; a.dB = dB; a.dC = dC;
        a.ddt = ddt; a.dA = dA; a.dD = dD; a.dh0 = dh0;
        a.dstates = cv.take<bf16_t>(d->batch * d->nheads * nc * PN);
        a.pA = cv.take<double>(d->batch * d->nheads * nc * (d->chunk / 64));
        a.pD = cv.take<double>(d->batch * d->nheads * nc * (d->chunk / 64));
        e = launch_ssd_bwd(a, ev_begin, ev_end, s);
    } else {
        ScanBwdArgs a{};
        a.Bsz = d->batch; a.T = d->seqlen; a.H = static_cast<int>(d->nheads);
        a.P = static_cast<int>(d->headdim); a.N = static_cast<int>(d->dstate);
        a.G = static_cast<int>(d->ngroups); a.L = d->chunk; a.nchunks = nc;
        a.x = x; a.B = B; a.C = C; a.dy = dy; a.dt = dt; a.A = A; a.D = D;
        a.chunk_states = chunk_states; a.dh_final = dh_final; a.dx = dx; a.dB = dB; a.dC = dC;
        a.ddt = ddt; a.dA = dA; a.dD = dD; a.dh0 = dh0;
        // the sweep rebuilds the states of one saved chunk at a time
        const int64_t Lslab = d->chunk < d->seqlen ? d->chunk : d->seqlen;
        a.slab_stride = (Lslab + 1) * PN;
        a.slab = cv.take<float>(d->batch * d->nheads * a.slab_stride);
        a.dB_part = cv.take<float>(d->batch * d->seqlen * d->nheads * d->dstate);
        a.dC_part = cv.take<float>(d->batch * d->seqlen * d->nheads * d->dstate);
        a.dA_part = cv.take<double>(d->batch * d->nheads);
        a.dD_part = cv.take<double>(d->batch * d->nheads);
        e = launch_scan_bwd(a, dtype == SSM_BF16, s);
    }
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

}  // namespace

extern "C" {

ssm_status ssm_bwd(const ssm_dims *d, ssm_dtype dtype, const void *x, const void *B,
                   const void *C, const float *dt, const float *A, const float *D,
                   const float *chunk_states, const void *dy, const float *dh_final, void *dx,
                   float *dB, float *dC, float *ddt, float *dA, float *dD, float *dh0,
                   void *workspace, size_t ws_bytes, ssm_stream stream) {
    return bwd_impl(d, dtype, x, B, C, dt, A, D, chunk_states, dy, dh_final, dx, dB, dC, ddt, dA,
                    dD, dh0, workspace, ws_bytes, nullptr, static_cast<hipStream_t>(stream));
}

ssm_status ssm_bwd_timed(const ssm_dims *d, ssm_dtype dtype, const void *x, const void *B,
                         const void *C, const float *dt, const float *A, const float *D,
                         const float *chunk_states, const void *dy, const float *dh_final,
                         void *dx, float *dB, float *dC, float *ddt, float *dA, float *dD,
                         float *dh0, void *workspace, size_t ws_bytes, void *const *block_events,
                         ssm_stream stream) {
    if (block_events == nullptr) return SSM_ERR_NULL;
    return bwd_impl(d, dtype, x, B, C, dt, A, D, chunk_states, dy, dh_final, dx, dB, dC, ddt, dA,
                    dD, dh0, workspace, ws_bytes, block_events, static_cast<hipStream_t>(stream));
}

ssm_status ssm_bwd_noalloc(const ssm_dims *d, ssm_dtype dtype, const void *x, const void *B,
                           const void *C, const float *dt, const float *A, const float *D,
                           const float *chunk_states, const void *dy, const float *dh_final,
                           void *dx, float *dB, float *dC, float *ddt, float *dA, float *dD,
                           float *dh0, ssm_stream stream) {
    ssm_status st = check_dims(d, true);
    if (st != SSM_OK) return st;
    if (!valid_dtype(dtype)) return SSM_ERR_DTYPE;
    if (!mfma_bwd_path(d, dtype) && !serial_supported(d)) return SSM_ERR_UNSUPPORTED;
    const bool tokens = d->batch > 0 && d->seqlen > 0;
    const size_t need = tokens ? bwd_ws_bytes(d, dtype) : 0;
    if (need > kNoAllocScratchBytes) return SSM_ERR_WORKSPACE;  // beyond the library's scratch
    void *ws = nullptr;
    if (need > 0 && noalloc_scratch(&ws) != hipSuccess) return SSM_ERR_HIP;
    return bwd_impl(d, dtype, x, B, C, dt, A, D, chunk_states, dy, dh_final, dx, dB, dC, ddt, dA,
                    dD, dh0, ws, need > 0 ? kNoAllocScratchBytes : 0, nullptr,
                    static_cast<hipStream_t>(stream));
}

ssm_status ssm_decode_step(const ssm_dims *d, ssm_dtype dtype, float *state, const void *x,
                           const void *B, const void *C, const float *dt, const float *A,
                           const float *D, void *y, ssm_stream stream) {
    ssm_status st = check_dims(d, false);
    if (st != SSM_OK) return st;
    if (!valid_dtype(dtype)) return SSM_ERR_DTYPE;
    if (!serial_supported(d)) return SSM_ERR_UNSUPPORTED;
    if (d->batch > 0 && (!state || !x || !B || !C || !dt || !y)) return SSM_ERR_NULL;
    if (!A || !D) return SSM_ERR_NULL;
    if (!check_align({state}, {B, C}, {x, y}, {dt, A, D}, dtype, false)) return SSM_ERR_ALIGN;
    if (d->batch == 0) return SSM_OK;
    DecodeArgs a{};
    a.Bsz = d->batch; a.H = static_cast<int>(d->nheads); a.P = static_cast<int>(d->headdim);
    a.N = static_cast<int>(d->dstate); a.G = static_cast<int>(d->ngroups);
    a.state = state; a.x = x; a.B = B; a.C = C; a.dt = dt; a.A = A; a.D = D; a.y = y;
    return launch_decode(a, dtype == SSM_BF16, static_cast<hipStream_t>(stream)) == hipSuccess
               ? SSM_OK
               : SSM_ERR_HIP;
}

ssm_status ssm_decode_step_sr16(const ssm_dims *d, ssm_dtype dtype, uint16_t *state16,
                                const void *x, const void *B, const void *C, const float *dt,
                                const float *A, const float *D, void *y, uint64_t seed,
                                uint64_t step, ssm_stream stream) {
    ssm_status st = check_dims(d, false);
    if (st != SSM_OK) return st;
    if (!valid_dtype(dtype)) return SSM_ERR_DTYPE;
    if (!serial_supported(d)) return SSM_ERR_UNSUPPORTED;
    if (d->batch > 0 && (!state16 || !x || !B || !C || !dt || !y)) return SSM_ERR_NULL;
    if (!A || !D) return SSM_ERR_NULL;
    if (!aligned(state16, 8)) return SSM_ERR_ALIGN;  // four binary16 per lane
    if (!check_align({}, {B, C}, {x, y}, {dt, A, D}, dtype, false)) return SSM_ERR_ALIGN;
    if (d->batch == 0) return SSM_OK;
    DecodeArgs a{};
    a.Bsz = d->batch; a.H = static_cast<int>(d->nheads); a.P = static_cast<int>(d->headdim);
    a.N = static_cast<int>(d->dstate); a.G = static_cast<int>(d->ngroups);
    a.state16 = state16; a.seed = seed; a.key = step;
    a.x = x; a.B = B; a.C = C; a.dt = dt; a.A = A; a.D = D; a.y = y;
    return launch_decode(a, dtype == SSM_BF16, static_cast<hipStream_t>(stream)) == hipSuccess
               ? SSM_OK
               : SSM_ERR_HIP;
}

ssm_status ssm_checkpoint_sr16(const float *state, uint16_t *out, uint64_t n_elems,
                               uint64_t seed, uint64_t ckpt_index, uint64_t elem_offset,
                               ssm_stream stream) {
    if (n_elems == 0) return SSM_OK;
    if (!state || !out) return SSM_ERR_NULL;
    if (!aligned(state, 4) || !aligned(out, 2)) return SSM_ERR_ALIGN;
    const char *a0 = reinterpret_cast<const char *>(state);
    const char *b0 = reinterpret_cast<const char *>(out);
    if (a0 < b0 + n_elems * 2 && b0 < a0 + n_elems * 4) return SSM_ERR_DIMS;  // aliasing
    Sr16Args a{state, out, n_elems, seed, ckpt_index, elem_offset};
    return launch_sr16(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status ssm_replay(const ssm_dims *d, ssm_dtype dtype, const void *ckpt, ssm_dtype ckpt_dtype,
                      float *state_out, const void *x, const void *B, const void *C,
                      const float *dt, const float *A, const float *D, int64_t t0, int64_t r,
                      void *y, const float *live_ckpt, float *drift_max, float *drift_mean,
                      void *workspace, size_t ws_bytes, ssm_stream stream) {
    ssm_status st = check_dims(d, false);
    if (st != SSM_OK) return st;
    if (!valid_dtype(dtype)) return SSM_ERR_DTYPE;
    if (ckpt_dtype != SSM_F32 && ckpt_dtype != SSM_F16) return SSM_ERR_DTYPE;
    if (!serial_supported(d)) return SSM_ERR_UNSUPPORTED;
    if (t0 < 0 || r < 0 || t0 + r > d->seqlen) return SSM_ERR_DIMS;
    if (d->batch > 0 && (!ckpt || !state_out)) return SSM_ERR_NULL;
    if (d->batch > 0 && r > 0 && (!x || !B || !C || !dt)) return SSM_ERR_NULL;
    if (!A || !D) return SSM_ERR_NULL;
    if (live_ckpt && r > 0 && (!drift_max || !drift_mean)) return SSM_ERR_NULL;
    if (!check_align({ckpt, state_out, live_ckpt, workspace}, {B, C}, {x, y},
                     {dt, A, D, drift_max, drift_mean}, dtype, false))
        return SSM_ERR_ALIGN;
    const size_t need = (live_ckpt && r > 0) ? replay_ws_bytes(d, r) : 0;
    if (need > 0 && (workspace == nullptr || ws_bytes < need)) return SSM_ERR_WORKSPACE;
    if (d->batch == 0) return SSM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    Carve cv{static_cast<char *>(workspace)};
    ScanArgs a{};
    a.Bsz = d->batch; a.T = d->seqlen; a.H = static_cast<int>(d->nheads);
    a.P = static_cast<int>(d->headdim); a.N = static_cast<int>(d->dstate);
    a.G = static_cast<int>(d->ngroups); a.t0 = t0; a.r = r; a.L = 1; a.nchunks = 0;
    a.ckpt = ckpt; a.live = (r > 0) ? live_ckpt : nullptr; a.state_out = state_out;
    a.x = x; a.B = B; a.C = C; a.dt = dt; a.A = A; a.D = D; a.y = y; a.chunk_states = nullptr;
    const int64_t nwaves = d->batch * d->nheads * 4;
    if (a.live) {
        a.part_max = cv.take<float>(r * nwaves);
        a.part_sum = cv.take<float>(r * nwaves);
    }
    hipError_t e = launch_scan(a, dtype == SSM_BF16, ckpt_dtype == SSM_F16, s);
    if (e == hipSuccess && a.live) {
        const double cnt = static_cast<double>(d->batch) * d->nheads * d->headdim * d->dstate;
        e = launch_drift_reduce(a.part_max, a.part_sum, nwaves, r, 1.0 / cnt, drift_max,
                                drift_mean, s);
    }
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status ssm_dt_prep(const ssm_dims *d, const float *dt_raw, const float *dt_bias,
                       const float *logA, float dt_lo, float dt_hi, float *dt, float *A,
                       ssm_stream stream) {
    ssm_status st = check_dt_prep_dims(d, dt_lo, dt_hi);
    if (st != SSM_OK) return st;
    const int64_t rows = d->batch * d->seqlen;
    if (!logA || !A || (rows > 0 && (!dt_raw || !dt_bias || !dt))) return SSM_ERR_NULL;
    if (!check_align({}, {}, {}, {dt_raw, dt_bias, logA, dt, A}, SSM_F32, false)) return SSM_ERR_ALIGN;
    DtPrepArgs a{};
    a.rows = rows; a.H = static_cast<int>(d->nheads); a.lo = dt_lo; a.hi = dt_hi;
    a.raw = dt_raw; a.bias = dt_bias; a.logA = logA; a.dt = dt; a.A = A;
    return launch_dt_prep(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status ssm_dt_prep_bwd(const ssm_dims *d, const float *dt_raw, const float *dt_bias,
                           const float *logA, float dt_lo, float dt_hi, const float *ddt,
                           const float *dA, float *d_raw, float *d_bias, float *d_logA,
                           void *workspace, size_t ws_bytes, ssm_stream stream) {
    ssm_status st = check_dt_prep_dims(d, dt_lo, dt_hi);
    if (st != SSM_OK) return st;
    const int64_t rows = d->batch * d->seqlen;
    if (!dt_bias || !logA || !dA || !d_bias || !d_logA) return SSM_ERR_NULL;
    if (rows > 0 && (!dt_raw || !ddt || !d_raw)) return SSM_ERR_NULL;
    if (!check_align({workspace}, {}, {}, {dt_raw, dt_bias, logA, ddt, dA, d_raw, d_bias, d_logA},
                     SSM_F32, false))
        return SSM_ERR_ALIGN;
    const size_t need = dt_prep_ws_bytes(d);
    if (need > 0 && (workspace == nullptr || ws_bytes < need)) return SSM_ERR_WORKSPACE;
    DtPrepArgs a{};
    a.rows = rows; a.H = static_cast<int>(d->nheads); a.lo = dt_lo; a.hi = dt_hi;
    a.raw = dt_raw; a.bias = dt_bias; a.logA = logA; a.ddt = ddt; a.dA = dA;
    a.d_raw = d_raw; a.d_bias = d_bias; a.d_logA = d_logA;
    a.part = static_cast<double *>(workspace);
    return launch_dt_prep_bwd(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status ssm_draft_snapshots(const ssm_dims *d, ssm_dtype dtype, float *snapshots,
                               const void *x, const void *B, const void *C, const float *dt,
                               const float *A, const float *D, void *y, ssm_stream stream) {
    ssm_status st = check_dims(d, false);
    if (st != SSM_OK) return st;
    if (!valid_dtype(dtype)) return SSM_ERR_DTYPE;
    if (!serial_supported(d)) return SSM_ERR_UNSUPPORTED;
    if (!A || !D) return SSM_ERR_NULL;
    if (d->batch > 0 && !snapshots) return SSM_ERR_NULL;
    if (d->batch > 0 && d->seqlen > 0 && (!x || !B || !C || !dt)) return SSM_ERR_NULL;
    if (!check_align({snapshots}, {B, C}, {x, y}, {dt, A, D}, dtype, false)) return SSM_ERR_ALIGN;
    if (d->batch == 0 || d->seqlen == 0) return SSM_OK;
    ScanArgs a{};
    a.Bsz = d->batch; a.T = d->seqlen; a.H = static_cast<int>(d->nheads);
    a.P = static_cast<int>(d->headdim); a.N = static_cast<int>(d->dstate);
    a.G = static_cast<int>(d->ngroups); a.t0 = 0; a.r = d->seqlen; a.L = 1; a.nchunks = 0;
    a.ckpt = snapshots; a.live = nullptr; a.state_out = nullptr;
    a.x = x; a.B = B; a.C = C; a.dt = dt; a.A = A; a.D = D; a.y = y; a.chunk_states = nullptr;
    a.snap = snapshots;
    a.snap_stride = d->batch * d->nheads * d->headdim * d->dstate;
    return launch_scan(a, dtype == SSM_BF16, false, static_cast<hipStream_t>(stream)) == hipSuccess
               ? SSM_OK
               : SSM_ERR_HIP;
}

ssm_status ssm_rollback(const ssm_dims *d, const float *snapshots, const int32_t *accepted,
                        float *state_out, int32_t *err, ssm_stream stream) {
    ssm_status st = check_dims(d, false);
    if (st != SSM_OK) return st;
    if (d->batch > 65535 || d->seqlen > INT32_MAX) return SSM_ERR_DIMS;
    if (d->batch == 0) return SSM_OK;
    if (!snapshots || !accepted || !state_out) return SSM_ERR_NULL;
    if (!aligned(snapshots, 16) || !aligned(state_out, 16) || !aligned(accepted, 4) ||
        !aligned(err, 4))
        return SSM_ERR_ALIGN;
    const int64_t per_seq = d->nheads * d->headdim * d->dstate;
    if (per_seq % 4 != 0) return SSM_ERR_UNSUPPORTED;  // 16-byte copies
    // state_out is one of the slots, or disjoint from the whole stack
    const char *s0 = reinterpret_cast<const char *>(snapshots);
    const size_t slot_bytes = static_cast<size_t>(d->batch) * per_seq * sizeof(float);
    const char *s1 = s0 + (d->seqlen + 1) * slot_bytes;
    const char *o = reinterpret_cast<const char *>(state_out);
    if (o + slot_bytes > s0 && o < s1 && (o < s0 || (o - s0) % slot_bytes != 0)) return SSM_ERR_DIMS;
    RollbackArgs a{};
    a.Bsz = d->batch; a.per_seq = per_seq; a.ndraft = d->seqlen;
    a.snap = snapshots; a.accepted = accepted; a.state_out = state_out; a.err = err;
    return launch_rollback(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status ssm_conv1d_silu(int64_t batch, int64_t seqlen, int64_t channels, int64_t width,
                           ssm_dtype dtype, const void *u, const float *w, const float *bias,
                           const void *conv_init, void *out, void *conv_final,
                           ssm_stream stream) {
    if (!valid_dtype(dtype)) return SSM_ERR_DTYPE;
    if (!conv_sizes_ok(batch, seqlen, channels, width)) return SSM_ERR_DIMS;
    if (!w || !bias) return SSM_ERR_NULL;
    if (batch > 0 && seqlen > 0 && (!u || !out)) return SSM_ERR_NULL;
    if (!aligned(u, 16) || !aligned(out, 16) || !aligned(bias, 16) || !aligned(conv_init, 16) ||
        !aligned(conv_final, 16) || !aligned(w, 4))
        return SSM_ERR_ALIGN;
    const size_t es = esize(dtype);
    const size_t nout = static_cast<size_t>(batch) * seqlen * channels * es;
    const size_t ninit = static_cast<size_t>(batch) * (width - 1) * channels * es;
    if (overlaps(out, nout, u, nout) || overlaps(out, nout, conv_init, ninit)) return SSM_ERR_DIMS;
    ConvArgs a{};
    a.Bsz = batch; a.T = seqlen; a.C = channels; a.K = static_cast<int>(width);
    a.u = u; a.init = conv_init; a.w = w; a.bias = bias; a.out = out; a.final_state = conv_final;
    return launch_conv(a, dtype == SSM_BF16, false, static_cast<hipStream_t>(stream)) == hipSuccess
               ? SSM_OK
               : SSM_ERR_HIP;
}

size_t ssm_conv1d_silu_workspace_bytes(int64_t batch, int64_t seqlen, int64_t channels,
                                       int64_t width) {
    if (!conv_sizes_ok(batch, seqlen, channels, width)) return static_cast<size_t>(-1);
    return conv_ws_bytes(batch, seqlen, channels, width);
}

ssm_status ssm_conv1d_silu_bwd(int64_t batch, int64_t seqlen, int64_t channels, int64_t width,
                               ssm_dtype dtype, const void *u, const float *w, const float *bias,
                               const void *conv_init, const void *dout, void *du, float *dw,
                               float *dbias, void *dconv_init, void *workspace, size_t ws_bytes,
                               ssm_stream stream) {
    if (!valid_dtype(dtype)) return SSM_ERR_DTYPE;
    if (!conv_sizes_ok(batch, seqlen, channels, width)) return SSM_ERR_DIMS;
    if (!w || !bias || !dw || !dbias) return SSM_ERR_NULL;
    if (batch > 0 && seqlen > 0 && (!u || !dout || !du)) return SSM_ERR_NULL;
    if (!aligned(u, 16) || !aligned(dout, 16) || !aligned(du, 16) || !aligned(bias, 16) ||
        !aligned(conv_init, 16) || !aligned(dconv_init, 16) || !aligned(workspace, 16) ||
        !aligned(w, 4) || !aligned(dw, 4) || !aligned(dbias, 4))
        return SSM_ERR_ALIGN;
    const size_t need = conv_ws_bytes(batch, seqlen, channels, width);
    if (need > 0 && (workspace == nullptr || ws_bytes < need)) return SSM_ERR_WORKSPACE;
    const size_t es = esize(dtype);
    const size_t nrow = static_cast<size_t>(batch) * seqlen * channels * es;
    if (overlaps(du, nrow, u, nrow) || overlaps(du, nrow, dout, nrow)) return SSM_ERR_DIMS;
    ConvArgs a{};
    a.Bsz = batch; a.T = seqlen; a.C = channels; a.K = static_cast<int>(width);
    a.ntiles = conv_bwd_tiles(seqlen);
    a.u = u; a.init = conv_init; a.w = w; a.bias = bias; a.dout = dout; a.du = du;
    a.dinit = dconv_init; a.dw = dw; a.dbias = dbias; a.part = static_cast<double *>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (batch == 0 || seqlen == 0) {  // no tokens: zero parameter gradients and dconv_init
        if (fill(dw, channels * width, s) != hipSuccess || fill(dbias, channels, s) != hipSuccess)
            return SSM_ERR_HIP;
        if (dconv_init && batch > 0 && width > 1) {
            // a float fill covers the bytes of either storage dtype (zero bits are zero)
            const int64_t nbytes = batch * (width - 1) * channels * static_cast<int64_t>(es);
            if (fill(static_cast<float *>(dconv_init), nbytes / 4, s) != hipSuccess) return SSM_ERR_HIP;
        }
        return SSM_OK;
    }
    return launch_conv(a, dtype == SSM_BF16, true, s) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

ssm_status ssm_gated_rmsnorm(int64_t rows, int64_t channels, int64_t ngroups, ssm_dtype dtype,
                             const void *y, const void *z, const float *w, float eps, void *out,
                             ssm_stream stream) {
    if (!valid_dtype(dtype)) return SSM_ERR_DTYPE;
    if (!norm_sizes_ok(rows, channels, ngroups) || !(eps >= 0.f) || eps == INFINITY)
        return SSM_ERR_DIMS;
    if (!w || (rows > 0 && (!y || !z || !out))) return SSM_ERR_NULL;
    if (!aligned(y, 16) || !aligned(z, 16) || !aligned(w, 16) || !aligned(out, 16)) return SSM_ERR_ALIGN;
    NormArgs a{};
    a.rows = rows; a.C = channels; a.G = ngroups; a.eps = eps; a.y = y; a.z = z; a.w = w; a.out = out;
    return launch_norm(a, dtype == SSM_BF16, false, static_cast<hipStream_t>(stream)) == hipSuccess
               ? SSM_OK
               : SSM_ERR_HIP;
}

size_t ssm_gated_rmsnorm_workspace_bytes(int64_t rows, int64_t channels, int64_t ngroups) {
    if (!norm_sizes_ok(rows, channels, ngroups)) return static_cast<size_t>(-1);
    return norm_ws_bytes(rows, channels);
}

ssm_status ssm_gated_rmsnorm_bwd(int64_t rows, int64_t channels, int64_t ngroups,
                                 ssm_dtype dtype, const void *y, const void *z, const float *w,
                                 float eps, const void *dout, void *dy, void *dz, float *dw,
                                 void *workspace, size_t ws_bytes, ssm_stream stream) {
    if (!valid_dtype(dtype)) return SSM_ERR_DTYPE;
    if (!norm_sizes_ok(rows, channels, ngroups) || !(eps >= 0.f) || eps == INFINITY)
        return SSM_ERR_DIMS;
    if (!w || !dw || (rows > 0 && (!y || !z || !dout || !dy || !dz))) return SSM_ERR_NULL;
    if (!aligned(y, 16) || !aligned(z, 16) || !aligned(w, 16) || !aligned(dout, 16) ||
        !aligned(dy, 16) || !aligned(dz, 16) || !aligned(dw, 4) || !aligned(workspace, 16))
        return SSM_ERR_ALIGN;
    const size_t need = norm_ws_bytes(rows, channels);
    if (need > 0 && (workspace == nullptr || ws_bytes < need)) return SSM_ERR_WORKSPACE;
    NormArgs a{};
    a.rows = rows; a.C = channels; a.G = ngroups; a.eps = eps; a.y = y; a.z = z; a.w = w;
    a.dout = dout; a.dy = dy; a.dz = dz; a.dw = dw; a.part = static_cast<double *>(workspace);
    return launch_norm(a, dtype == SSM_BF16, true, static_cast<hipStream_t>(stream)) == hipSuccess
               ? SSM_OK
               : SSM_ERR_HIP;
}

}  // extern "C"
