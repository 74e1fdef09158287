// Host-only driver of the C boundary (include/ssm.h) for the sanitized build: every call
// below either fails validation -- and must then return the documented status with no
// launcher reached ("Reverse-mode automatic differentiation" (OneModel docs), section 2:
// errors are detected before any work) -- or is a valid call whose workspace is a real
// host buffer of exactly the size ssm_workspace_bytes reports, which the stand-in
// launchers fill region by region.  Device pointers that validation never dereferences
// are a fixed 256-byte-aligned address.  Exit status 0 when every check holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "ssm.h"
#include "stubs.hpp"

namespace {

int failures = 0;
void *const F = reinterpret_cast<void *>(uintptr_t{0x7F0000000000});  // never dereferenced
float *const Ff = static_cast<float *>(F);
char *const Fc = static_cast<char *>(F);

#define EXPECT(cond)                                                           \
    do {                                                                       \
        if (!(cond)) {                                                         \
            ++failures;                                                        \
            std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
        }                                                                      \
    } while (0)

// an invalid call: the expected status and no launcher reached
#define REJECT(status, call)                                                   \
    do {                                                                       \
        const int before = stub::launches;                                     \
        const ssm_status got = (call);                                         \
        if (got != (status) || stub::launches != before) {                     \
            ++failures;                                                        \
            std::fprintf(stderr, "%s:%d: %s -> %d (expected %d), launches %d\n", __FILE__, \
                         __LINE__, #call, static_cast<int>(got), static_cast<int>(status), \
                         stub::launches - before);                             \
        }                                                                      \
    } while (0)

// a valid call: SSM_OK and at least one launcher reached
#define ACCEPT(call)                                                           \
    do {                                                                       \
        const int before = stub::launches;                                     \
        const ssm_status got = (call);                                         \
        if (got != SSM_OK || stub::launches == before) {                       \
            ++failures;                                                        \
            std::fprintf(stderr, "%s:%d: %s -> %d, launches %d\n", __FILE__, __LINE__, #call, \
                         static_cast<int>(got), stub::launches - before);      \
        }                                                                      \
    } while (0)

ssm_dims dims(int64_t b, int64_t t, int64_t h, int64_t p, int64_t n, int64_t g, int64_t L) {
    return ssm_dims{b, t, h, p, n, g, L};
}

// a host buffer of exactly `bytes` bytes standing in for the device workspace
struct Ws {
    void *p = nullptr;
    size_t n = 0;
    explicit Ws(size_t bytes) : n(bytes) { p = bytes ? std::aligned_alloc(256, (bytes + 255) / 256 * 256) : nullptr; }
    ~Ws() { std::free(p); }
};

ssm_status fwd(const ssm_dims *d, ssm_dtype t, void *x = F, void *y = F, float *h0 = nullptr) {
    return ssm_fwd_chunked(d, t, x, F, F, Ff, Ff, Ff, h0, y, nullptr, nullptr, nullptr, 0, nullptr);
}

ssm_status bwd(const ssm_dims *d, ssm_dtype t, void *ws, size_t wsb, const float *cs = Ff) {
    return ssm_bwd(d, t, F, F, F, Ff, Ff, Ff, cs, F, nullptr, F, Ff, Ff, Ff, Ff, Ff, nullptr, ws,
                   wsb, nullptr);
}

void chunked() {
    const ssm_dims d = dims(2, 100, 4, 64, 128, 2, 64);
    REJECT(SSM_ERR_NULL, fwd(nullptr, SSM_BF16));
    const ssm_dims bad_groups = dims(2, 100, 6, 64, 128, 4, 64);
    REJECT(SSM_ERR_DIMS, fwd(&bad_groups, SSM_BF16));
    const ssm_dims zero_chunk = dims(2, 100, 4, 64, 128, 2, 0);
    REJECT(SSM_ERR_DIMS, fwd(&zero_chunk, SSM_BF16));
    const ssm_dims neg_batch = dims(-1, 100, 4, 64, 128, 2, 64);
    REJECT(SSM_ERR_DIMS, fwd(&neg_batch, SSM_BF16));
    REJECT(SSM_ERR_DTYPE, fwd(&d, static_cast<ssm_dtype>(7)));
    const ssm_dims odd_state = dims(2, 100, 4, 64, 100, 2, 64);
    REJECT(SSM_ERR_UNSUPPORTED, fwd(&odd_state, SSM_BF16));
    REJECT(SSM_ERR_NULL, fwd(&d, SSM_BF16, nullptr));
    REJECT(SSM_ERR_ALIGN, fwd(&d, SSM_BF16, F, Fc + 2));
    REJECT(SSM_ERR_ALIGN, fwd(&d, SSM_BF16, F, F, Ff + 2));
    ACCEPT(fwd(&d, SSM_BF16));
    const ssm_dims no_batch = dims(0, 100, 4, 64, 128, 2, 64);
    REJECT(SSM_OK, fwd(&no_batch, SSM_BF16, nullptr, nullptr));  // nothing to do

    // backward: chunked MFMA path and the exact-fp32 path, each with an exact workspace
    for (int pass = 0; pass < 2; ++pass) {
        const ssm_dims db = pass == 0 ? dims(2, 300, 8, 64, 128, 2, 128) : dims(2, 37, 4, 8, 16, 2, 16);
        const ssm_dtype t = pass == 0 ? SSM_BF16 : SSM_F32;
        EXPECT(ssm_uses_mfma_path(&db, t) == (pass == 0));
        const size_t need = ssm_workspace_bytes(&db, t, SSM_WS_BWD, 0);
        EXPECT(need > 0 && need != static_cast<size_t>(-1));
        REJECT(SSM_ERR_WORKSPACE, bwd(&db, t, nullptr, 0));
        REJECT(SSM_ERR_WORKSPACE, bwd(&db, t, F, need - 1));
        REJECT(SSM_ERR_ALIGN, bwd(&db, t, Fc + 8, need));
        REJECT(SSM_ERR_NULL, bwd(&db, t, F, need, nullptr));
        Ws ws(need);
        const int ov = stub::overlaps;
        ACCEPT(bwd(&db, t, ws.p, ws.n));
        EXPECT(stub::overlaps == ov);
    }
    // the timed backward: events required, validated like ssm_bwd
    const ssm_dims db = dims(2, 300, 8, 64, 128, 2, 128);
    const size_t need = ssm_workspace_bytes(&db, SSM_BF16, SSM_WS_BWD, 0);
    void *nullev[2] = {nullptr, nullptr};
    REJECT(SSM_ERR_NULL, ssm_bwd_timed(&db, SSM_BF16, F, F, F, Ff, Ff, Ff, Ff, F, nullptr, F, Ff,
                                       Ff, Ff, Ff, Ff, nullptr, F, need, nullptr, nullptr));
    REJECT(SSM_ERR_NULL, ssm_bwd_timed(&db, SSM_BF16, F, F, F, Ff, Ff, Ff, Ff, F, nullptr, F, Ff,
                                       Ff, Ff, Ff, Ff, nullptr, F, need, nullev, nullptr));
    void *ev[2] = {F, Fc + 256};  // the stand-in hipEventRecord accepts any handle
    Ws ws(need);
    ACCEPT(ssm_bwd_timed(&db, SSM_BF16, F, F, F, Ff, Ff, Ff, Ff, F, nullptr, F, Ff, Ff, Ff, Ff, Ff,
                         nullptr, ws.p, ws.n, ev, nullptr));
    // the no-allocation backward: up to the library's scratch, whose regions it carves
    auto noalloc = [&](const ssm_dims *dd, const float *cs) {
        return ssm_bwd_noalloc(dd, SSM_BF16, F, F, F, Ff, Ff, Ff, cs, F, nullptr, F, Ff, Ff, Ff,
                               Ff, Ff, nullptr, nullptr);
    };
    const ssm_dims one_seq = dims(1, 4096, 256, 64, 128, 8, 256);   // fits the scratch
    const ssm_dims two_seq = dims(2, 4096, 256, 64, 128, 8, 256);   // does not
    EXPECT(ssm_workspace_bytes(&one_seq, SSM_BF16, SSM_WS_BWD, 0) <= SSM_NOALLOC_SCRATCH_BYTES);
    REJECT(SSM_ERR_WORKSPACE, noalloc(&two_seq, Ff));
    REJECT(SSM_ERR_DIMS, noalloc(&bad_groups, Ff));
    REJECT(SSM_ERR_NULL, noalloc(&one_seq, nullptr));
    {
        const int ov = stub::overlaps;
        ACCEPT(noalloc(&one_seq, Ff));
        ACCEPT(noalloc(&db, Ff));
        EXPECT(stub::overlaps == ov);
    }
    EXPECT(ssm_workspace_bytes(&odd_state, SSM_BF16, SSM_WS_BWD, 0) == static_cast<size_t>(-1));
    EXPECT(ssm_workspace_bytes(&d, static_cast<ssm_dtype>(9), SSM_WS_FWD, 0) == static_cast<size_t>(-1));
}

void decode_replay() {
    const ssm_dims d = dims(2, 1, 4, 64, 128, 2, 1);
    auto dec = [&](const ssm_dims *dd, float *state) {
        return ssm_decode_step(dd, SSM_BF16, state, F, F, F, Ff, Ff, Ff, F, nullptr);
    };
    REJECT(SSM_ERR_NULL, dec(&d, nullptr));
    REJECT(SSM_ERR_ALIGN, dec(&d, Ff + 1));
    const ssm_dims odd_state = dims(2, 1, 4, 64, 48, 2, 1);
    REJECT(SSM_ERR_UNSUPPORTED, dec(&odd_state, Ff));
    ACCEPT(dec(&d, Ff));
    auto dec16 = [&](uint16_t *s16) {
        return ssm_decode_step_sr16(&d, SSM_BF16, s16, F, F, F, Ff, Ff, Ff, F, 1, 2, nullptr);
    };
    REJECT(SSM_ERR_ALIGN, dec16(reinterpret_cast<uint16_t *>(Fc + 2)));
    ACCEPT(dec16(static_cast<uint16_t *>(F)));
    auto sr = [&](const float *s, uint16_t *o, uint64_t n) {
        return ssm_checkpoint_sr16(s, o, n, 0, 0, 0, nullptr);
    };
    REJECT(SSM_ERR_NULL, sr(nullptr, static_cast<uint16_t *>(F), 10));
    REJECT(SSM_ERR_DIMS, sr(Ff, reinterpret_cast<uint16_t *>(Fc + 16), 10));  // aliasing
    REJECT(SSM_OK, sr(nullptr, nullptr, 0));
    ACCEPT(sr(Ff, reinterpret_cast<uint16_t *>(Fc + 4096), 10));

    const ssm_dims rd = dims(2, 50, 4, 64, 128, 2, 1);
    auto rep = [&](int64_t t0, int64_t r, const float *live, float *dm, void *ws, size_t wsb) {
        return ssm_replay(&rd, SSM_BF16, F, SSM_F16, Ff, F, F, F, Ff, Ff, Ff, t0, r, nullptr, live,
                          dm, dm, ws, wsb, nullptr);
    };
    REJECT(SSM_ERR_DIMS, rep(40, 11, nullptr, nullptr, nullptr, 0));
    REJECT(SSM_ERR_DIMS, rep(-1, 5, nullptr, nullptr, nullptr, 0));
    REJECT(SSM_ERR_NULL, rep(0, 5, Ff, nullptr, nullptr, 0));
    const size_t need = ssm_workspace_bytes(&rd, SSM_BF16, SSM_WS_REPLAY, 7);
    REJECT(SSM_ERR_WORKSPACE, rep(0, 7, Ff, Ff, F, need - 1));
    Ws ws(need);
    const int ov = stub::overlaps;
    ACCEPT(rep(3, 7, Ff, Ff, ws.p, ws.n));
    EXPECT(stub::overlaps == ov);
    ACCEPT(rep(0, 50, nullptr, nullptr, nullptr, 0));
}

void prep_draft_conv_norm() {
    const ssm_dims d = dims(4, 100, 256, 1, 1, 1, 1);
    REJECT(SSM_ERR_DIMS, ssm_dt_prep(&d, Ff, Ff, Ff, 1.f, 0.5f, Ff, Ff, nullptr));
    REJECT(SSM_ERR_DIMS, ssm_dt_prep(&d, Ff, Ff, Ff, NAN, 1.f, Ff, Ff, nullptr));
    ACCEPT(ssm_dt_prep(&d, Ff, Ff, Ff, 0.f, INFINITY, Ff, Ff, nullptr));
    const size_t need = ssm_workspace_bytes(&d, SSM_F32, SSM_WS_DT_PREP_BWD, 0);
    REJECT(SSM_ERR_WORKSPACE, ssm_dt_prep_bwd(&d, Ff, Ff, Ff, 0.f, 1.f, Ff, Ff, Ff, Ff, Ff, F,
                                              need - 1, nullptr));
    {
        Ws ws(need);
        const int ov = stub::overlaps;
        ACCEPT(ssm_dt_prep_bwd(&d, Ff, Ff, Ff, 0.f, 1.f, Ff, Ff, Ff, Ff, Ff, ws.p, ws.n, nullptr));
        EXPECT(stub::overlaps == ov);
    }

    const ssm_dims dr = dims(2, 4, 8, 64, 128, 2, 1);
    ACCEPT(ssm_draft_snapshots(&dr, SSM_BF16, Ff, F, F, F, Ff, Ff, Ff, F, nullptr));
    REJECT(SSM_ERR_ALIGN, ssm_draft_snapshots(&dr, SSM_BF16, Ff + 1, F, F, F, Ff, Ff, Ff, F, nullptr));
    const size_t slot = size_t{2} * 8 * 64 * 128;  // floats per snapshot slot
    int32_t *acc = reinterpret_cast<int32_t *>(Fc + (size_t{1} << 32));
    REJECT(SSM_ERR_DIMS, ssm_rollback(&dr, Ff, acc, Ff + 4, nullptr, nullptr));  // straddles slots
    ACCEPT(ssm_rollback(&dr, Ff, acc, Ff, nullptr, nullptr));                   // into slot 0
    ACCEPT(ssm_rollback(&dr, Ff, acc, Ff + 2 * slot, nullptr, nullptr));        // into slot 2

    REJECT(SSM_ERR_DIMS, ssm_conv1d_silu(2, 64, 16, 9, SSM_BF16, F, Ff, Ff, nullptr, Fc + 65536,
                                         nullptr, nullptr));
    REJECT(SSM_ERR_DIMS, ssm_conv1d_silu(2, 64, 18, 4, SSM_BF16, F, Ff, Ff, nullptr, Fc + 65536,
                                         nullptr, nullptr));
    REJECT(SSM_ERR_DIMS, ssm_conv1d_silu(2, 64, 16, 4, SSM_BF16, F, Ff, Ff, nullptr, Fc + 16,
                                         nullptr, nullptr));  // out overlaps u
    ACCEPT(ssm_conv1d_silu(2, 64, 16, 4, SSM_BF16, F, Ff, Ff, nullptr, Fc + 65536, nullptr, nullptr));
    {
        const size_t cneed = ssm_conv1d_silu_workspace_bytes(2, 1000, 16, 4);
        EXPECT(cneed > 0 && cneed != static_cast<size_t>(-1));
        REJECT(SSM_ERR_WORKSPACE, ssm_conv1d_silu_bwd(2, 1000, 16, 4, SSM_BF16, F, Ff, Ff, nullptr,
                                                      Fc + 65536, Fc + 131072, Ff, Ff, nullptr, F,
                                                      cneed - 1, nullptr));
        Ws ws(cneed);
        const int ov = stub::overlaps;
        ACCEPT(ssm_conv1d_silu_bwd(2, 1000, 16, 4, SSM_BF16, F, Ff, Ff, nullptr, Fc + 65536,
                                   Fc + 131072, Ff, Ff, nullptr, ws.p, ws.n, nullptr));
        EXPECT(stub::overlaps == ov);
    }
    REJECT(SSM_ERR_DIMS, ssm_gated_rmsnorm(10, 20, 2, SSM_BF16, F, F, Ff, 1e-5f, F, nullptr));
    REJECT(SSM_ERR_DIMS, ssm_gated_rmsnorm(10, 32, 2, SSM_BF16, F, F, Ff, -1.f, F, nullptr));
    ACCEPT(ssm_gated_rmsnorm(10, 32, 2, SSM_BF16, F, F, Ff, 1e-5f, F, nullptr));
    {
        const size_t nneed = ssm_gated_rmsnorm_workspace_bytes(1000, 64, 2);
        EXPECT(nneed > 0 && nneed != static_cast<size_t>(-1));
        Ws ws(nneed);
        const int ov = stub::overlaps;
        ACCEPT(ssm_gated_rmsnorm_bwd(1000, 64, 2, SSM_F32, F, F, Ff, 1e-5f, F, F, F, Ff, ws.p, ws.n,
                                     nullptr));
        EXPECT(stub::overlaps == ov);
    }
}

}  // namespace

int main() {
    chunked();
    decode_replay();
    prep_draft_conv_norm();
    for (int s = 0; s <= 8; ++s) EXPECT(ssm_status_string(static_cast<ssm_status>(s)) != nullptr);
    std::printf("%s: %d failures, %d launcher calls\n", failures ? "FAIL" : "OK", failures,
                stub::launches);
    return failures ? 1 : 0;
}
