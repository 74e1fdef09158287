// Host stand-ins for the library's kernel launchers and for the one HIP runtime call the
// boundary makes itself.  Linked with abi.cpp into a host-only program built with
// AddressSanitizer and UndefinedBehaviorSanitizer (no GPU, no HIP runtime).
//
// Every launcher counts that it ran.  The launchers of calls that take a workspace also
// fill each workspace region the real kernels index (extents restated from the kernels'
// indexing) with its own byte, then check that every region still holds its byte: a
// region that runs past the caller's buffer is an AddressSanitizer error, and two regions
// that overlap fail the check.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "launch.hpp"
#include "stubs.hpp"

namespace stub {
int launches = 0;
int overlaps = 0;
}  // namespace stub

namespace {

struct Region {
    void *p;
    size_t bytes;
};

void fill_and_check(std::initializer_list<Region> regions) {
    unsigned char tag = 1;
    for (const Region &r : regions) std::memset(r.p, tag++, r.bytes);
    tag = 1;
    for (const Region &r : regions) {
        const unsigned char *b = static_cast<const unsigned char *>(r.p);
        for (size_t i = 0; i < r.bytes; ++i)
            if (b[i] != tag) {
                ++stub::overlaps;
                std::fprintf(stderr, "workspace region %d overwritten at byte %zu\n", tag, i);
                break;
            }
        ++tag;
    }
}

}  // namespace

extern "C" hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }

namespace ssm {
// the no-allocation backward's scratch: a host buffer of the stated size
hipError_t noalloc_scratch(void **ptr) {
    static void *buf = std::aligned_alloc(256, kNoAllocScratchBytes);
    *ptr = buf;
    return buf ? hipSuccess : hipErrorOutOfMemory;
}
}  // namespace ssm

namespace ssm {

hipError_t launch_fill(float *, int64_t, float, hipStream_t) { ++stub::launches; return hipSuccess; }
hipError_t launch_copy(float *, const float *, int64_t, hipStream_t) { ++stub::launches; return hipSuccess; }
hipError_t launch_decode(const DecodeArgs &, bool, hipStream_t) { ++stub::launches; return hipSuccess; }
hipError_t launch_rollback(const RollbackArgs &, hipStream_t) { ++stub::launches; return hipSuccess; }
hipError_t launch_sr16(const Sr16Args &, hipStream_t) { ++stub::launches; return hipSuccess; }
hipError_t launch_ssd_fwd(const SsdFwdArgs &, hipStream_t) { ++stub::launches; return hipSuccess; }
hipError_t launch_dt_prep(const DtPrepArgs &, hipStream_t) { ++stub::launches; return hipSuccess; }

hipError_t launch_scan(const ScanArgs &a, bool, bool, hipStream_t) {
    ++stub::launches;
    if (a.live != nullptr) {  // per-step, per-wave drift partials: [r][Bsz * H * 4]
        const size_t n = static_cast<size_t>(a.r) * a.Bsz * a.H * 4 * sizeof(float);
        fill_and_check({{a.part_max, n}, {a.part_sum, n}});
    }
    return hipSuccess;
}

hipError_t launch_drift_reduce(const float *, const float *, int64_t, int64_t, double, float *,
                               float *, hipStream_t) {
    ++stub::launches;
    return hipSuccess;
}

hipError_t launch_scan_bwd(const ScanBwdArgs &a, bool, hipStream_t) {
    ++stub::launches;
    const size_t bh = static_cast<size_t>(a.Bsz) * a.H;
    const size_t part = static_cast<size_t>(a.Bsz) * a.T * a.H * a.N * sizeof(float);
    fill_and_check({{a.slab, bh * a.slab_stride * sizeof(float)},
                    {a.dB_part, part},
                    {a.dC_part, part},
                    {a.dA_part, bh * sizeof(double)},
                    {a.dD_part, bh * sizeof(double)}});
    return hipSuccess;
}

hipError_t launch_ssd_bwd(const SsdBwdArgs &a, hipEvent_t, hipEvent_t, hipStream_t) {
    ++stub::launches;
    const size_t units = static_cast<size_t>(a.Bsz) * a.H * a.nchunks;
    fill_and_check({{a.dstates, units * kP * kN * sizeof(bf16_t)},
                    {a.pA, units * (a.L / kLs) * sizeof(double)},
                    {a.pD, units * (a.L / kLs) * sizeof(double)}});
    return hipSuccess;
}

hipError_t launch_dt_prep_bwd(const DtPrepArgs &a, hipStream_t) {
    ++stub::launches;
    const size_t n = static_cast<size_t>(dt_prep_row_tiles(a.rows)) * a.H * sizeof(double);
    if (n > 0) fill_and_check({{a.part, n}});
    return hipSuccess;
}

hipError_t launch_conv(const ConvArgs &a, bool, bool bwd, hipStream_t) {
    ++stub::launches;
    if (bwd) {
        const size_t n = static_cast<size_t>(a.Bsz) * a.ntiles * (a.K + 1) * a.C * sizeof(double);
        if (n > 0) fill_and_check({{a.part, n}});
    }
    return hipSuccess;
}

hipError_t launch_norm(const NormArgs &a, bool, bool bwd, hipStream_t) {
    ++stub::launches;
    if (bwd) {
        const size_t n = static_cast<size_t>(norm_row_tiles(a.rows)) * a.C * sizeof(double);
        if (n > 0) fill_and_check({{a.part, n}});
    }
    return hipSuccess;
}

}  // namespace ssm
