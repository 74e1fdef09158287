// ssd_fwd.hip -- chunked forward of the selective SSM recurrence on gfx950 MFMA.
//
// Specialised for the Nemotron 3 Ultra head shape (headdim P = 64, dstate
// N = 128; "Nemotron 3 Ultra: replaying a rounded state", section "Counting
// the state and attention cache") with bf16 x, B, C and an fp32 state.
//
// Chunk algebra (exact rearrangement of the recurrence of theorem
// updateHead_apply, same page, "The Mamba state update"; the pages give no
// chunked form, this is derived).  For one (batch, head) and a block of
// Ls = 64 tokens entering with state H (P x N), let a_j = dt_j * A,
// Lam_i = a_0 + ... + a_i (inclusive, local to the block), then
//   h_i  = exp(Lam_i) H + sum_{j<=i} exp(Lam_i - Lam_j) dt_j x_j B_j^T
//   y_i  = C_i . h_i + D x_i
//        = exp(Lam_i) (H C_i) + sum_{j<=i} [(C_i.B_j) exp(Lam_i-Lam_j) dt_j] x_j + D x_i
//   H'   = exp(Lam_63) H + sum_j [exp(Lam_63 - Lam_j) dt_j] x_j B_j^T
// Every exponent is <= 0, so no factor exceeds 1.  The three products
//   G^T = B C^T (Gram of the group's B and C, causal half, masked and decayed),
//   Y^T = H C^T (scaled by exp(Lam)) + X^T Gm^T, with D added to the diagonal of
//         Gm so the same product carries the skip term D x,
//   H'^T = exp(Lam_63) H^T + Bs^T X   (Bs = B scaled per token)
// run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation; the state lives in
// the accumulators of the workgroup for the whole sequence (the inter-block
// pass is the serial loop itself), so HBM sees each input once, y once, and
// the state once per saved chunk.  chunk_states[c] (state entering chunk c)
// is stored whenever a block starts a chunk of L tokens (L % 64 == 0).
//
// One 512-thread workgroup (8 waves) per (batch, head), two per CU (LDS exactly
// 80 KB, at most 128 VGPRs: 16 waves per CU to hide the latency of the serial
// block loop).  Every tile is staged in its natural [token][channel] row layout
// with whole 16-byte row pieces per lane (no bank conflicts); the operands that
// contract over tokens (X^T, Bs^T) are read with gfx950's transposing LDS load.
// Each wave holds 2 x 2 tiles of the state and computes two output tiles of one
// p-tile (one of its state p-tiles, so the X^T fragments serve both products); the
// 10 causal Gram tiles are spread so no wave computes more than two.  Workgroup ids are remapped so the heads of one group run on
// the same XCD and share B/C in that XCD's L2.
//
// MFMA tiles follow the "NT" convention of ssd_common.hpp.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"
#include "ssd_common.hpp"

namespace ssm {
namespace {

// Row stride of the x tile: 40 dwords, so the four rows one transposing read spans
// fall on distinct banks.
constexpr int kSX = kLs + 16;

struct __align__(16) FwdSmem {
    bf16_t C[kLs * kS128];    // [tok][n]
    bf16_t B[kLs * kS128];    // [tok][n]; after the Gram product: H in bf16, [p][n]
    bf16_t Bs[kLs * kS128];   // [tok][n] = B[tok][n] * exp(Lam_63 - Lam_tok) * dt_tok
    bf16_t X[kLs * kSX];      // [tok][p]
    bf16_t Gm[kLs * kS64];    // [i][j] = (C_i.B_j) exp(Lam_i - Lam_j) dt_j for j <= i, else 0
    float2 ld[2][kLs];        // (Lam, dt) per token, double-buffered by block parity
    bf16_t Y[kLs * kS64];     // [tok][p]: the block's outputs, stored to HBM as whole rows
};
static_assert(sizeof(FwdSmem) <= 81920, "two workgroups per CU");

// DEPTH: blocks of rows held in registers ahead of the one being computed.  1 when two
// workgroups share a CU (at most 128 registers); 2 when the grid has fewer (batch, head)
// pairs than two per CU, so each workgroup has a CU to itself and nothing else covers its
// load latency (batch 1 at long context).  The arithmetic is the same either way.
template <int DEPTH>
__global__ void __launch_bounds__(512) ssd_fwd_kernel(SsdFwdArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    FwdSmem &sm = *reinterpret_cast<FwdSmem *>(smem_raw);
    const int nwg = gridDim.x;
    const int bh = xcd_remap(blockIdx.x, nwg);
    const int b = bh / a.H, h = bh % a.H, g = h / (a.H / a.G);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 15, lk = (lane >> 4) * 8, lq = (lane >> 4) * 4;
    const int64_t T = a.T;
    const float Ah = a.A[h], Dh = a.D[h];
    const bf16_t *x = static_cast<const bf16_t *>(a.x);
    const bf16_t *Bm = static_cast<const bf16_t *>(a.B);
    const bf16_t *Cm = static_cast<const bf16_t *>(a.C);
    bf16_t *y = static_cast<bf16_t *>(a.y);

    // Output tiles Y^T of wave w: p-tile pw, token tiles 2 ih + {0, 1}.  State H^T of wave w:
    // tile q = n-tile 2 (w % 4) + q / 2, p-tile pw ^ (q % 2) (the output's p-tile and its
    // neighbour), so the state update reuses the X^T fragments the output product read.
    // Lane layout of a state tile: n = 16 nt + lq + v, p = 16 pt + lr.
    const int pw = 2 * (wave >> 2) + (wave & 1), ih = (wave >> 1) & 1;
    auto st_n = [&](int q) { return 16 * (2 * (wave & 3) + (q >> 1)) + lq; };
    auto st_p = [&](int q) { return 16 * (pw ^ (q & 1)) + lr; };
    f32x4 H[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int n = st_n(q), p = st_p(q);
        if (a.h0 != nullptr) {
            const float4 v = *reinterpret_cast<const float4 *>(a.h0 + (static_cast<int64_t>(bh) * kP + p) * kN + n);
            H[q] = f32x4{v.x, v.y, v.z, v.w};
        } else {
            H[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    // staging map: B, C, Bs rows rt and rt + 32 from coordinate rc; x (and y) row xt from
    // channel xc.  A wave covers whole rows, 16 contiguous bytes per lane.
    const int rt = tid >> 4, rc = (tid & 15) * 8;
    const int xt = tid >> 3, xc = (tid & 7) * 8;
    struct Rows {
        u16x8 v[5];  // B rows rt, rt + 32; C rows rt, rt + 32; x row xt
        float dt;    // dt of token `tid` (wave 0)
    };
    const uint32_t tokx = static_cast<uint32_t>(a.H) * kP * 2;
    const uint32_t tokbc = static_cast<uint32_t>(a.G) * kN * 2;
    // Per-block pointers advance by a fixed stride (no 64-bit multiply or divide in the
    // loop); the buffer range check zeroes / drops the ragged tail.
    const int64_t sx = static_cast<int64_t>(kLs) * a.H * kP;   // elements between blocks of x, y
    const int64_t sbc = static_cast<int64_t>(kLs) * a.G * kN;  // ... of B, C
    const int64_t sdt = static_cast<int64_t>(kLs) * a.H;       // ... of dt
    const bf16_t *px = x + (b * T * a.H + h) * kP;  // next block to prefetch
    const bf16_t *pB = Bm + (b * T * a.G + g) * kN;
    const bf16_t *pC = Cm + (b * T * a.G + g) * kN;
    const float *pdt = a.dt + b * T * a.H + h;
    bf16_t *py = y + (b * T * a.H + h) * kP;        // block being computed
    auto nvalid_of = [&](int64_t rem) { return static_cast<uint32_t>(rem < kLs ? rem : kLs); };
    auto prefetch = [&](Rows &R, int64_t rem) {  // rem: tokens from the prefetched block to the end
        const uint32_t nv = nvalid_of(rem);
        const rsrc_t rb = make_rsrc(pB, nv * tokbc), rcc = make_rsrc(pC, nv * tokbc);
        const rsrc_t rx = make_rsrc(px, nv * tokx);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            R.v[i] = buf_ld_16b(rb, (rt + 32 * i) * tokbc + rc * 2);
            R.v[2 + i] = buf_ld_16b(rcc, (rt + 32 * i) * tokbc + rc * 2);
        }
        R.v[4] = buf_ld_16b(rx, xt * tokx + xc * 2);
        R.dt = 0.f;
        if (tid < kLs) {
            const rsrc_t rd = make_rsrc(pdt, nv * a.H * 4u);
            R.dt = buf_ld_f32(rd, static_cast<uint32_t>(tid) * a.H * 4u);
        }
        px += sx;
        pB += sbc;
        pC += sbc;
        pdt += sdt;
    };
    // Outputs leave through LDS: each thread stores 16 bytes of one token row, so a
    // wave writes 8 tokens x 128 B (whole rows of this head) per instruction instead
    // of 16 tokens x 32 B from the MFMA accumulator layout.
    auto store_y = [&](int64_t tb) {
        const rsrc_t ry = make_rsrc(py, nvalid_of(T - tb) * tokx);
        const u16x8 v = *reinterpret_cast<const u16x8 *>(&sm.Y[xt * kS64 + xc]);
        buf_st_16b(ry, static_cast<uint32_t>(xt) * tokx + xc * 2, v);
        py += sx;
    };
    // Gram tile assignment (i-tile, j-tiles): every tile with j <= i once, plus the two
    // zero tiles (0,1) and (2,3) that the output products read
    const int gi = (wave < 2) ? 3 : (wave < 4) ? 2 : (wave < 6) ? 1 : 0;
    const int gj0 = (wave == 0) ? 0 : (wave == 1) ? 2 : (wave == 2) ? 0 : (wave == 3) ? 2 : (wave == 4) ? 0 : (wave == 5) ? 1 : 0;
    const int gnj = (wave <= 3) ? 2 : (wave == 6) ? 2 : (wave == 7) ? 0 : 1;  // waves 3, 6 write a zero second tile

    const int64_t nblk = (T + kLs - 1) / kLs;
    const int bpc = static_cast<int>(a.L / kLs);  // blocks per chunk
    int kc = 0;                                   // block index within its chunk
    float *cs = (a.chunk_states != nullptr) ? a.chunk_states + static_cast<int64_t>(bh) * a.nchunks * (kP * kN) : nullptr;
    // one block; R holds its rows and is refilled with block s + DEPTH
    auto step = [&](int64_t s, Rows &R) {
        const int64_t t0 = s * kLs;
        const int buf = static_cast<int>(s & 1);
        // (1) cumulative log-retention of the block (one wave, one token per lane)
        if (wave == 0) sm.ld[buf][lane] = make_float2(wave_prefix_sum(R.dt * Ah), R.dt);
        __syncthreads();
        const float2 *ld = sm.ld[buf];
        const float lam_end = ld[kLs - 1].x;
        // (2) stage the block in LDS: B, C, Bs = B scaled per token, x
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = rt + 32 * i;
            *reinterpret_cast<u16x8 *>(&sm.B[r * kS128 + rc]) = R.v[i];
            *reinterpret_cast<u16x8 *>(&sm.C[r * kS128 + rc]) = R.v[2 + i];
            const float2 lt = ld[r];
            const float cf = __expf(lam_end - lt.x) * lt.y;
            const u16x8 v = R.v[i];
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 w = {pack2_bf16(bf16_to_f32(v[0]) * cf, bf16_to_f32(v[1]) * cf),
                             pack2_bf16(bf16_to_f32(v[2]) * cf, bf16_to_f32(v[3]) * cf),
                             pack2_bf16(bf16_to_f32(v[4]) * cf, bf16_to_f32(v[5]) * cf),
                             pack2_bf16(bf16_to_f32(v[6]) * cf, bf16_to_f32(v[7]) * cf)};
            *reinterpret_cast<u32x4 *>(&sm.Bs[r * kS128 + rc]) = w;
        }
        *reinterpret_cast<u16x8 *>(&sm.X[xt * kSX + xc]) = R.v[4];
        __syncthreads();
        // This phase's stores go out after the staging barrier rather than before the
        // staging writes (0.559 -> 0.550 ms): the previous block's outputs (complete since
        // the first barrier, rewritten only after the fourth) and the state entering a
        // chunk of L tokens (H changes only in the state update).
        if (s > 0) store_y(t0 - kLs);
        if (cs != nullptr && kc == 0) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = st_n(q), p = st_p(q);
                *reinterpret_cast<float4 *>(cs + p * kN + n) = make_float4(H[q][0], H[q][1], H[q][2], H[q][3]);
            }
            cs += kP * kN;
        }
        if (++kc == bpc) kc = 0;
        // (3) masked, decayed Gram tiles (i-tile gi, j-tiles gj0, gj0+1); the wave's C
        //     fragments are read once for both
        if (gnj > 0) {
            const int i = 16 * gi + lr;
            const float lam_i = ld[i].x;
            bf16x8 fc[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) fc[kk] = frag_row(&sm.C[i * kS128 + 32 * kk + lk]);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                if (q >= gnj) break;
                const int jt = gj0 + q;
                float gv[4] = {0.f, 0.f, 0.f, 0.f};
                if (jt <= gi) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        acc = mfma(frag_row(&sm.B[(16 * jt + lr) * kS128 + 32 * kk + lk]), fc[kk], acc);
                    const float4 l01 = *reinterpret_cast<const float4 *>(&ld[16 * jt + lq]);
                    const float4 l23 = *reinterpret_cast<const float4 *>(&ld[16 * jt + lq + 2]);
                    const float2 ljs[4] = {make_float2(l01.x, l01.y), make_float2(l01.z, l01.w),
                                           make_float2(l23.x, l23.y), make_float2(l23.z, l23.w)};
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int j = 16 * jt + lq + v;
                        const float2 lj = ljs[v];
                        gv[v] = (j <= i) ? acc[v] * __expf(lam_i - lj.x) * lj.y : 0.f;
                        if (j == i) gv[v] += Dh;
                    }
                }
                *reinterpret_cast<u16x4 *>(&sm.Gm[i * kS64 + 16 * jt + lq]) = pack4(gv[0], gv[1], gv[2], gv[3]);
            }
        }
        __syncthreads();
        // (4) H in bf16 over the consumed B rows: [p][n]
        bf16_t *Hb = sm.B;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = st_n(q), p = st_p(q);
            *reinterpret_cast<u16x4 *>(&Hb[p * kS128 + n]) = pack4(H[q][0], H[q][1], H[q][2], H[q][3]);
        }
        __syncthreads();
        // The next block's rows are requested here, after the Gram and H phases: the
        // kernel took 0.61 ms with the request at the end of staging, 0.57 after the Gram
        // barrier, 0.56 here and 0.62 or more later in this phase.
        if (s + DEPTH < nblk) prefetch(R, T - t0 - DEPTH * kLs);
        // (5) outputs Y^T: p-tile pw, token tiles 2 ih + {0, 1}; the wave's H and X^T
        //     fragments are read once for both, and X^T again serves the state update
        {
            const int prow = 16 * pw + lr;
            bf16x8 fh[4], fx[2];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) fh[kk] = frag_row(&Hb[prow * kS128 + 32 * kk + lk]);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) fx[kk] = frag_tr(sm.X, kSX, 16 * pw, 32 * kk, lane);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int tt = 2 * ih + q;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    acc = mfma(fh[kk], frag_row(&sm.C[(16 * tt + lr) * kS128 + 32 * kk + lk]), acc);
                const int tok = 16 * tt + lr;
                const float el = __expf(ld[tok].x);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[v] *= el;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if (kk > ih) break;
                    acc = mfma(fx[kk], frag_row(&sm.Gm[(16 * tt + lr) * kS64 + 32 * kk + lk]), acc);
                }
                *reinterpret_cast<u16x4 *>(&sm.Y[tok * kS64 + 16 * pw + lq]) = pack4(acc[0], acc[1], acc[2], acc[3]);
            }
            // (6) state update H^T = exp(Lam_63) H^T + Bs^T X on the wave's 2 x 2 state tiles
            const float el = __expf(lam_end);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int v = 0; v < 4; ++v) H[q][v] *= el;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 fo = frag_tr(sm.X, kSX, 16 * (pw ^ 1), 32 * kk, lane);  // the other p-tile
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const bf16x8 fb = frag_tr(sm.Bs, kS128, 16 * (2 * (wave & 3) + t), 32 * kk, lane);
                    H[2 * t] = mfma(fb, fx[kk], H[2 * t]);
                    H[2 * t + 1] = mfma(fb, fo, H[2 * t + 1]);
                }
            }
        }
    };
    Rows RA, RB;
    prefetch(RA, T);
    if (DEPTH == 1) {
        for (int64_t s = 0; s < nblk; ++s) step(s, RA);
    } else {
        if (nblk > 1) prefetch(RB, T - kLs);
        for (int64_t s = 0; s < nblk; s += 2) {
            step(s, RA);
            if (s + 1 < nblk) step(s + 1, RB);
        }
    }
    __syncthreads();
    if (nblk > 0) store_y((nblk - 1) * kLs);
    if (a.h_final != nullptr) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = st_n(q), p = st_p(q);
            *reinterpret_cast<float4 *>(a.h_final + (static_cast<int64_t>(bh) * kP + p) * kN + n) =
                make_float4(H[q][0], H[q][1], H[q][2], H[q][3]);
        }
    }
}

}  // namespace

hipError_t launch_ssd_fwd(const SsdFwdArgs &a, hipStream_t s) {
    const size_t smem = sizeof(FwdSmem);
    // The dynamic-LDS limit is a per-device attribute of the kernel: set it once on
    // every device this process launches on.
    static std::atomic<uint64_t> configured{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t{1} << dev) : 0;
    if (bit == 0 || (configured.load() & bit) == 0) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&ssd_fwd_kernel<1>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
        if (e != hipSuccess) return e;
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&ssd_fwd_kernel<2>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
        if (e != hipSuccess) return e;
        configured.fetch_or(bit);
    }
    int cus = 0;
    if ((e = device_cu_count(&cus)) != hipSuccess) return e;
    const int64_t nbh = a.Bsz * a.H;
    const unsigned grid = static_cast<unsigned>(nbh);
    if (nbh >= 2 * static_cast<int64_t>(cus))
        ssd_fwd_kernel<1><<<grid, 512, smem, s>>>(a);
    else
        ssd_fwd_kernel<2><<<grid, 512, smem, s>>>(a);
    return hipGetLastError();
}

}  // namespace ssm
