// ssd_bwd.hip -- reverse-mode backward of the chunked selective SSM recurrence
// on gfx950 MFMA (headdim 64, dstate 128, bf16 x/B/C/dy, fp32 state).
//
// "Nemotron Kernels: From Inference To Backpropagation", Kernel 1
// "Backpropagation: What Mamba2 Backward Must Do": the reverse walk runs from
// the last token to the first, the gradient reaching a state is the output
// path plus the future recurrent path, and a group's shared B/C receive the sum
// over every head and channel of the group; Part I "Branches Copy Forward And
// Add Backward": where a forward value is used twice the reverse contributions
// add (dt feeds the retention and the write; x the write and the D skip).
//
// Derived block form (not printed on the pages).  For one (batch, head) and a
// 64-token block with entering state H, exit-state gradient dH (everything
// downstream), block-local inclusive Lam_i = sum_{k<=i} dt_k A,
// M[i][j] = exp(Lam_i - Lam_j) (j <= i), G[i][j] = C_i . B_j, w_j = exp(Lam_63 - Lam_j):
//   dXpre[j][p] = sum_{i>=j} G[i][j] M[i][j] dy_i[p] + w_j (dH B_j)[p]
//   dx_j        = D dy_j + dt_j dXpre_j,          ddt_j = x_j . dXpre_j + A da_j
//   K[i][j]     = (dy_i . x_j) M[i][j] dt_j
//   dC_i        = exp(Lam_i) H^T dy_i + sum_j K[i][j] B_j      (summed over heads)
//   dB_j        = w_j dt_j dH^T x_j + sum_i K[i][j] C_i        (summed over heads)
//   dLam_i      = sum_j K[i][j] G[i][j] - sum_i' K[i'][i] G[i'][i]
//               + exp(Lam_i) dy_i . (H C_i) - w_i dt_i x_i . (dH B_i)
//               + [i = 63] (exp(Lam_63) <dH, H> + sum_j w_j dt_j x_j . (dH B_j))
//   da_j        = sum_{i>=j} dLam_i,  dA += sum_j dt_j da_j,  dD += sum dy . x
//   dH_in       = exp(Lam_63) dH + sum_i exp(Lam_i) dy_i C_i^T
//
// Three launches:
//  1. ssd_bwd_dstate: one workgroup per (batch, head) walks 64-token blocks in
//     reverse with dH in MFMA accumulators and stores the gradient on the state
//     leaving every chunk (and dh0).
//  2. ssd_bwd_block: one workgroup per (batch, group, chunk, 64-token block).
//     It loops over the group's heads in ascending order; per head it rebuilds
//     the block-entry state from chunk_states (forward over the earlier blocks
//     of the chunk) and the block-exit gradient from step 1 (reverse over the
//     later blocks), then does the block algebra above.  dC/dB accumulate over
//     the heads in registers (fixed order, no atomics), and sum_h K is applied
//     to B and C once after the loop.  ddt is complete per block.
//  3. ssd_bwd_params: dA, dD as fixed-order fp64 sums of per-block partials.
#include "common.hpp"
#include "launch.hpp"
#include "ssd_common.hpp"

namespace ssm {
namespace {

// ===========================================================================
// 1. reverse pass of the state gradient
// ===========================================================================
struct DstSmem {
    bf16_t CT[kN * kS64];    // [n][tok]
    bf16_t EdYT[kP * kS64];  // [p][tok] = dy[tok][p] * exp(Lam_tok)
    float lam[2][kLs];
};

__global__ void __launch_bounds__(256) ssd_bwd_dstate_kernel(SsdBwdArgs a) {
    __shared__ DstSmem sm;
    const int bh = xcd_remap(blockIdx.x, gridDim.x);
    const int b = bh / a.H, h = bh % a.H, g = h / (a.H / a.G);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lk = (lane >> 4) * 8, lq = (lane >> 4) * 4;
    const int64_t T = a.T;
    const float Ah = a.A[h];
    const bf16_t *dy = static_cast<const bf16_t *>(a.dy);
    const bf16_t *Cm = static_cast<const bf16_t *>(a.C);
    constexpr int PN = kP * kN;

    // dH^T accumulators: tile q: nt = 2w + q/4, pt = q%4; n = 16nt + lq + v, p = 16pt + lr
    f32x4 G[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int n = 16 * (2 * wave + q / 4) + lq, p = 16 * (q % 4) + lr;
        if (a.dh_final != nullptr) {
            const float4 v = *reinterpret_cast<const float4 *>(a.dh_final + static_cast<int64_t>(bh) * PN + p * kN + n);
            G[q] = f32x4{v.x, v.y, v.z, v.w};
        } else {
            G[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    const int yt0 = map64_tok(tid), yp0 = map64_col(tid);    // dy: 2 tokens x 8 channels
    const int ct0 = map128_tok(tid), cn0 = map128_col(tid);  // C: 4 tokens x 8 coords
    u16x8 yr[2], cr[4];
    float dtr = 0.f;
    const u16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};
    auto prefetch = [&](int64_t t0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int64_t t = t0 + yt0 + i;
            yr[i] = (t < T) ? *reinterpret_cast<const u16x8 *>(dy + ((b * T + t) * a.H + h) * kP + yp0) : z8;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t t = t0 + ct0 + i;
            cr[i] = (t < T) ? *reinterpret_cast<const u16x8 *>(Cm + ((b * T + t) * a.G + g) * kN + cn0) : z8;
        }
        if (tid < kLs) {
            const int64_t t = t0 + tid;
            dtr = (t < T) ? a.dt[(b * T + t) * a.H + h] : 0.f;
        }
    };
    const int64_t nblk = (T + kLs - 1) / kLs;
    prefetch((nblk - 1) * kLs);
    for (int64_t s = nblk - 1; s >= 0; --s) {
        const int64_t t0 = s * kLs;
        const int buf = static_cast<int>(s & 1);
        if (s == nblk - 1 || ((t0 + kLs) % a.L) == 0) {
            // gradient on the state leaving chunk c (everything after it)
            float *dst = a.dstates + (static_cast<int64_t>(bh) * a.nchunks + t0 / a.L) * PN;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int n = 16 * (2 * wave + q / 4) + lq, p = 16 * (q % 4) + lr;
                *reinterpret_cast<float4 *>(dst + p * kN + n) = make_float4(G[q][0], G[q][1], G[q][2], G[q][3]);
            }
        }
        if (wave == 0) sm.lam[buf][lane] = wave_prefix_sum(dtr * Ah, lane);
        __syncthreads();
        const float *lam = sm.lam[buf];
        const float lam_end = lam[kLs - 1];
        {
            const float e0 = __expf(lam[yt0]), e1 = __expf(lam[yt0 + 1]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                *reinterpret_cast<uint32_t *>(&sm.EdYT[(yp0 + e) * kS64 + yt0]) =
                    pack2_bf16(bf16_to_f32(yr[0][e]) * e0, bf16_to_f32(yr[1][e]) * e1);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const u16x4 v = {cr[0][e], cr[1][e], cr[2][e], cr[3][e]};
                *reinterpret_cast<u16x4 *>(&sm.CT[(cn0 + e) * kS64 + ct0]) = v;
            }
        }
        if (s > 0) prefetch(t0 - kLs);
        __syncthreads();
        const float el = __expf(lam_end);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int nt = 2 * wave + q / 4, pt = q % 4;
            f32x4 acc = G[q];
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] *= el;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                acc = mma16(&sm.CT[(16 * nt + lr) * kS64 + 32 * kk + lk],
                            &sm.EdYT[(16 * pt + lr) * kS64 + 32 * kk + lk], acc);
            G[q] = acc;
        }
    }
    if (a.dh0 != nullptr) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int n = 16 * (2 * wave + q / 4) + lq, p = 16 * (q % 4) + lr;
            *reinterpret_cast<float4 *>(a.dh0 + static_cast<int64_t>(bh) * PN + p * kN + n) =
                make_float4(G[q][0], G[q][1], G[q][2], G[q][3]);
        }
    }
}

// ===========================================================================
// 2. per (batch, group, chunk, block): everything else
// ===========================================================================
// phase-aliased region U (bf16 element offsets)
constexpr int kT64 = kLs * kS64;   // a [64][72] tile
constexpr int kT128 = kN * kS64;   // a [128][72] tile
// block phase
constexpr int oX = 0, odY = kT64, odYT = 2 * kT64, oQT = 3 * kT64, oHT = 4 * kT64;
constexpr int odHT = oHT + kT128, odH = odHT + kT128, kUsize = odH + kP * kS128;
// recompute phase
constexpr int oR1 = 0, oR2 = kT64;
// final phase
constexpr int oK = 0, oKT = kT64, oBT = 2 * kT64, oCT = 2 * kT64 + kT128;
static_assert(oCT + kT128 <= kUsize, "final phase fits");

struct BlkSmem {
    bf16_t B[kLs * kS128];  // block rows [j][n]
    bf16_t C[kLs * kS128];  // block rows [i][n]
    bf16_t U[kUsize];
    float lam[kLs], dt[kLs];
    float row[kLs];
    float col[4][kLs], off[4][kLs], fin[4][kLs], dd[4][kLs];
    float dot[4], dd_sum[4];
};

__global__ void __launch_bounds__(256) ssd_bwd_block_kernel(SsdBwdArgs a) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    BlkSmem &sm = *reinterpret_cast<BlkSmem *>(smem_raw);
    const int nb = static_cast<int>(a.L / kLs);
    int id = xcd_remap(blockIdx.x, gridDim.x);
    const int k = id % nb;
    id /= nb;
    const int c = static_cast<int>(id % a.nchunks);
    id = static_cast<int>(id / a.nchunks);
    const int g = id % a.G, b = id / a.G;
    const int64_t T = a.T;
    const int64_t cstart = static_cast<int64_t>(c) * a.L;
    const int64_t tk = cstart + static_cast<int64_t>(k) * kLs;
    if (tk >= T) return;  // uniform for the whole workgroup, before any barrier
    const int64_t cend = (cstart + a.L < T) ? cstart + a.L : T;
    const int nbc = static_cast<int>((cend - cstart + kLs - 1) / kLs);
    const int hpg = a.H / a.G;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lk = (lane >> 4) * 8, lq = (lane >> 4) * 4;
    constexpr int PN = kP * kN;
    const bf16_t *x = static_cast<const bf16_t *>(a.x);
    const bf16_t *dy = static_cast<const bf16_t *>(a.dy);
    const bf16_t *Bm = static_cast<const bf16_t *>(a.B);
    const bf16_t *Cm = static_cast<const bf16_t *>(a.C);
    bf16_t *dx = static_cast<bf16_t *>(a.dx);
    bf16_t *U = sm.U;
    const u16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};

    const int rt0 = map64_tok(tid), rp0 = map64_col(tid);    // [tok][p] rows: 2 tokens x 8 channels
    const int nt0 = map128_tok(tid), nn0 = map128_col(tid);  // [tok][n] rows: 4 tokens x 8 coords

    auto load_rows64 = [&](const bf16_t *src, int64_t t0, int h, u16x8 *r) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int64_t t = t0 + rt0 + i;
            r[i] = (t < T) ? *reinterpret_cast<const u16x8 *>(src + ((b * T + t) * a.H + h) * kP + rp0) : z8;
        }
    };
    auto load_rows128 = [&](const bf16_t *src, int64_t t0, u16x8 *r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t t = t0 + nt0 + i;
            r[i] = (t < T) ? *reinterpret_cast<const u16x8 *>(src + ((b * T + t) * a.G + g) * kN + nn0) : z8;
        }
    };
    auto load_dt = [&](int64_t t0, int h) -> float {
        const int64_t t = t0 + lane;
        return (t < T) ? a.dt[(b * T + t) * a.H + h] : 0.f;
    };

    // block rows of B and C, and the group's Gram tile G[i][j] (wave w: i-tile w)
    {
        u16x8 br[4], cr[4];
        load_rows128(Bm, tk, br);
        load_rows128(Cm, tk, cr);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<u16x8 *>(&sm.B[(nt0 + i) * kS128 + nn0]) = br[i];
            *reinterpret_cast<u16x8 *>(&sm.C[(nt0 + i) * kS128 + nn0]) = cr[i];
        }
    }
    __syncthreads();
    f32x4 Gt[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        Gt[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (jt <= wave) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                Gt[jt] = mma16(&sm.C[(16 * wave + lr) * kS128 + 32 * kk + lk],
                               &sm.B[(16 * jt + lr) * kS128 + 32 * kk + lk], Gt[jt]);
        }
    }
    f32x4 Ks[4];                 // sum over heads of K, [i][j] like Gt
    f32x4 dCa[8], dBa[8];        // [n][tok]: tile q: nt = 2w + q/4, tt = q%4
#pragma unroll
    for (int q = 0; q < 4; ++q) Ks[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        dCa[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        dBa[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int hh = 0; hh < hpg; ++hh) {
        const int h = g * hpg + hh;
        const int64_t bh = static_cast<int64_t>(b) * a.H + h;
        const float Ah = a.A[h], Dh = a.D[h];
        // entering state and exit gradient of block k, [p][n]: p = 16w + lq + v, n = 16nt + lr
        f32x4 Hs[8], dHs[8];
        {
            const float *hc = a.chunk_states + (bh * a.nchunks + c) * PN;
            const float *dc = a.dstates + (bh * a.nchunks + c) * PN;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int o = (16 * wave + lq + v) * kN + 16 * nt + lr;
                    Hs[nt][v] = hc[o];
                    dHs[nt][v] = dc[o];
                }
            }
        }
        // forward over the earlier blocks of the chunk: H <- exp(Lam_63) H + X^T Bs
        for (int kb = 0; kb < k; ++kb) {
            const int64_t t0 = cstart + static_cast<int64_t>(kb) * kLs;
            u16x8 xr[2], br[4];
            load_rows64(x, t0, h, xr);
            load_rows128(Bm, t0, br);
            if (wave == 0) {
                const float d = load_dt(t0, h);
                sm.lam[lane] = wave_prefix_sum(d * Ah, lane);
                sm.dt[lane] = d;
            }
            __syncthreads();
            const float lam_end = sm.lam[kLs - 1];
            {
                bf16_t *XT = U + oR1, *BsT = U + oR2;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t pr = static_cast<uint32_t>(xr[0][e]) | (static_cast<uint32_t>(xr[1][e]) << 16);
                    *reinterpret_cast<uint32_t *>(&XT[(rp0 + e) * kS64 + rt0]) = pr;
                }
                float coef[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) coef[i] = __expf(lam_end - sm.lam[nt0 + i]) * sm.dt[nt0 + i];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    *reinterpret_cast<u16x4 *>(&BsT[(nn0 + e) * kS64 + nt0]) =
                        pack4(bf16_to_f32(br[0][e]) * coef[0], bf16_to_f32(br[1][e]) * coef[1],
                              bf16_to_f32(br[2][e]) * coef[2], bf16_to_f32(br[3][e]) * coef[3]);
            }
            __syncthreads();
            const float el = __expf(lam_end);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                f32x4 acc = Hs[nt];
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[v] *= el;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    acc = mma16(&U[oR1 + (16 * wave + lr) * kS64 + 32 * kk + lk],
                                &U[oR2 + (16 * nt + lr) * kS64 + 32 * kk + lk], acc);
                Hs[nt] = acc;
            }
        }
        // reverse over the later blocks: dH <- exp(Lam_63) dH + (E dY)^T C
        for (int kb = nbc - 1; kb > k; --kb) {
            const int64_t t0 = cstart + static_cast<int64_t>(kb) * kLs;
            u16x8 yr[2], cr[4];
            load_rows64(dy, t0, h, yr);
            load_rows128(Cm, t0, cr);
            if (wave == 0) {
                const float d = load_dt(t0, h);
                sm.lam[lane] = wave_prefix_sum(d * Ah, lane);
            }
            __syncthreads();
            const float lam_end = sm.lam[kLs - 1];
            {
                bf16_t *EdYT = U + oR1, *CT = U + oR2;
                const float e0 = __expf(sm.lam[rt0]), e1 = __expf(sm.lam[rt0 + 1]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    *reinterpret_cast<uint32_t *>(&EdYT[(rp0 + e) * kS64 + rt0]) =
                        pack2_bf16(bf16_to_f32(yr[0][e]) * e0, bf16_to_f32(yr[1][e]) * e1);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const u16x4 v = {cr[0][e], cr[1][e], cr[2][e], cr[3][e]};
                    *reinterpret_cast<u16x4 *>(&CT[(nn0 + e) * kS64 + nt0]) = v;
                }
            }
            __syncthreads();
            const float el = __expf(lam_end);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                f32x4 acc = dHs[nt];
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[v] *= el;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    acc = mma16(&U[oR1 + (16 * wave + lr) * kS64 + 32 * kk + lk],
                                &U[oR2 + (16 * nt + lr) * kS64 + 32 * kk + lk], acc);
                dHs[nt] = acc;
            }
        }

        // ---- block k ----
        {
            u16x8 xr[2], yr[2];
            load_rows64(x, tk, h, xr);
            load_rows64(dy, tk, h, yr);
            if (wave == 0) {
                const float d = load_dt(tk, h);
                sm.lam[lane] = wave_prefix_sum(d * Ah, lane);
                sm.dt[lane] = d;
            }
            __syncthreads();
            bf16_t *X = U + oX, *dY = U + odY, *dYT = U + odYT;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                *reinterpret_cast<u16x8 *>(&X[(rt0 + i) * kS64 + rp0]) = xr[i];
                *reinterpret_cast<u16x8 *>(&dY[(rt0 + i) * kS64 + rp0]) = yr[i];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t pr = static_cast<uint32_t>(yr[0][e]) | (static_cast<uint32_t>(yr[1][e]) << 16);
                *reinterpret_cast<uint32_t *>(&dYT[(rp0 + e) * kS64 + rt0]) = pr;
            }
            float dotp = 0.f;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                const int p0 = 16 * wave + lq, n = 16 * nt + lr;
                *reinterpret_cast<u16x4 *>(&U[oHT + n * kS64 + p0]) = pack4(Hs[nt][0], Hs[nt][1], Hs[nt][2], Hs[nt][3]);
                *reinterpret_cast<u16x4 *>(&U[odHT + n * kS64 + p0]) = pack4(dHs[nt][0], dHs[nt][1], dHs[nt][2], dHs[nt][3]);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    U[odH + (p0 + v) * kS128 + n] = f32_to_bf16(dHs[nt][v]);
                    dotp = fmaf(Hs[nt][v], dHs[nt][v], dotp);
                }
            }
            dotp = wave_sum(dotp);
            if (lane == 0) sm.dot[wave] = dotp;
        }
        __syncthreads();
        const float *lam = sm.lam, *dts = sm.dt;
        const float lam_end = lam[kLs - 1];
        // Phase I: dW = dY X^T, K, R = K G, Q = G M   (wave w: rows i in [16w, 16w+16))
        {
            const bf16_t *X = U + oX, *dY = U + odY;
            bf16_t *QT = U + oQT;
            float lam_i[4], rowacc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int v = 0; v < 4; ++v) lam_i[v] = lam[16 * wave + lq + v];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                const int j = 16 * jt + lr;
                f32x4 dW = {0.f, 0.f, 0.f, 0.f};
                if (jt <= wave) {
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
                        dW = mma16(&dY[(16 * wave + lr) * kS64 + 32 * kk + lk],
                                   &X[(16 * jt + lr) * kS64 + 32 * kk + lk], dW);
                }
                const float lam_j = lam[j], dt_j = dts[j];
                float q[4], colacc = 0.f;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int i = 16 * wave + lq + v;
                    const float m = (j <= i) ? __expf(lam_i[v] - lam_j) : 0.f;
                    const float kv = dW[v] * m * dt_j;
                    Ks[jt][v] += kv;
                    const float r = kv * Gt[jt][v];
                    rowacc[v] += r;
                    colacc += r;
                    q[v] = Gt[jt][v] * m;
                }
                *reinterpret_cast<u16x4 *>(&QT[j * kS64 + 16 * wave + lq]) = pack4(q[0], q[1], q[2], q[3]);
                colacc += __shfl_xor(colacc, 16, 64);
                colacc += __shfl_xor(colacc, 32, 64);
                if (lane < 16) sm.col[wave][j] = colacc;
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float r = rowacc[v];
                r += __shfl_xor(r, 1, 64);
                r += __shfl_xor(r, 2, 64);
                r += __shfl_xor(r, 4, 64);
                r += __shfl_xor(r, 8, 64);
                if (lr == 0) sm.row[16 * wave + lq + v] = r;
            }
        }
        __syncthreads();
        // Phase II: dXpre^T = dY^T Q + w (dH B^T)   (wave w: p in [16w, 16w+16))
        {
            const bf16_t *X = U + oX, *dY = U + odY, *dYT = U + odYT, *QT = U + oQT, *dH = U + odH;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                const int j = 16 * jt + lr;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if (32 * (kk + 1) <= 16 * jt) continue;  // Q[i][j] = 0 for i < j
                    acc = mma16(&dYT[(16 * wave + lr) * kS64 + 32 * kk + lk],
                                &QT[(16 * jt + lr) * kS64 + 32 * kk + lk], acc);
                }
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    acc4 = mma16(&dH[(16 * wave + lr) * kS128 + 32 * kk + lk],
                                 &sm.B[(16 * jt + lr) * kS128 + 32 * kk + lk], acc4);
                const float wj = __expf(lam_end - lam[j]), dt_j = dts[j];
                const u16x4 x4 = *reinterpret_cast<const u16x4 *>(&X[j * kS64 + 16 * wave + lq]);
                const u16x4 y4 = *reinterpret_cast<const u16x4 *>(&dY[j * kS64 + 16 * wave + lq]);
                float ddp = 0.f;
                f32x4 dxv;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float pre = fmaf(wj, acc4[v], acc[v]);
                    ddp = fmaf(bf16_to_f32(x4[v]), pre, ddp);
                    dxv[v] = fmaf(Dh, bf16_to_f32(y4[v]), dt_j * pre);
                }
                if (tk + j < T) {
                    *reinterpret_cast<u16x4 *>(dx + ((b * T + tk + j) * a.H + h) * kP + 16 * wave + lq) =
                        pack4(dxv[0], dxv[1], dxv[2], dxv[3]);
                }
                ddp += __shfl_xor(ddp, 16, 64);
                ddp += __shfl_xor(ddp, 32, 64);
                if (lane < 16) sm.dd[wave][j] = ddp;
            }
        }
        // Phase III / IV: per-head dC, dB contributions   (wave w: n in [32w, 32w+32))
        {
            const bf16_t *X = U + oX, *dY = U + odY, *HT = U + oHT, *dHT = U + odHT;
            float offacc[4] = {0.f, 0.f, 0.f, 0.f}, finacc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int nt = 2 * wave + q / 4, tt = q % 4;
                const int i = 16 * tt + lr;
                f32x4 ac = {0.f, 0.f, 0.f, 0.f}, ab = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    ac = mma16(&HT[(16 * nt + lr) * kS64 + 32 * kk + lk],
                               &dY[(16 * tt + lr) * kS64 + 32 * kk + lk], ac);
                    ab = mma16(&dHT[(16 * nt + lr) * kS64 + 32 * kk + lk],
                               &X[(16 * tt + lr) * kS64 + 32 * kk + lk], ab);
                }
                const float ei = __expf(lam[i]);
                const float wdt = __expf(lam_end - lam[i]) * dts[i];
                const u16x4 c4 = *reinterpret_cast<const u16x4 *>(&sm.C[i * kS128 + 16 * nt + lq]);
                const u16x4 b4 = *reinterpret_cast<const u16x4 *>(&sm.B[i * kS128 + 16 * nt + lq]);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    ac[v] *= ei;
                    ab[v] *= wdt;
                    offacc[tt] = fmaf(bf16_to_f32(c4[v]), ac[v], offacc[tt]);
                    finacc[tt] = fmaf(bf16_to_f32(b4[v]), ab[v], finacc[tt]);
                    dCa[q][v] += ac[v];
                    dBa[q][v] += ab[v];
                }
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                float o = offacc[tt], f = finacc[tt];
                o += __shfl_xor(o, 16, 64);
                o += __shfl_xor(o, 32, 64);
                f += __shfl_xor(f, 16, 64);
                f += __shfl_xor(f, 32, 64);
                if (lane < 16) {
                    sm.off[wave][16 * tt + lr] = o;
                    sm.fin[wave][16 * tt + lr] = f;
                }
            }
            // dD share: 16 products of dy . x per thread
            float dsum = 0.f;
            const int jr = tid >> 2, pc = (tid & 3) * 16;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                dsum = fmaf(bf16_to_f32(dY[jr * kS64 + pc + e]), bf16_to_f32(X[jr * kS64 + pc + e]), dsum);
            dsum = wave_sum(dsum);
            if (lane == 0) sm.dd_sum[wave] = dsum;
        }
        __syncthreads();
        // combine per token (wave 0, lane = token of the block), suffix sum, ddt
        if (wave == 0) {
            const int j = lane;
            float dl = sm.row[j];
            float ddd = 0.f, fs = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                dl += sm.off[w][j] - sm.col[w][j] - sm.fin[w][j];
                fs += sm.fin[w][j];
                ddd += sm.dd[w][j];
            }
            const float fin_total = wave_sum(fs);
            if (j == kLs - 1) {
                const float dotv = (sm.dot[0] + sm.dot[1]) + (sm.dot[2] + sm.dot[3]);
                dl += fin_total + __expf(lam_end) * dotv;
            }
            // da_j = sum_{i >= j} dLam_i
            float da = dl;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float t = __shfl_down(da, o, 64);
                if (lane + o < 64) da += t;
            }
            if (tk + j < T) a.ddt[(b * T + tk + j) * a.H + h] = fmaf(Ah, da, ddd);
            const float pa = wave_sum(dts[j] * da);
            if (lane == 0) {
                const int64_t pi = (bh * a.nchunks + c) * nb + k;
                a.pA[pi] = static_cast<double>(pa);
                a.pD[pi] = static_cast<double>((sm.dd_sum[0] + sm.dd_sum[1]) + (sm.dd_sum[2] + sm.dd_sum[3]));
            }
        }
    }

    // sum_h K applied once: dC += K B (contract over j), dB += K^T C (contract over i)
    __syncthreads();
    {
        bf16_t *Kr = U + oK, *KT = U + oKT, *BT = U + oBT, *CT = U + oCT;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            const int j = 16 * jt + lr, i0 = 16 * wave + lq;
            *reinterpret_cast<u16x4 *>(&KT[j * kS64 + i0]) = pack4(Ks[jt][0], Ks[jt][1], Ks[jt][2], Ks[jt][3]);
#pragma unroll
            for (int v = 0; v < 4; ++v) Kr[(i0 + v) * kS64 + j] = f32_to_bf16(Ks[jt][v]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const u16x4 vb = {sm.B[(nt0 + 0) * kS128 + nn0 + e], sm.B[(nt0 + 1) * kS128 + nn0 + e],
                              sm.B[(nt0 + 2) * kS128 + nn0 + e], sm.B[(nt0 + 3) * kS128 + nn0 + e]};
            const u16x4 vc = {sm.C[(nt0 + 0) * kS128 + nn0 + e], sm.C[(nt0 + 1) * kS128 + nn0 + e],
                              sm.C[(nt0 + 2) * kS128 + nn0 + e], sm.C[(nt0 + 3) * kS128 + nn0 + e]};
            *reinterpret_cast<u16x4 *>(&BT[(nn0 + e) * kS64 + nt0]) = vb;
            *reinterpret_cast<u16x4 *>(&CT[(nn0 + e) * kS64 + nt0]) = vc;
        }
    }
    __syncthreads();
    {
        const bf16_t *Kr = U + oK, *KT = U + oKT, *BT = U + oBT, *CT = U + oCT;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int nt = 2 * wave + q / 4, tt = q % 4;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                dCa[q] = mma16(&BT[(16 * nt + lr) * kS64 + 32 * kk + lk],
                               &Kr[(16 * tt + lr) * kS64 + 32 * kk + lk], dCa[q]);
                dBa[q] = mma16(&CT[(16 * nt + lr) * kS64 + 32 * kk + lk],
                               &KT[(16 * tt + lr) * kS64 + 32 * kk + lk], dBa[q]);
            }
            const int t = 16 * tt + lr;
            if (tk + t < T) {
                const int64_t o = ((b * T + tk + t) * a.G + g) * kN + 16 * nt + lq;
                *reinterpret_cast<float4 *>(a.dC + o) = make_float4(dCa[q][0], dCa[q][1], dCa[q][2], dCa[q][3]);
                *reinterpret_cast<float4 *>(a.dB + o) = make_float4(dBa[q][0], dBa[q][1], dBa[q][2], dBa[q][3]);
            }
        }
    }
}

// ===========================================================================
// 3. dA, dD: fixed-order fp64 sums over batch, chunks and blocks
// ===========================================================================
__global__ void ssd_bwd_params_kernel(SsdBwdArgs a) {
    const int h = blockIdx.x * blockDim.x + threadIdx.x;
    if (h >= a.H) return;
    const int64_t per = a.nchunks * (a.L / kLs);
    double sa = 0.0, sd = 0.0;
    for (int64_t b = 0; b < a.Bsz; ++b) {
        const int64_t base = (b * a.H + h) * per;
        for (int64_t i = 0; i < per; ++i) {
            sa += a.pA[base + i];
            sd += a.pD[base + i];
        }
    }
    a.dA[h] = static_cast<float>(sa);
    a.dD[h] = static_cast<float>(sd);
}

}  // namespace

hipError_t launch_ssd_bwd(const SsdBwdArgs &a, hipStream_t s) {
    // partials of blocks past the end of the sequence stay untouched: clear them
    const int64_t nparts = a.Bsz * a.H * a.nchunks * (a.L / kLs);
    hipError_t e = launch_fill(reinterpret_cast<float *>(a.pA), 2 * nparts, 0.f, s);
    if (e != hipSuccess) return e;
    e = launch_fill(reinterpret_cast<float *>(a.pD), 2 * nparts, 0.f, s);
    if (e != hipSuccess) return e;
    ssd_bwd_dstate_kernel<<<static_cast<unsigned>(a.Bsz * a.H), 256, 0, s>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t smem = sizeof(BlkSmem);
    static bool configured = false;
    if (!configured) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&ssd_bwd_block_kernel),
                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
        if (e != hipSuccess) return e;
        configured = true;
    }
    const int64_t nwg = a.Bsz * a.G * a.nchunks * (a.L / kLs);
    if (a.ev_begin != nullptr && (e = hipEventRecord(a.ev_begin, s)) != hipSuccess) return e;
    ssd_bwd_block_kernel<<<static_cast<unsigned>(nwg), 256, smem, s>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.ev_end != nullptr && (e = hipEventRecord(a.ev_end, s)) != hipSuccess) return e;
    ssd_bwd_params_kernel<<<static_cast<unsigned>((a.H + 255) / 256), 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace ssm
