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
//   dLam_i      = sum_{j<i} K[i][j] G[i][j] - sum_{i'>i} K[i'][i] G[i'][i]
//               + exp(Lam_i) dy_i . (H C_i) - f_i
//               + [i = 63] (exp(Lam_63) <dH, H> + sum_j f_j),   f_j = w_j dt_j x_j . (dH B_j)
//   da_j        = sum_{i>=j} dLam_i,  dA += sum_j dt_j da_j,  dD += sum dy . x
// (the diagonal K[i][i] G[i][i] would enter both sums of dLam_i and cancel; the f terms
// reach da_j as sum_{i<j} f_i.  Both are summed that way, so that with strong decay the
// order-one terms that cancel never meet the small ones in float32.)
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
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "ssd_common.hpp"


namespace ssm {
namespace {

// ===========================================================================
// 1. reverse pass of the state gradient
// ===========================================================================
// Both tiles keep the natural [tok][channel] layout and are read with the transposing
// LDS load; their row strides (72 and 40 dwords) put the four rows one such read spans
// on distinct banks, and a wave's 16-byte row writes are conflict-free.
constexpr int kSC = kN + 16;
constexpr int kSY = kP + 16;
// Offset (bf16 elements) of lane `lane`'s eight values of the tile pair (n-tiles 2 np
// and 2 np + 1, p-tile pt) in one chunk's gradient of the workspace: the four
// accumulator values of tile (2 np, pt) followed by those of tile (2 np + 1, pt), lane l
// holding p = 16 pt + l % 16, n = 16 nt + 4 (l / 16) + 0..3.  Each lane moves 16 bytes,
// and a wave a whole 1 KB, in both kernels (the 8-wave reverse pass, one n-tile per
// wave, writes 8-byte halves).  The gradient is rounded to bf16 here: every use in the
// per-block kernel rounds the block-exit gradient it builds from it to bf16 for the
// MFMA operands anyway.
__device__ __forceinline__ int dstate_pair(int np, int pt, int lane) {
    return ((np * (kP / 16) + pt) * 64 + lane) * 8;
}

struct __align__(16) DstSmem {
    bf16_t C[kLs * kSC];     // [tok][n]
    bf16_t EdY[kLs * kSY];   // [tok][p] = dy[tok][p] * exp(Lam_tok)
    float lam[2][kLs];
};
// The small-grid form: the staged tiles and the prefix double-buffered by block parity.
struct __align__(16) DstSmem2 {
    bf16_t C[2][kLs * kSC];
    bf16_t EdY[2][kLs * kSY];
    float lam[2][kLs];
};

// NW waves per workgroup: 4 when the (batch, head) workgroups fill every CU four deep,
// 8 for smaller grids (batch 1 at long context).  Each wave w < NW owns two n-tiles of dH^T
// and four p-tiles (NW = 4) or two (NW = 8), so its 32-token steps read two C fragments
// and as many dy fragments as it has p-tiles; every tile sees the same MFMA sequence
// either way, so the results do not depend on NW.
//
// With four workgroups per CU (NW = 4) the other workgroups cover each one's load latency
// and the rows of one block are loaded ahead.  The small-grid form (NW = 8), alone on its
// CU, keeps three blocks of rows in flight and runs one barrier per block (kSmall below).
template <int NW>
__global__ void __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(NW == 4 ? 4 : 2, NW == 4 ? 4 : 2))) ssd_bwd_dstate_kernel(SsdBwdArgs a) {
    static_assert(NW == 4 || NW == 8, "two n-tiles of four p-tiles per wave, or of two");
    constexpr int kTiles = 32 / NW;  // dH^T tiles per wave
    constexpr int kPT = kTiles / 2;  // p-tiles per wave (of n-tiles 2 np, 2 np + 1)
    constexpr bool kSmall = (NW == 8);
    constexpr int DEPTH = kSmall ? 3 : 1;  // blocks of rows in flight
    typedef typename std::conditional<kSmall, DstSmem2, DstSmem>::type Smem;
    __shared__ Smem sm;
    const int bh = xcd_remap(blockIdx.x, gridDim.x);
    const int b = bh / a.H, h = bh % a.H, g = h / (a.H / a.G);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lq = (lane >> 4) * 4;
    const int64_t T = a.T;
    const float Ah = a.A[h];
    const bf16_t *dy = static_cast<const bf16_t *>(a.dy);
    const bf16_t *Cm = static_cast<const bf16_t *>(a.C);
    constexpr int PN = kP * kN;

    // dH^T accumulators: tile q: n-tile 2 np + q / kPT, p-tile p0 + q % kPT (np = w, p0 = 0
    // with four waves; np = w / 2, p0 = 2 (w % 2) with eight); n = 16 nt + lq + v, p = 16 pt + lr
    const int np = (NW == 4) ? wave : wave >> 1, p0 = (NW == 4) ? 0 : 2 * (wave & 1);
    auto tile_nt = [&](int q) { return 2 * np + q / kPT; };
    auto tile_pt = [&](int q) { return p0 + q % kPT; };
    f32x4 G[kTiles];
#pragma unroll
    for (int q = 0; q < kTiles; ++q) {
        const int n = 16 * tile_nt(q) + lq, p = 16 * tile_pt(q) + lr;
        if (a.dh_final != nullptr) {
            const float4 v = *reinterpret_cast<const float4 *>(a.dh_final + static_cast<int64_t>(bh) * PN + p * kN + n);
            G[q] = f32x4{v.x, v.y, v.z, v.w};
        } else {
            G[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    // staging map: dy rows yt0 + 8 NW i from channel yp0; C rows ct0 + 4 NW i from coordinate cn0
    const int yt0 = tid >> 3, yp0 = (tid & 7) * 8;
    const int ct0 = tid >> 4, cn0 = (tid & 15) * 8;
    // A block's rows in registers, loaded one block ahead (right after the previous
    // block's rows were staged); four workgroups per CU cover each other's latency.
    constexpr int kYR = 8 / NW, kCR = 16 / NW;  // 16-byte row pieces per thread
    struct Rows {
        u16x8 yr[kYR], cr[kCR];
        float dtr;
    };
    // per-block buffer descriptors: rows at or past the end of the sequence read zero.
    // Block s starts at base + s * stride; 32-bit block counts keep 64-bit multiplies
    // and divides out of the loop.
    const uint32_t toky = static_cast<uint32_t>(a.H) * kP * 2, tokc = static_cast<uint32_t>(a.G) * kN * 2;
    const bf16_t *dy0 = dy + (b * T * a.H + h) * kP;
    const bf16_t *C0 = Cm + (b * T * a.G + g) * kN;
    const float *dt0 = a.dt + b * T * a.H + h;
    const int64_t sy = static_cast<int64_t>(kLs) * a.H * kP, sc = static_cast<int64_t>(kLs) * a.G * kN;
    const int64_t sd = static_cast<int64_t>(kLs) * a.H;
    auto prefetch = [&](Rows &R, int s) {
        const int64_t rem = T - static_cast<int64_t>(s) * kLs;
        const uint32_t nv = static_cast<uint32_t>(rem < kLs ? rem : kLs);
        const rsrc_t ry = make_rsrc(dy0 + s * sy, nv * toky);
        const rsrc_t rc = make_rsrc(C0 + s * sc, nv * tokc);
        const rsrc_t rd = make_rsrc(dt0 + s * sd, nv * a.H * 4u);
        R.dtr = 0.f;
        // (the small-grid form uses dt a step before the rows, so it is loaded first there)
        if (kSmall && tid < kLs) R.dtr = buf_ld_f32(rd, static_cast<uint32_t>(tid) * a.H * 4u);
#pragma unroll
        for (int i = 0; i < kYR; ++i) R.yr[i] = buf_ld_16b(ry, (yt0 + 8 * NW * i) * toky + yp0 * 2);
#pragma unroll
        for (int i = 0; i < kCR; ++i) R.cr[i] = buf_ld_16b(rc, (ct0 + 4 * NW * i) * tokc + cn0 * 2);
        if (!kSmall && tid < kLs) R.dtr = buf_ld_f32(rd, static_cast<uint32_t>(tid) * a.H * 4u);
    };
    const int nblk = static_cast<int>((T + kLs - 1) / kLs);
    const int bpc = static_cast<int>(a.L / kLs);  // blocks per chunk
    bf16_t *const dst0 = a.dstates + static_cast<int64_t>(bh) * a.nchunks * PN;
    // the gradient on the state leaving chunk c (everything after it) by tile pairs in
    // accumulator lane order (tiles q and q + kPT share a p-tile)
    auto put_exit_gradient = [&](bf16_t *dst) {
#pragma unroll
        for (int q = 0; q < kPT; ++q) {
            const u16x4 lo = pack4(G[q][0], G[q][1], G[q][2], G[q][3]);
            const u16x4 hi = pack4(G[q + kPT][0], G[q + kPT][1], G[q + kPT][2], G[q + kPT][3]);
            const u16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            *reinterpret_cast<u16x8 *>(dst + dstate_pair(np, tile_pt(q), lane)) = v;
        }
    };
    // dy rows scaled by exp(Lam) and C rows into the given tiles
    auto stage = [&](const Rows &R, const float *lam, bf16_t *sC, bf16_t *sE) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int i = 0; i < kYR; ++i) {
            const float e = __expf(lam[yt0 + 8 * NW * i]);
            const u16x8 v = R.yr[i];
            const u32x4 w = {pack2_bf16(bf16_to_f32(v[0]) * e, bf16_to_f32(v[1]) * e),
                             pack2_bf16(bf16_to_f32(v[2]) * e, bf16_to_f32(v[3]) * e),
                             pack2_bf16(bf16_to_f32(v[4]) * e, bf16_to_f32(v[5]) * e),
                             pack2_bf16(bf16_to_f32(v[6]) * e, bf16_to_f32(v[7]) * e)};
            *reinterpret_cast<u32x4 *>(&sE[(yt0 + 8 * NW * i) * kSY + yp0]) = w;
        }
#pragma unroll
        for (int i = 0; i < kCR; ++i)
            *reinterpret_cast<u16x8 *>(&sC[(ct0 + 4 * NW * i) * kSC + cn0]) = R.cr[i];
    };
    // dH^T = exp(Lam_63) dH^T + C^T (exp(Lam) dy) over the staged block
    auto products = [&](const bf16_t *sC, const bf16_t *sE, float lam_end) {
        const float el = __expf(lam_end);
#pragma unroll
        for (int q = 0; q < kTiles; ++q) {
            const int nt = tile_nt(q), pt = tile_pt(q);
            f32x4 acc = G[q];
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] *= el;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                acc = mfma(frag_tr(sC, kSC, 16 * nt, 32 * kk, lane), frag_tr(sE, kSY, 16 * pt, 32 * kk, lane), acc);
            G[q] = acc;
        }
    };
    auto chunk_end = [&](int s) { return s >= 0 && (s == nblk - 1 || (s + 1) % bpc == 0); };
    if constexpr (!kSmall) {
        // two barriers per block: the prefix of block s, then its staged rows
        auto step = [&](int s, Rows &R) {
            const int buf = s & 1;
            if (chunk_end(s)) put_exit_gradient(dst0 + static_cast<int64_t>(s / bpc) * PN);
            if (wave == 0) sm.lam[buf][lane] = wave_prefix_sum(R.dtr * Ah);
            __syncthreads();
            stage(R, sm.lam[buf], sm.C, sm.EdY);
            const float lam_end = sm.lam[buf][kLs - 1];
            if (s >= 1) prefetch(R, s - 1);
            __syncthreads();
            products(sm.C, sm.EdY, lam_end);
        };
        Rows R;
        prefetch(R, nblk - 1);
        for (int s = nblk - 1; s >= 0; --s) step(s, R);
    } else {
        // One barrier per block.  Before it: block s's rows are staged into the tiles of its
        // parity (the prefix Lam of block s was formed one step earlier) and wave 0 forms
        // block s - 1's prefix from the queued rows; after it: the products of block s.  A
        // tile pair or a prefix is rewritten two steps after the barrier that published it,
        // after the next barrier, which every wave reaches only once done with it.
        //
        // The waits on the queued rows count exactly only if every path through the loop
        // issues the same loads: with the last prefetches skipped, or a pass of the unrolled
        // loop cut short, the compiler can no longer tell how many loads are still pending
        // behind a block's rows and waits for all of them, which drains the queue.  So the
        // prefetch is unconditional (the last steps re-read block 0) and the walk runs steps
        // s = nblk - 1 down to send + 1, a whole number of DEPTH steps: those below 0 pad the
        // last pass (they stage re-read rows and wait at the barrier, nothing else).
        const int send = nblk - 1 - ((nblk + DEPTH - 1) / DEPTH) * DEPTH;
        // R refilled with block s - DEPTH once staged; Rn holds block s - 1
        auto step = [&](int s, Rows &R, const Rows &Rn) {
            const int buf = s & 1;
            if (chunk_end(s)) put_exit_gradient(dst0 + static_cast<int64_t>(s / bpc) * PN);
            stage(R, sm.lam[buf], sm.C[buf], sm.EdY[buf]);
            const float lam_end = sm.lam[buf][kLs - 1];
            if (wave == 0) sm.lam[buf ^ 1][lane] = wave_prefix_sum(Rn.dtr * Ah);
            // unconditional, so that every pass issues the same loads (the last steps re-read
            // block 0)
            prefetch(R, s >= DEPTH ? s - DEPTH : 0);
            __syncthreads();
            if (s >= 0) products(sm.C[buf], sm.EdY[buf], lam_end);
        };
        Rows R[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) prefetch(R[d], nblk - 1 - d >= 0 ? nblk - 1 - d : 0);
        if (wave == 0) sm.lam[(nblk - 1) & 1][lane] = wave_prefix_sum(R[0].dtr * Ah);
        __syncthreads();
        for (int s = nblk - 1; s > send; s -= DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) step(s - d, R[d], R[(d + 1) % DEPTH]);
        }
    }
    if (a.dh0 != nullptr) {
#pragma unroll
        for (int q = 0; q < kTiles; ++q) {
            const int n = 16 * tile_nt(q) + lq, p = 16 * tile_pt(q) + lr;
            *reinterpret_cast<float4 *>(a.dh0 + static_cast<int64_t>(bh) * PN + p * kN + n) =
                make_float4(G[q][0], G[q][1], G[q][2], G[q][3]);
        }
    }
}

// ===========================================================================
// 2. per (batch, group, chunk, block): everything else
// ===========================================================================
// All LDS tiles keep the natural global row layout ([tok][p] or [tok][n]), unpadded, with
// the 16-byte pieces of each row permuted (SwzLane); operands that contract over a tile's
// row index are read with the transposing read.
//
// Per head the block-entry state and block-exit gradient are single products
// over the chunk's other blocks, with chunk-local cumulative Lc:
//   H_k^T  = exp(Lc[s]) H_c^T + sum_{tok < 64k} B_tok (x) [exp(Lc[s]-Lc[tok]) dt_tok x_tok]
//   dH^T   = exp(Lc[end]-Lc[e]) dH_{c+1}^T + sum_{tok > e} C_tok (x) [exp(Lc[tok]-Lc[e]) dy_tok]
// (s = last token before block k, e = last token of block k; every exponent <= 0).
constexpr int kT64 = kLs * 64;    // a [64][64] tile (swizzled)
constexpr int kT128 = kLs * 128;  // a [64][128] tile (swizzled)
constexpr int kMaxBlk = 4;          // blocks per chunk (chunk <= 256)

constexpr int kBlkThreads = 1024;  // 16 waves

struct __align__(16) BlkSmem {
    bf16_t B[kT128];                    // block k rows of B [j][n]
    bf16_t C[kT128];                    // block k rows of C [i][n]
    bf16_t chainBC[(kMaxBlk - 1) * kT128];  // B rows of earlier blocks / C rows of later blocks,
                                            // transposed: [n][token], 64-wide rows
    bf16_t R[2 * kT128];                // per head: scaled x / dy rows of the other blocks,
                                        // then H and dH in bf16 ([p][n])
    bf16_t X[kT64], dY[kT64], QT[kT64]; // block k rows of x, dy; Q^T [j][i]
    float2 ld[2][kMaxBlk * kLs];  // chunk-local (Lam, dt) per token, by head parity
    // row, col, dd_sum are written before the S2 barrier and read by the combine of the
    // previous head during S2, so they are double-buffered by head parity
    // (token-major, so the combine reads each token's partials with a few wide loads)
    float row[2][4][kLs], col[2][kLs][4], dd[kLs][4];  // row: [j-tile][token], col: [token][i-tile]
    float fp[kLs][4];      // f_j = w_j dt_j x_j.(dH B_j) partials per token and p-tile
    float offin[kLs][8];   // dy_i.(H C_i) exp(Lam_i) partials per token and n-tile
    float dot[16], dd_sum[2][16];
    // Per-token decay factors of a head, by head parity, computed once per head one phase
    // ahead of their use (instead of an exponential per thread per use): fac[t] for a
    // chunk token t outside block k is the factor that scales its row for the state
    // products; es = exp(Lam_blk0), ee = exp(Lam_end - Lam_e); w_i = exp(Lam_e - Lam_i).
    float fac[2][kMaxBlk * kLs], es[2], ee[2];
    // block k's tokens, by head parity: (exp(Lam_i - Lam_blk0), w_i dt_i, w_i, dt_i), read
    // as two pairs by the last phase
    float4 tk[2][kLs];
    uint32_t lanetab[64][8];  // SwzLane of lane l, formed once (6 words and 2 of padding)
};
static_assert((kMaxBlk - 1) * kT64 <= 2 * kT128, "scaled rows fit under the state tiles");
static_assert(offsetof(BlkSmem, X) == offsetof(BlkSmem, R) + sizeof(BlkSmem::R) &&
                  offsetof(BlkSmem, dY) == offsetof(BlkSmem, X) + sizeof(BlkSmem::X) &&
                  sizeof(BlkSmem::R) + sizeof(BlkSmem::X) + sizeof(BlkSmem::dY) >= (kMaxBlk - 1) * kT128 * sizeof(bf16_t),
              "R, X and dY hold the chain's B/C rows before their transposition");

// Sixteen waves, four per SIMD, so that each SIMD has other waves to issue from while
// one waits on LDS, an MFMA result or a barrier.  Wave w's tiles (every tile 16 x 16):
//   Gram / K / Phase I, [i][j]:   i-tile gi, j-tile gj from kGramTiles
//   state products, [n][p]:       n-tiles 2 wq, 2 wq + 1, p-tile wj
//   Phase II, [p][j]:             p-tile wq, j-tiles 2 wj, 2 wj + 1 (waves 0 .. 7)
//   Phase III/IV and K, [n][tok]: n-tile wn, token tiles 2 wm, 2 wm + 1
// Gram tile (i-tile << 2 | j-tile) of wave w in bits 4w .. 4w + 3.  The ten tiles on or
// below the diagonal carry Phase I's work; wave w runs on SIMD w % 4, and the table gives
// SIMDs 0 .. 3 two, three, three and two of them (wave 0, which also runs the per-token
// combine, holds a zero tile), instead of one to four with i = w % 4, j = w / 4.
constexpr uint64_t kGramTiles = 0xb6327d94fc80ea51ull;

// Sums over the 16 lanes of a row for four values at once: lane lr of the row returns
// the row's total of v[lr / 4].  Row mirror, then half-row mirror, exchange the values a
// lane does not keep (two of four, then one of two); two quad swaps finish the sums.
// The additions run in a fixed order, so the sums are deterministic.
__device__ __forceinline__ float row16_sum4(const float (&v)[4], int lr) {
#define SSM_DPP(x, ctrl) \
    __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, (x)), (ctrl), 0xf, 0xf, false))
    const bool lo8 = lr < 8, lo4 = (lr & 7) < 4;
    float a = lo8 ? v[0] : v[2], b = lo8 ? v[1] : v[3];
    a += SSM_DPP(lo8 ? v[2] : v[0], 0x140);  // row_mirror: lane lr <-> 15 - lr
    b += SSM_DPP(lo8 ? v[3] : v[1], 0x140);
    float k = lo4 ? a : b;
    k += SSM_DPP(lo4 ? b : a, 0x141);        // row_half_mirror: lr <-> 7 - lr within halves
    k += SSM_DPP(k, 0xB1);                    // quad_perm [1,0,3,2]
    k += SSM_DPP(k, 0x4E);                    // quad_perm [2,3,0,1]
#undef SSM_DPP
    return k;
}

__global__ void __launch_bounds__(kBlkThreads) ssd_bwd_block_kernel(SsdBwdArgs a) {
    __shared__ BlkSmem sm;
    const int nb = static_cast<int>(a.L / kLs);
    int id = xcd_remap(blockIdx.x, gridDim.x);
    int k = id % nb;
    id /= nb;
    const int c = static_cast<int>(id % a.nchunks);
    id = static_cast<int>(id / a.nchunks);
    const int g = id % a.G, b = id / a.G;
    const int64_t T = a.T;
    const int64_t cstart = static_cast<int64_t>(c) * a.L;
    const int64_t tk = cstart + static_cast<int64_t>(k) * kLs;
    const int hpg = a.H / a.G;
    if (tk >= T) {  // uniform for the whole workgroup, before any barrier
        // a block past the end of the sequence: its heads' dA, dD partials are zero
        const int hl = static_cast<int>(threadIdx.x);
        if (hl < hpg) {
            const int64_t pi = ((static_cast<int64_t>(b) * a.H + g * hpg + hl) * a.nchunks + c) * nb + k;
            a.pA[pi] = 0.0;
            a.pD[pi] = 0.0;
        }
        return;
    }
    const int64_t cend = (cstart + a.L < T) ? cstart + a.L : T;
    int nbc = static_cast<int>((cend - cstart + kLs - 1) / kLs);
    int kS_ = 64 * k - 1, kE_ = 64 * k + kLs - 1, kEnd_ = 64 * nbc - 1, base_ = 64 * k;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    int wq = wave & 3, wj = wave >> 2, wn = wave & 7, wm = wave >> 3;
    int gi = static_cast<int>((kGramTiles >> (4 * wave)) >> 2) & 3, gj = static_cast<int>(kGramTiles >> (4 * wave)) & 3;
    // Lane-derived indices are re-formed at the top of every head iteration from a
    // value the compiler cannot see through, so the LDS addresses built from them are
    // computed next to their uses instead of occupying registers across the loop.
    int tid, lane, lr, lq, pid;
    uint32_t stg;  // this thread's piece of the per-head row staging
    SwzLane sl;
    auto refresh_lane = [&]() {
        tid = static_cast<int>(threadIdx.x);
        asm volatile("" : "+v"(tid));
        lane = tid & 63;
        lr = lane & 15;
        lq = (lane >> 4) * 4;
        pid = tid & 511;  // staging piece: row pid / 8, piece pid % 8 (two threads per piece)
        stg = swz_stage64(pid >> 3, pid & 7);
        // two LDS reads instead of the thirty-odd operations that form the offsets
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x4 t0 = *reinterpret_cast<const u32x4 *>(&sm.lanetab[lane][0]);
        const u32x2 t1 = *reinterpret_cast<const u32x2 *>(&sm.lanetab[lane][4]);
        sl.row64 = t0[0];
        sl.row128 = t0[1];
        sl.tr64 = t0[2];
        sl.tr128 = t0[3];
        sl.pc64 = t1[0];
        sl.pc128 = t1[1];
    };
    tid = static_cast<int>(threadIdx.x);
    lane = tid & 63;
    lr = lane & 15;
    lq = (lane >> 4) * 4;
    pid = tid & 511;
    stg = swz_stage64(pid >> 3, pid & 7);
    sl = swz_lane(lane);
    if (wave == 0) {  // read inside the head loop, after several barriers
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<u32x4 *>(&sm.lanetab[lane][0]) = u32x4{sl.row64, sl.row128, sl.tr64, sl.tr128};
        *reinterpret_cast<u32x2 *>(&sm.lanetab[lane][4]) = u32x2{sl.pc64, sl.pc128};
    }
    // A and D of the group's heads, lane l holding head h0 + l; a head's value is read
    // with readlane (a scalar, no memory wait).  Loads through the kernel's pointers would
    // be vector loads whose waits also drain every row and state load in flight.
    const int h0 = g * hpg;
    const float A_lane = (lane < hpg) ? a.A[h0 + lane] : 0.f;
    const float D_lane = (lane < hpg) ? a.D[h0 + lane] : 0.f;
    // (the host sends groups of at most 64 heads here)
    auto head_A = [&](int hh) -> float {
        return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(A_lane), hh));
    };
    auto head_D = [&](int hh) -> float {
        return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(D_lane), hh));
    };
    constexpr int PN = kP * kN;
    const bf16_t *x = static_cast<const bf16_t *>(a.x);
    const bf16_t *dy = static_cast<const bf16_t *>(a.dy);
    const bf16_t *Bm = static_cast<const bf16_t *>(a.B);
    const bf16_t *Cm = static_cast<const bf16_t *>(a.C);
    bf16_t *dx = static_cast<bf16_t *>(a.dx);
    const u16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};
    // [tok][n] tiles: one 16-byte piece per thread
    const int nr_tok = tid >> 4, nr_col = (tid & 15) * 8;
    const uint32_t nr_stg = swz_stage128(nr_tok, tid & 15);

    auto load_rows_n = [&](const bf16_t *src, int64_t t0, bf16_t *dst) {
        const int64_t t = t0 + nr_tok;
        const u16x8 r = (t < T) ? *reinterpret_cast<const u16x8 *>(src + ((b * T + t) * a.G + g) * kN + nr_col) : z8;
        *reinterpret_cast<u16x8 *>(reinterpret_cast<char *>(dst) + nr_stg) = r;
    };
    // head-independent tiles: block k B and C rows, B rows of earlier blocks, C rows of later
    // ones (the latter staged in R, X and dY, free until the first head's staging, and
    // transposed into chainBC below)
    bf16_t *chain_tmp = sm.R;
    load_rows_n(Bm, tk, sm.B);
    load_rows_n(Cm, tk, sm.C);
    for (int kb = 0; kb < nbc; ++kb) {
        if (kb == k) continue;
        const int slot = kb < k ? kb : kb - 1;
        load_rows_n(kb < k ? Bm : Cm, cstart + static_cast<int64_t>(kb) * kLs, chain_tmp + slot * kT128);
    }

    // per-head inputs held in registers one head ahead: waves 0..7 stage blocks 0, 1 and
    // the dy rows of block k, waves 8..15 blocks 2, 3
    u16x8 xr[2];  // x rows of blocks 2 wm + i <= k, dy rows of later blocks
    u16x8 yk;     // dy rows of block k (wm = 0)
    float dtr[4];
    // Per-head rows of x, dy, dx and dt, ddt through buffer descriptors over this
    // chunk: offsets past the chunk's valid tokens read zero / drop the write.
    const int nvalid = static_cast<int>(cend - cstart);   // valid tokens of this chunk
    const uint32_t tokb = static_cast<uint32_t>(a.H) * kP * 2;  // bytes between tokens of x, dy, dx
    const int64_t row0 = (static_cast<int64_t>(b) * T + cstart) * a.H;  // first (token, head) of the chunk
    const rsrc_t rx = make_rsrc(x + row0 * kP, nvalid * tokb);
    const rsrc_t ry = make_rsrc(dy + row0 * kP, nvalid * tokb);
    const rsrc_t rdx = make_rsrc(dx + row0 * kP, nvalid * tokb);
    const rsrc_t rdt = make_rsrc(a.dt + row0, nvalid * a.H * 4u);
    const rsrc_t rddt = make_rsrc(a.ddt + row0, nvalid * a.H * 4u);
    const uint32_t row_off = static_cast<uint32_t>(pid >> 3) * tokb + (pid & 7) * 16;  // this thread's row segment
    auto prefetch = [&](int h) {
        const uint32_t o = row_off + static_cast<uint32_t>(h) * (kP * 2);
#pragma unroll
        for (int i = 0; i < 2; ++i) {  // blocks past the chunk read zero
            const int kb = 2 * wm + i;
            xr[i] = buf_ld_16b(kb <= k ? rx : ry, o + kb * kLs * tokb);
        }
        if (wm == 0) yk = buf_ld_16b(ry, o + k * kLs * tokb);
    };
    // dt of head h, four tokens per lane (wave 0 only; consumed by the scan)
    auto prefetch_dt = [&](int h) {
        if (wave == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dtr[e] = buf_ld_f32(rdt, (static_cast<uint32_t>(4 * lane + e) * a.H + h) * 4u);
        }
    };
    // chunk-local cumulative log-retention of head h (wave 0; lane = 4 tokens)
    auto scan = [&](int h, int par) {
        const float Ah = head_A(h - h0);
        const float v0 = dtr[0] * Ah, v1 = v0 + dtr[1] * Ah, v2 = v1 + dtr[2] * Ah, v3 = v2 + dtr[3] * Ah;
        const float off = wave_prefix_sum(v3) - v3;
        typedef float f32x4v __attribute__((ext_vector_type(4)));
        f32x4v* dstp = reinterpret_cast<f32x4v *>(&sm.ld[par][4 * lane]);
        dstp[0] = f32x4v{off + v0, dtr[0], off + v1, dtr[1]};
        dstp[1] = f32x4v{off + v2, dtr[2], off + v3, dtr[3]};
    };
    // the decay factors of the head whose (Lam, dt) sit in ld[par] (threads 0..255, one
    // chunk token each; two exponentials where the token is in block k, one elsewhere)
    auto factors = [&](int par) {
        const int t = static_cast<int>(threadIdx.x);
        if (t < kMaxBlk * kLs) {
            const float2 *lp = sm.ld[par];
            const float lb0 = kS_ >= 0 ? lp[kS_].x : 0.f, le = lp[kE_].x;
            const float2 lt = lp[t];
            if (t >= base_ && t < base_ + kLs) {  // whole waves: block k is 64 aligned tokens
                const float wt = __expf(le - lt.x);
                sm.tk[par][t - base_] = make_float4(__expf(lt.x - lb0), wt * lt.y, wt, lt.y);
            } else {
                sm.fac[par][t] = t < base_ ? __expf(lb0 - lt.x) * lt.y : __expf(lt.x - le);
            }
            if (t == 0) {
                sm.es[par] = __expf(lb0);
                sm.ee[par] = __expf(lp[kEnd_].x - le);
            }
        }
    };
    // raw chunk-boundary state and chunk-exit gradient of the next head, loaded a full
    // head ahead of their use in S2; the state tiles in accumulator layout, [n][p]:
    // q -> n-tile 2 wq + q, p-tile wj
    f32x4 Hs[2];
    u16x8 dHr;  // chunk-exit gradient tile pair (n-tiles 2 wq, 2 wq + 1, p-tile wj), bf16
    // (through buffer descriptors over the head's tile: the 64-bit address arithmetic
    // stays in scalar registers and the lanes add 32-bit offsets)
    auto load_states = [&](int h) {
        const int64_t tile = ((static_cast<int64_t>(b) * a.H + h) * a.nchunks + c) * PN;
        const rsrc_t rh = make_rsrc(a.chunk_states + tile, PN * 4u);
        const rsrc_t rd = make_rsrc(a.dstates + tile, PN * 2u);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint32_t n = 16 * (2 * wq + q) + lq, p = 16 * wj + lr;
            Hs[q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rh, (p * kN + n) * 4u, 0, 0));
        }
        dHr = buf_ld_16b(rd, static_cast<uint32_t>(dstate_pair(wq, wj, lane)) * 2u);
    };

    prefetch(h0);
    prefetch_dt(h0);
    load_states(h0);
    if (wave == 0) scan(h0, 0);
    __syncthreads();
    factors(0);
    // The chain's B/C tiles transposed once to [n][token]: every state product of every head
    // then reads its B/C operand as one 16-byte row fragment instead of two transposing reads.
    // Fragment (n-tile nt, 32-token step kk) of a slot is read where the transposing read
    // leaves it, so lane l writes exactly the piece it would have read.
    for (int f = wave; f < (kMaxBlk - 1) * 16; f += 16) {
        const int slot = f >> 4, nt = (f >> 1) & 7, kk = f & 1;
        if (slot >= nbc - 1) break;
        const bf16x8 v = frag_tr128(chain_tmp + slot * kT128, sl, nt, kk);
        *reinterpret_cast<bf16x8 *>(reinterpret_cast<char *>(sm.chainBC + slot * kT128) + swz_row64(sl, nt, kk)) = v;
    }
    // Gram tile of block k, [i][j]: i-tile gi, j-tile gj
    f32x4 Gt = {0.f, 0.f, 0.f, 0.f};
    if (gj <= gi) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            Gt = mfma(lds_frag(sm.C, swz_row128(sl, gi, kk)), lds_frag(sm.B, swz_row128(sl, gj, kk)), Gt);
    }
    // C of block k at this lane's (token, n) positions of the Phase III tiles
    float cC[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const u16x4 c4 = *reinterpret_cast<const u16x4 *>(reinterpret_cast<const char *>(sm.C) + swz_pc128(sl, 2 * wm + t, wn));
#pragma unroll
        for (int v = 0; v < 4; ++v) cC[t][v] = bf16_to_f32(c4[v]);
    }
    f32x4 Ks = {0.f, 0.f, 0.f, 0.f}, dCa[2], dBa[2];  // Ks like Gt; dCa/dBa [n][tok]: n-tile wn, tok-tiles 2wm + t
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        dCa[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        dBa[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // Tiles above the diagonal are zero for every head: their Q^T pieces and partial
    // sums, and the dD partials of the off-diagonal tiles, are written once here (for both
    // head parities) rather than in every head's Phase I.
    if (gj > gi) {
        *reinterpret_cast<u16x4 *>(reinterpret_cast<char *>(sm.QT) + swz_pc64(sl, gj, gi)) = pack4(0.f, 0.f, 0.f, 0.f);
        typedef float f32x4v __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            if (lane < 16) sm.col[q][16 * gj + lr][gi] = 0.f;
            if (lr == 0) *reinterpret_cast<f32x4v *>(&sm.row[q][gj][16 * gi + lq]) = f32x4v{0.f, 0.f, 0.f, 0.f};
        }
    }
    if (gj != gi && lane == 0) {
        sm.dd_sum[0][wave] = 0.f;
        sm.dd_sum[1][wave] = 0.f;
    }
    const int kS = kS_;      // chunk-local index of the token before block k
    const int kE = kE_;      // last token of block k
    const int base = base_;
    __syncthreads();  // the first head's decay factors

    // Per-token combine of head hc (wave 0, lane = token of the block): the dLam terms,
    // da = reverse cumulative sum within the block, ddt, and the dA/dD partials.  Runs
    // for head h-1 at the end of head h's S2 (the arrays it reads are rewritten only
    // after that phase's barrier, or are double-buffered by head parity).
    auto combine = [&](int hc, int pc) {
        const int j = lane;
        const float2 *ldc = sm.ld[pc];
        const float lb0 = kS >= 0 ? ldc[kS].x : 0.f;
        const float le = ldc[kE].x;
        typedef float f32x4v __attribute__((ext_vector_type(4)));
        const f32x4v cl = *reinterpret_cast<const f32x4v *>(sm.col[pc][j]);
        const f32x4v dv = *reinterpret_cast<const f32x4v *>(sm.dd[j]);
        const f32x4v fv = *reinterpret_cast<const f32x4v *>(sm.fp[j]);
        const f32x4v o0 = *reinterpret_cast<const f32x4v *>(&sm.offin[j][0]);
        const f32x4v o1 = *reinterpret_cast<const f32x4v *>(&sm.offin[j][4]);
        float dl = (sm.row[pc][0][j] + sm.row[pc][1][j]) + (sm.row[pc][2][j] + sm.row[pc][3][j]);
        float ddd = 0.f, fs = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            dl -= cl[w];
            ddd += dv[w];
            fs += fv[w];
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) dl += o0[w];
#pragma unroll
        for (int w = 0; w < 4; ++w) dl += o1[w];
        if (j == kLs - 1) {
            float dotv = 0.f;
#pragma unroll
            for (int w = 0; w < 16; ++w) dotv += sm.dot[w];
            dl += __expf(le - lb0) * dotv;
        }
        // The exit-gradient term f_i = w_i dt_i x_i.(dH B_i) enters dLam_i as -f_i and the
        // block's last token as +sum_i f_i, so it reaches da_j = sum_{i >= j} dLam_i as the
        // exclusive prefix sum_{i < j} f_i, summed directly (f_63, of order one even when
        // every other term underflows, never meets the small ones).
        // (a whole-wave DPP shift by one lane: lane j reads lane j - 1, lane 0 reads 0)
        const float fprev = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, fs), 0x138, 0xf, 0xf, true));
        const float da = wave_suffix_sum(dl) + wave_prefix_sum(fprev);  // da_j = sum_{i >= j} dLam_i
        buf_st_f32(rddt, (static_cast<uint32_t>(k * kLs + j) * a.H + hc) * 4u, fmaf(head_A(hc - h0), da, ddd));
        const float pa = wave_total(ldc[base + j].y * da);
        if (lane == 0) {
            float ds = 0.f;
#pragma unroll
            for (int w = 0; w < 16; ++w) ds += sm.dd_sum[pc][w];
            const int64_t pi = ((static_cast<int64_t>(b) * a.H + hc) * a.nchunks + c) * nb + k;
            a.pA[pi] = static_cast<double>(pa);
            a.pD[pi] = static_cast<double>(ds);
        }
    };

    for (int hh = 0; hh < hpg; ++hh) {
        refresh_lane();
        // The block and wave indices pass through an empty asm at every head, so that the
        // comparisons and offsets derived from them are re-formed in scalar registers at
        // their uses rather than hoisted out of the loop, where they outnumber the scalar
        // registers and are parked in vector lanes (one readlane per use).
        asm volatile("" : "+s"(k), "+s"(nbc), "+s"(wq), "+s"(wj), "+s"(wn), "+s"(wm), "+s"(gi), "+s"(gj));
        asm volatile("" : "+s"(kS_), "+s"(kE_), "+s"(kEnd_), "+s"(base_));
        const int h = h0 + hh, par = hh & 1;
        const float Dh = head_D(hh);
        const float2 *ld = sm.ld[par];  // (Lam, dt) of this head's chunk
        // The next head's loads are issued on every iteration (the last one re-reads its own
        // head), so each iteration issues the same memory operations and the waits on them
        // count exactly instead of draining everything in flight.
        const int hn = (hh + 1 < hpg) ? h + 1 : h;
        prefetch_dt(hn);  // used by the next head's scan in S3
        // ---- S1: stage this head's rows (scaled for the state products) ----
        {
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int kb = 2 * wm + i;
                if (kb >= nbc) break;
                if (kb == k) {
                    *reinterpret_cast<u16x8 *>(reinterpret_cast<char *>(sm.X) + stg) = xr[i];
                    continue;
                }
                const float cf = sm.fac[par][64 * kb + (pid >> 3)];
                const int slot = kb < k ? kb : kb - 1;
                const u16x8 v = xr[i];
                const u32x4 w = {pack2_bf16(bf16_to_f32(v[0]) * cf, bf16_to_f32(v[1]) * cf),
                                 pack2_bf16(bf16_to_f32(v[2]) * cf, bf16_to_f32(v[3]) * cf),
                                 pack2_bf16(bf16_to_f32(v[4]) * cf, bf16_to_f32(v[5]) * cf),
                                 pack2_bf16(bf16_to_f32(v[6]) * cf, bf16_to_f32(v[7]) * cf)};
                *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(sm.R + slot * kT64) + stg) = w;
            }
            if (wm == 0) *reinterpret_cast<u16x8 *>(reinterpret_cast<char *>(sm.dY) + stg) = yk;
        }
        __syncthreads();
        prefetch(hn);  // registers are free once staged
        // ---- S2: Phase I of block k, then the state products over the other blocks ----
        // Phase I: dW = dY X^T, K, R = K G, Q = G M   (i-tile gi, j-tile gj)
        // (above the diagonal every entry is zero: those tiles' Q^T pieces and partial sums
        // were written once, before the head loop)
        if (gj <= gi) {
            f32x4 dW = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                dW = mfma(lds_frag(sm.dY, swz_row64(sl, gi, kk)), lds_frag(sm.X, swz_row64(sl, gj, kk)), dW);
            const int j = 16 * gj + lr;
            const float2 lj = ld[base + j];
            const float lam_j = lj.x, dt_j = lj.y;
            float rowv[4], qv[4], colacc = 0.f;
            // off the diagonal every (i, j) has j < i; on it the masks apply
            auto entries = [&](bool on_diag) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int i = 16 * gi + lq + v;
                    float m = __expf(ld[base + i].x - lam_j);
                    if (on_diag) m = (j <= i) ? m : 0.f;
                    const float kv = dW[v] * dt_j * m;
                    Ks[v] += kv;
                    // R[i][i] enters row sum i and column sum i alike and cancels in
                    // dLam_i, so it is left out of both: with strong decay it is the only
                    // O(1) entry, and subtracting it would bury the small terms in rounding
                    float r = kv * Gt[v];
                    if (on_diag) r = (j < i) ? r : 0.f;
                    rowv[v] = r;
                    colacc += r;
                    qv[v] = Gt[v] * m;
                }
            };
            if (gj == gi) {
                entries(true);
                float diag = 0.f;  // dW[i][i] = dy_i . x_i feeds dD
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (lq + v == lr) diag += dW[v];
                diag = wave_total(diag);
                if (lane == 0) sm.dd_sum[par][wave] = diag;
            } else {
                entries(false);
            }
            *reinterpret_cast<u16x4 *>(reinterpret_cast<char *>(sm.QT) + swz_pc64(sl, gj, gi)) = pack4(qv[0], qv[1], qv[2], qv[3]);
            colacc = rows4_sum(colacc);
            if (lane < 16) sm.col[par][j][gi] = colacc;
            // row sums of the tile's four rows in one pass: lane lr ends with row lq + lr / 4
            const float rs = row16_sum4(rowv, lr);
            if ((lr & 3) == 0) sm.row[par][gj][16 * gi + lq + (lr >> 2)] = rs;
        }
        // The sums start from the decayed chunk-boundary terms (the state entering the
        // chunk, the gradient leaving it).  Per 32-token step the wave reads two n fragments
        // (row reads) and one p fragment (the transposing read).
        f32x4 aH[2], adH[2];
        {
            const float es = sm.es[par];  // chunk start -> block k start
            const float ee = sm.ee[par];  // block k end -> chunk end
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    aH[q][v] = es * Hs[q][v];
                    adH[q][v] = ee * bf16_to_f32(dHr[4 * q + v]);
                }
        }
        {
            auto chain = [&](const bf16_t *bc, const bf16_t *xs, f32x4 *acc) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    bf16x8 fa[2];
#pragma unroll
                    for (int q = 0; q < 2; ++q) fa[q] = lds_frag(bc, swz_row64(sl, 2 * wq + q, kk));
                    const bf16x8 fb = frag_tr64(xs, sl, wj, kk);
#pragma unroll
                    for (int q = 0; q < 2; ++q) acc[q] = mfma(fa[q], fb, acc[q]);
                }
            };
#pragma unroll
            for (int kb = 0; kb < kMaxBlk - 1; ++kb) {  // H_k = e H_c + sum over earlier blocks
                if (kb >= k) break;
                chain(sm.chainBC + kb * kT128, sm.R + kb * kT64, aH);
            }
#pragma unroll
            for (int sb = 0; sb < kMaxBlk - 1; ++sb) {  // dH_{k+1} = e dH_c + sum over later blocks (slot sb = block sb+1)
                if (sb < k || sb + 1 >= nbc) continue;
                chain(sm.chainBC + sb * kT128, sm.R + sb * kT64, adH);
            }
        }
        // the previous head's per-token combine, after this wave's products (wave 0, which
        // holds a zero Gram tile; 1.313 -> 1.297 ms against running it first)
        if (wave == 0 && hh > 0) combine(h - 1, par ^ 1);
        __syncthreads();
        // ---- S3: block-entry state and exit gradient in bf16, [p][n] ----
        bf16_t *Hb = sm.R, *dHb = sm.R + kT128;
        {
            float dotp = 0.f;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const f32x4 hv = aH[q], gv = adH[q];
#pragma unroll
                for (int v = 0; v < 4; ++v) dotp = fmaf(hv[v], gv[v], dotp);
                const uint32_t o = swz_pc128(sl, wj, 2 * wq + q);  // [p][n]
                *reinterpret_cast<u16x4 *>(reinterpret_cast<char *>(Hb) + o) = pack4(hv[0], hv[1], hv[2], hv[3]);
                *reinterpret_cast<u16x4 *>(reinterpret_cast<char *>(dHb) + o) = pack4(gv[0], gv[1], gv[2], gv[3]);
            }
            dotp = wave_total(dotp);
            if (lane == 0) sm.dot[wave] = dotp;
        }
        // the other parity slot is free: this head reads only lam[par], dt[par], and
        // the barrier below publishes the next head's values before its first use
        if (wave == 0) scan(hn, par ^ 1);
        __syncthreads();
        // the next head's chunk-boundary state and exit gradient (this head's were consumed
        // by the state products in S2)
        load_states(hn);
        // the next head's decay factors (waves 0..3)
        factors(par ^ 1);
        // this head's per-token scales of the Phase III/IV tiles (token 16 (2 wm + t) + lr)
        float ei_t[2], wdt_t[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int i = 16 * (2 * wm + t) + lr;
            const float2 e = *reinterpret_cast<const float2 *>(&sm.tk[par][i]);
            ei_t[t] = e.x;
            wdt_t[t] = e.y;
        }
        // ---- S4: Phase II (dx, ddt direct) on waves 0..7: p-tile wq, j-tiles 2 wj, 2 wj + 1.
        // Waves 8..15, the youngest of each SIMD and the last to reach every barrier, go
        // straight to Phases III/IV; the two j-tiles of a wave share its dy and dH fragments.
        if (wave < 8) {
            const int jb = 2 * wj;
            f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            f32x4 acc4[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            // Q[i][j] = 0 for i < j, so the kk block below the diagonal adds zeros
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 fy = frag_tr64(sm.dY, sl, wq, kk);
#pragma unroll
                for (int t = 0; t < 2; ++t) acc[t] = mfma(fy, lds_frag(sm.QT, swz_row64(sl, jb + t, kk)), acc[t]);
            }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x8 fd = lds_frag(dHb, swz_row128(sl, wq, kk));
#pragma unroll
                for (int t = 0; t < 2; ++t) acc4[t] = mfma(fd, lds_frag(sm.B, swz_row128(sl, jb + t, kk)), acc4[t]);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int j = 16 * (jb + t) + lr;
                const float2 wd = *reinterpret_cast<const float2 *>(&sm.tk[par][j].z);
                const float wjv = wd.x, dt_j = wd.y;
                const uint32_t o = swz_pc64(sl, jb + t, wq);
                const u16x4 x4 = *reinterpret_cast<const u16x4 *>(reinterpret_cast<const char *>(sm.X) + o);
                const u16x4 y4 = *reinterpret_cast<const u16x4 *>(reinterpret_cast<const char *>(sm.dY) + o);
                // acc4[j][p] = (dH B_j)[p]: with x it also gives the exit-gradient term
                // f_j = w_j dt_j x_j.(dH B_j) of dLam (this wave's p-tile)
                float ddp = 0.f, xb = 0.f, dxv[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float xv = bf16_to_f32(x4[v]);
                    const float pre = fmaf(wjv, acc4[t][v], acc[t][v]);
                    ddp = fmaf(xv, pre, ddp);
                    xb = fmaf(xv, acc4[t][v], xb);
                    dxv[v] = fmaf(Dh, bf16_to_f32(y4[v]), dt_j * pre);
                }
                buf_st_8b(rdx, static_cast<uint32_t>(k * kLs + j) * tokb + (h * kP + 16 * wq + lq) * 2,
                          pack4(dxv[0], dxv[1], dxv[2], dxv[3]));
                // both sums over the tile's four lane rows in one pass: row 0 holds dd, row 1 f
                const float sums = rows4_sum2(ddp, xb * (wjv * dt_j));
                if (lane < 32) *(lane < 16 ? &sm.dd[j][wq] : &sm.fp[j][wq]) = sums;
            }
        }
        // Phase III / IV: per-head dC, dB contributions (n-tile wn, tok-tiles 2wm, 2wm+1);
        // the state fragments are read once for both token tiles.
        {
            bf16x8 fH[2], fdH[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                fH[kk] = frag_tr128(Hb, sl, wn, kk);
                fdH[kk] = frag_tr128(dHb, sl, wn, kk);
            }
            float o[2];  // dy_i.(H C_i) exp(Lam_i), partial over the lane's n
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int tt = 2 * wm + t;
                f32x4 ac = {0.f, 0.f, 0.f, 0.f}, ab = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    ac = mfma(fH[kk], lds_frag(sm.dY, swz_row64(sl, tt, kk)), ac);
                    ab = mfma(fdH[kk], lds_frag(sm.X, swz_row64(sl, tt, kk)), ab);
                }
                const float ei = ei_t[t], wdt = wdt_t[t];
                // the token's scale ei is fused into the accumulate and applied to the dot
                // product once per lane
                float ot = 0.f;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    ot = fmaf(cC[t][v], ac[v], ot);
                    dCa[t][v] = fmaf(ac[v], ei, dCa[t][v]);
                    dBa[t][v] = fmaf(ab[v], wdt, dBa[t][v]);
                }
                o[t] = ot * ei;
            }
            // both token tiles' sums over the four lane rows in one pass: row t holds tile t
            const float os = rows4_sum2(o[0], o[1]);
            if (lane < 32) sm.offin[16 * (2 * wm + (lane >> 4)) + lr][wn] = os;
        }
        __syncthreads();
    }
    // the last head's combine (its partials were published by the final S4 barrier)
    if (wave == 0) combine(h0 + hpg - 1, (hpg - 1) & 1);

    // sum_h K applied once: dC^T[n][i] += sum_j B[j][n] K[i][j]; dB^T[n][j] += sum_i C[i][n] K[i][j]
    refresh_lane();
    __syncthreads();
    *reinterpret_cast<u16x4 *>(reinterpret_cast<char *>(sm.QT) + swz_pc64(sl, gj, gi)) = pack4(Ks[0], Ks[1], Ks[2], Ks[3]);
    __syncthreads();
    {
        const bf16_t *KT = sm.QT;  // [j][i]
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int tt = 2 * wm + t;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                dCa[t] = mfma(frag_tr128(sm.B, sl, wn, kk), frag_tr64(KT, sl, tt, kk), dCa[t]);
                dBa[t] = mfma(frag_tr128(sm.C, sl, wn, kk), lds_frag(KT, swz_row64(sl, tt, kk)), dBa[t]);
            }
            const int tl = 16 * tt + lr;
            if (tk + tl < T) {
                const int64_t o = ((b * T + tk + tl) * a.G + g) * kN + 16 * wn + lq;
                *reinterpret_cast<float4 *>(a.dC + o) = make_float4(dCa[t][0], dCa[t][1], dCa[t][2], dCa[t][3]);
                *reinterpret_cast<float4 *>(a.dB + o) = make_float4(dBa[t][0], dBa[t][1], dBa[t][2], dBa[t][3]);
            }
        }
    }
}

// ===========================================================================
// 3. dA, dD: fixed-order fp64 sums over batch, chunks and blocks
// ===========================================================================
// One 64-lane workgroup per head: lane l sums partials l, l+64, ... of the head's
// (batch, block) list in order, then lane 0 adds the 64 lane sums in lane order
// (a fixed order, so dA and dD do not depend on scheduling).
__global__ void __launch_bounds__(64) ssd_bwd_params_kernel(SsdBwdArgs a) {
    __shared__ double red[2][64];
    const int h = blockIdx.x, lane = threadIdx.x;
    const int64_t per = a.nchunks * (a.L / kLs);
    const int64_t total = a.Bsz * per;
    double sa = 0.0, sd = 0.0;
    for (int64_t i = lane; i < total; i += 64) {
        const int64_t bidx = i / per, k = i % per;
        const int64_t o = (bidx * a.H + h) * per + k;
        sa += a.pA[o];
        sd += a.pD[o];
    }
    red[0][lane] = sa;
    red[1][lane] = sd;
    __syncthreads();
    if (lane == 0) {
        double ta = 0.0, td = 0.0;
        for (int l = 0; l < 64; ++l) {
            ta += red[0][l];
            td += red[1][l];
        }
        a.dA[h] = static_cast<float>(ta);
        a.dD[h] = static_cast<float>(td);
    }
}

}  // namespace

hipError_t launch_ssd_bwd(const SsdBwdArgs &a, hipEvent_t ev_begin, hipEvent_t ev_end, hipStream_t s) {
    // (every dA, dD partial is written by the per-block kernel, zero for blocks past the end
    // of the sequence, so the workspace needs no clearing)
    // four 4-wave workgroups per CU when the grid fills the chip that deep, else 8 waves
    hipError_t e;
    int cus = 0;
    if ((e = device_cu_count(&cus)) != hipSuccess) return e;
    const int64_t nbh = a.Bsz * a.H;
    if (nbh >= 4 * static_cast<int64_t>(cus))
        ssd_bwd_dstate_kernel<4><<<static_cast<unsigned>(nbh), 256, 0, s>>>(a);
    else
        ssd_bwd_dstate_kernel<8><<<static_cast<unsigned>(nbh), 512, 0, s>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nwg = a.Bsz * a.G * a.nchunks * (a.L / kLs);
    if (ev_begin != nullptr && (e = hipEventRecord(ev_begin, s)) != hipSuccess) return e;
    ssd_bwd_block_kernel<<<static_cast<unsigned>(nwg), kBlkThreads, 0, s>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev_end != nullptr && (e = hipEventRecord(ev_end, s)) != hipSuccess) return e;
    ssd_bwd_params_kernel<<<static_cast<unsigned>(a.H), 64, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace ssm
