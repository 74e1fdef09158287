// recurrence.hip -- token-serial kernels of the selective SSM recurrence on gfx950:
//   * decode step (one token, state streamed from HBM and written back in place)
//   * replay / sequential scan (state held in registers across tokens; optional
//     y, chunk-state saves, and a lockstep "live" copy with per-step drift)
//   * exact-fp32 reverse sweep (the backward for dims or dtypes the chunked
//     MFMA kernels do not serve)
//
// The per-token update is the coordinate formula of theorem updateHead_apply
// ("Nemotron 3 Ultra: replaying a rounded state", section "The Mamba state
// update"): s = exp(dt*A) * s + x[p] * (B[n] * dt), and the output reads the
// updated state (section "Recovering the state by replay", the example whose
// output is 12).  Decode and replay call the same row_step() with the same lane
// mapping and the same reduction tree, so one replayed token equals one decode
// call bit for bit (every rounding is pinned with explicit fmaf / __fmul_rn).
//
// Thread mapping (both kernels): a state row of N floats is covered by
// LPR = N/4 lanes holding 4 consecutive coordinates each (16-byte accesses);
// a 256-thread workgroup covers 256/LPR rows per pass and one (batch, head).
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "sr16.hpp"

namespace ssm {

// Update 4 consecutive coordinates of one row and return their part of C.s.
__device__ __forceinline__ float row_step(float4 &s, float a, float xp, const float4 &bdt,
                                          const float4 &c) {
    s.x = fmaf(a, s.x, __fmul_rn(xp, bdt.x));
    s.y = fmaf(a, s.y, __fmul_rn(xp, bdt.y));
    s.z = fmaf(a, s.z, __fmul_rn(xp, bdt.z));
    s.w = fmaf(a, s.w, __fmul_rn(xp, bdt.w));
    float acc = __fmul_rn(c.x, s.x);
    acc = fmaf(c.y, s.y, acc);
    acc = fmaf(c.z, s.z, acc);
    acc = fmaf(c.w, s.w, acc);
    return acc;
}

// Same update without the read (for the lockstep live copy).
__device__ __forceinline__ void row_update(float4 &s, float a, float xp, const float4 &bdt) {
    s.x = fmaf(a, s.x, __fmul_rn(xp, bdt.x));
    s.y = fmaf(a, s.y, __fmul_rn(xp, bdt.y));
    s.z = fmaf(a, s.z, __fmul_rn(xp, bdt.z));
    s.w = fmaf(a, s.w, __fmul_rn(xp, bdt.w));
}

// Sum over the LPR lanes of one row (DPP within 16-lane rows, permlane swaps
// across them; the same fixed order in decode and replay).
template <int LPR>
__device__ __forceinline__ float row_reduce(float acc) {
    return lane_group_reduce<LPR, false>(acc);
}

__device__ __forceinline__ float retention(float dtv, float Ah) { return expf(__fmul_rn(dtv, Ah)); }

__device__ __forceinline__ float4 scale4(const float4 &v, float s) {
    return make_float4(__fmul_rn(v.x, s), __fmul_rn(v.y, s), __fmul_rn(v.z, s), __fmul_rn(v.w, s));
}

// ---------------------------------------------------------------------------
// Decode: one (batch, head) per workgroup, all row passes unrolled so all state
// loads are in flight before the arithmetic.  With SR16 the state lives in
// binary16: it is widened exactly, updated in float32 with the same arithmetic,
// and stored back stochastically rounded ("Nemotron 3 Ultra: replaying a rounded
// state": the quantized model keeps its recurrent state cache in FP16 with
// stochastic rounding), element e of the state using entropy (seed, key, e).
// A lane holds CPL consecutive coordinates of a row: 4 for the float32 state
// (16-byte accesses), 8 for the binary16 one (16-byte accesses too, so the binary16
// cache needs half the memory instructions).  With 8 the lane first adds its two
// 4-coordinate partial sums and the row reduction runs over half as many lanes: the
// same pairs are added in the same tree as with 4, so y is bit-identical to the
// float32 decode of the same (widened) state.
// ---------------------------------------------------------------------------
template <int N, int MAXR, typename T, bool SR16>
__global__ void __launch_bounds__(256) decode_kernel(DecodeArgs a) {
    constexpr int CPL = SR16 ? 8 : 4;          // coordinates per lane
    constexpr int NV = CPL / 4;                // float4 sub-vectors per lane
    constexpr int LPR = N / CPL;               // lanes per state row
    constexpr int RPW = 256 / LPR;             // rows per pass
    constexpr int NPASS = MAXR * 4 / CPL;      // passes (same row capacity for both CPL)
    const int bh = blockIdx.x;
    const int b = bh / a.H, h = bh % a.H, g = h / (a.H / a.G);
    const int tid = threadIdx.x;
    const int n0 = (tid % LPR) * CPL;
    const int r0 = tid / LPR;
    const T *x = static_cast<const T *>(a.x);
    const T *Bm = static_cast<const T *>(a.B);
    const T *Cm = static_cast<const T *>(a.C);
    const int64_t row_base = static_cast<int64_t>(bh) * a.P;  // state row index of p = 0
    float *st = SR16 ? nullptr : a.state + row_base * N;
    uint16_t *st16 = SR16 ? a.state16 + row_base * N : nullptr;

    float4 s[NPASS][NV];
#pragma unroll
    for (int i = 0; i < NPASS; ++i) {
        const int p = r0 + i * RPW;
#pragma unroll
        for (int q = 0; q < NV; ++q) s[i][q] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (p < a.P) {
            if constexpr (SR16) {
                // binary16 -> float32 is exact; convert the whole vector (an element-wise
                // bit_cast of a vector subscript is not reliable here)
                typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
                typedef float f32x8 __attribute__((ext_vector_type(8)));
                const h16x8 hv = __builtin_nontemporal_load(reinterpret_cast<const h16x8 *>(st16 + static_cast<int64_t>(p) * N + n0));
                const f32x8 fv = __builtin_convertvector(hv, f32x8);
                s[i][0] = make_float4(fv[0], fv[1], fv[2], fv[3]);
                s[i][1] = make_float4(fv[4], fv[5], fv[6], fv[7]);
            } else {
                s[i][0] = nt_ld4(st + static_cast<int64_t>(p) * N + n0);
            }
        }
    }
    const float dtv = a.dt[bh];
    const float av = retention(dtv, a.A[h]);
    const float Dh = a.D[h];
    const int64_t bgN = (static_cast<int64_t>(b) * a.G + g) * N + n0;
    float4 bdt[NV], c[NV];
#pragma unroll
    for (int q = 0; q < NV; ++q) {
        bdt[q] = scale4(IO<T>::ld4(Bm, bgN + 4 * q), dtv);
        c[q] = IO<T>::ld4(Cm, bgN + 4 * q);
    }
    const uint64_t sub = SR16 ? sr16_stream(a.seed, a.key) : 0ull;
#pragma unroll
    for (int i = 0; i < NPASS; ++i) {
        if (i * RPW >= a.P) break;  // uniform: no row of this pass exists
        const int p = r0 + i * RPW;
        const float xp = (p < a.P) ? IO<T>::ld(x, static_cast<int64_t>(bh) * a.P + p) : 0.f;
        float acc = row_step(s[i][0], av, xp, bdt[0], c[0]);
        if constexpr (NV == 2) acc = acc + row_step(s[i][1], av, xp, bdt[1], c[1]);
        acc = row_reduce<LPR>(acc);  // whole rows are active or inactive together
        if (p < a.P) {
            if constexpr (SR16) {
                const uint64_t e0 = static_cast<uint64_t>(row_base + p) * N + n0;  // element index
                uint32_t u[8];
                sr16_entropy_run<8>(sub, e0, u);
                const float v[8] = {s[i][0].x, s[i][0].y, s[i][0].z, s[i][0].w,
                                    s[i][1].x, s[i][1].y, s[i][1].z, s[i][1].w};
                u16x8 o;
#pragma unroll
                for (int j = 0; j < 8; ++j) o[j] = sr16_bits(v[j], u[j]);
                __builtin_nontemporal_store(o, reinterpret_cast<u16x8 *>(st16 + static_cast<int64_t>(p) * N + n0));
            } else {
                nt_st4(st + static_cast<int64_t>(p) * N + n0, s[i][0]);
            }
            if ((tid % LPR) == 0)
                IO<T>::st(static_cast<T *>(a.y), static_cast<int64_t>(bh) * a.P + p,
                          fmaf(Dh, xp, acc));
        }
    }
}

// ---------------------------------------------------------------------------
// Token-serial scan / replay: state in registers across r tokens.  The per-token
// inputs are staged in LDS TT tokens at a time (the retention factor, B*dt and C
// as floats, x permuted so a thread's MAXR rows are contiguous), and the next
// tile is loaded into registers while the current one is consumed.
// ---------------------------------------------------------------------------
template <int N>
struct ScanTile {
    static constexpr int LPR = N / 4;                       // lanes per state row
    static constexpr int RPW = 256 / LPR;                   // rows per pass
    static constexpr int TT = (2 * LPR < 16) ? 2 * LPR : 16;  // tokens per tile
    static constexpr int NJ = (TT * LPR + 255) / 256;       // (token, 4 coords) items per thread
    static constexpr int XW = 8 * RPW;                      // staged x width (MAXR = 8 passes)
    static constexpr int XJ = TT * XW / 256;                // x elements per thread
};

template <int N, int MAXR, typename T, typename CK, bool LIVE>
__global__ void __launch_bounds__(256) scan_kernel(ScanArgs a) {
    using TL = ScanTile<N>;
    constexpr int LPR = TL::LPR, RPW = TL::RPW, TT = TL::TT, NJ = TL::NJ, XW = TL::XW, XJ = TL::XJ;
    static_assert(MAXR == 8, "tile layout assumes 8 row passes");
    __shared__ float s_av[TT];
    __shared__ __align__(16) float s_bdt[TT * N];
    __shared__ __align__(16) float s_c[TT * N];
    __shared__ __align__(16) float s_x[TT * XW];

    const int bh = blockIdx.x;
    const int b = bh / a.H, h = bh % a.H, g = h / (a.H / a.G);
    const int tid = threadIdx.x;
    const int n0 = (tid % LPR) * 4;
    const int r0 = tid / LPR;
    const int64_t PN = static_cast<int64_t>(a.P) * N;
    const T *x = static_cast<const T *>(a.x);
    const T *Bm = static_cast<const T *>(a.B);
    const T *Cm = static_cast<const T *>(a.C);
    T *y = static_cast<T *>(a.y);
    const bool want_y = (y != nullptr);

    float4 s[MAXR];
    float4 l[LIVE ? MAXR : 1];
#pragma unroll
    for (int i = 0; i < MAXR; ++i) {
        const int p = r0 + i * RPW;
        s[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (LIVE) l[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (p < a.P) {
            const int64_t off = bh * PN + static_cast<int64_t>(p) * N + n0;
            if (a.ckpt != nullptr) {
                const CK *ck = static_cast<const CK *>(a.ckpt);
                if constexpr (sizeof(CK) == 4) {
                    s[i] = nt_ld4(ck + off);
                } else {
                    const _Float16 *hk = reinterpret_cast<const _Float16 *>(ck + off);
                    s[i] = make_float4(static_cast<float>(hk[0]), static_cast<float>(hk[1]),
                                       static_cast<float>(hk[2]), static_cast<float>(hk[3]));
                }
            }
            if constexpr (LIVE) l[i] = nt_ld4(a.live + off);
        }
    }
    const float Ah = a.A[h];
    const float Dh = a.D[h];
    const int wave = tid / 64, lane = tid % 64;
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * 4;

    // next tile in registers: (token, 4 coords) items of B, C with their dt; x elements
    using Raw4 = typename std::conditional<sizeof(T) == 2, u16x4, float4>::type;
    Raw4 rb[NJ], rc[NJ];
    float rdt[NJ], rx[XJ];
    auto raw4 = [](const T *p, int64_t i) { return *reinterpret_cast<const Raw4 *>(p + i); };
    auto wide4 = [](const Raw4 &v) -> float4 {
        if constexpr (sizeof(T) == 2)
            return make_float4(bf16_to_f32(v[0]), bf16_to_f32(v[1]), bf16_to_f32(v[2]), bf16_to_f32(v[3]));
        else
            return v;
    };
    auto prefetch = [&](int64_t k0) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int q = tid + 256 * j, tt = q / LPR, nn = (q % LPR) * 4;
            rb[j] = rc[j] = Raw4{};
            rdt[j] = 0.f;
            if (q < TT * LPR && k0 + tt < a.r) {
                const int64_t bt = static_cast<int64_t>(b) * a.T + a.t0 + k0 + tt;
                const int64_t bgN = (bt * a.G + g) * N + nn;
                rb[j] = raw4(Bm, bgN);
                rc[j] = raw4(Cm, bgN);
                rdt[j] = a.dt[bt * a.H + h];
            }
        }
#pragma unroll
        for (int j = 0; j < XJ; ++j) {
            const int e = tid + 256 * j, tt = e / XW, p = e % XW;
            rx[j] = 0.f;
            if (p < a.P && k0 + tt < a.r) {
                const int64_t bt = static_cast<int64_t>(b) * a.T + a.t0 + k0 + tt;
                rx[j] = IO<T>::ld(x, (bt * a.H + h) * a.P + p);
            }
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int q = tid + 256 * j, tt = q / LPR, nn = (q % LPR) * 4;
            if (q < TT * LPR) {
                *reinterpret_cast<float4 *>(&s_bdt[tt * N + nn]) = scale4(wide4(rb[j]), rdt[j]);
                *reinterpret_cast<float4 *>(&s_c[tt * N + nn]) = wide4(rc[j]);
                if (nn == 0) s_av[tt] = retention(rdt[j], Ah);
            }
        }
#pragma unroll
        for (int j = 0; j < XJ; ++j) {
            const int e = tid + 256 * j, tt = e / XW, p = e % XW;
            s_x[tt * XW + (p % RPW) * MAXR + p / RPW] = rx[j];  // row p = r0 + i*RPW -> r0*MAXR + i
        }
    };

    if (a.r > 0) prefetch(0);
    for (int64_t k0 = 0; k0 < a.r; k0 += TT) {
        __syncthreads();  // the previous tile has been consumed
        stage();
        __syncthreads();
        if (k0 + TT < a.r) prefetch(k0 + TT);
        const int nt = (a.r - k0 < TT) ? static_cast<int>(a.r - k0) : TT;
        for (int tt = 0; tt < nt; ++tt) {
            const int64_t k = k0 + tt;
            if (a.chunk_states != nullptr && (k % a.L) == 0) {
                float *cs = a.chunk_states + (bh * a.nchunks + k / a.L) * PN;
#pragma unroll
                for (int i = 0; i < MAXR; ++i) {
                    const int p = r0 + i * RPW;
                    if (p < a.P) *reinterpret_cast<float4 *>(cs + static_cast<int64_t>(p) * N + n0) = s[i];
                }
            }
            const float av = s_av[tt];
            const float4 bdt = *reinterpret_cast<const float4 *>(&s_bdt[tt * N + n0]);
            const float4 xa = *reinterpret_cast<const float4 *>(&s_x[tt * XW + r0 * MAXR]);
            const float4 xb = *reinterpret_cast<const float4 *>(&s_x[tt * XW + r0 * MAXR + 4]);
            const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
            float dmax = 0.f, dsum = 0.f;
            if (want_y) {
                const float4 c = *reinterpret_cast<const float4 *>(&s_c[tt * N + n0]);
                const int64_t xrow = ((static_cast<int64_t>(b) * a.T + a.t0 + k) * a.H + h) * a.P;
#pragma unroll
                for (int i = 0; i < MAXR; ++i) {
                    if (i * RPW >= a.P) break;  // uniform
                    const int p = r0 + i * RPW;
                    float acc = row_step(s[i], av, xv[i], bdt, c);
                    acc = row_reduce<LPR>(acc);
                    if (p < a.P && (tid % LPR) == 0) IO<T>::st(y, xrow + p, fmaf(Dh, xv[i], acc));
                }
            } else {
#pragma unroll
                for (int i = 0; i < MAXR; ++i) row_update(s[i], av, xv[i], bdt);
            }
            if (a.snap != nullptr) {  // snapshot stack: the state after this token
                float *sp = a.snap + (k + 1) * a.snap_stride + bh * PN;
#pragma unroll
                for (int i = 0; i < MAXR; ++i) {
                    const int p = r0 + i * RPW;
                    if (p < a.P) *reinterpret_cast<float4 *>(sp + static_cast<int64_t>(p) * N + n0) = s[i];
                }
            }
            if constexpr (LIVE) {
#pragma unroll
                for (int i = 0; i < MAXR; ++i) {
                    row_update(l[i], av, xv[i], bdt);  // rows past P stay zero in both copies
                    const float d0 = fabsf(s[i].x - l[i].x), d1 = fabsf(s[i].y - l[i].y);
                    const float d2 = fabsf(s[i].z - l[i].z), d3 = fabsf(s[i].w - l[i].w);
                    dmax = fmaxf(dmax, fmaxf(fmaxf(d0, d1), fmaxf(d2, d3)));
                    dsum += (d0 + d1) + (d2 + d3);
                }
                dmax = lane_group_reduce<64, true>(dmax);
                dsum = lane_group_reduce<64, false>(dsum);
                if (lane == 0) {
                    const int64_t w = static_cast<int64_t>(bh) * 4 + wave;
                    a.part_max[k * nwaves + w] = dmax;
                    a.part_sum[k * nwaves + w] = dsum;
                }
            }
        }
    }
    if (a.state_out != nullptr) {
#pragma unroll
        for (int i = 0; i < MAXR; ++i) {
            const int p = r0 + i * RPW;
            if (p < a.P)
                *reinterpret_cast<float4 *>(a.state_out + bh * PN + static_cast<int64_t>(p) * N + n0) = s[i];
        }
    }
}

// ---------------------------------------------------------------------------
// Replay without the lockstep copy, snapshots or chunk saves: the state (and, when
// asked, y) of r retained tokens.  No LDS and no barrier: a thread holds 8
// consecutive rows of 4 coordinates, so each token needs one 16-byte load of x (its 8
// rows in bf16), 4 values of B (and of C), and every wave streams its own rows.  The
// retention factors are computed 64 tokens at a time, one token per lane, and each
// token's dt and exp(dt*A) are then read from its lane with readlane (one transcendental
// per 64 tokens instead of one per token).  A token's inputs are loaded one token
// ahead, as raw bits, and widened when used.  The update and the read are row_update /
// row_step with the retention, B*dt and lane tree of the decode kernel, so the states
// and outputs equal those of r decode calls bit for bit.  A 256-thread workgroup covers
// 1024 * 8 / N rows of one (batch, head).  Requires x 16-byte aligned and headdim a
// multiple of 8 (the host checks); rows past headdim are never touched.
// ---------------------------------------------------------------------------
constexpr int kReplayRows = 8;  // rows per thread

template <int N, typename T, typename CK, bool Y>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 4 ? 4 : (Y ? 6 : 8))))
replay_kernel(ScanArgs a) {
    constexpr int LPR = N / 4;  // lanes per state row
    constexpr int R = kReplayRows;
    const int bh = blockIdx.x;
    const int b = bh / a.H, h = bh % a.H, g = h / (a.H / a.G);
    const int tid = threadIdx.x, lane = tid & 63;
    const int n0 = (tid % LPR) * 4;
    const int p0 = (tid / LPR) * R;  // first of this thread's rows
    const int64_t PN = static_cast<int64_t>(a.P) * N;
    const bool rows = p0 < a.P;      // all R rows exist (P % R == 0); whole lane groups agree
    const int xoff = rows ? p0 : 0;  // lanes without rows read row 0's x and discard it

    float4 s[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        s[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (rows && a.ckpt != nullptr) {
            const int64_t off = bh * PN + static_cast<int64_t>(p0 + i) * N + n0;
            const CK *ck = static_cast<const CK *>(a.ckpt);
            if constexpr (sizeof(CK) == 4) {
                s[i] = nt_ld4(ck + off);
            } else {
                typedef _Float16 h16x4 __attribute__((ext_vector_type(4)));
                typedef float f32x4v __attribute__((ext_vector_type(4)));
                const h16x4 hv = __builtin_nontemporal_load(reinterpret_cast<const h16x4 *>(ck + off));
                const f32x4v fv = __builtin_convertvector(hv, f32x4v);
                s[i] = make_float4(fv[0], fv[1], fv[2], fv[3]);
            }
        }
    }
    if (a.r > 0) {
        const float Ah = a.A[h], Dh = a.D[h];
        // token k of the replay is token t0 + k of the sequence
        const int64_t tok0 = static_cast<int64_t>(b) * a.T + a.t0;
        const int64_t xs = static_cast<int64_t>(a.H) * a.P, bs = static_cast<int64_t>(a.G) * N;
        const T *xk = static_cast<const T *>(a.x) + (tok0 * a.H + h) * a.P + xoff;
        const T *bk = static_cast<const T *>(a.B) + (tok0 * a.G + g) * N + n0;
        const T *ck = static_cast<const T *>(a.C) + (tok0 * a.G + g) * N + n0;
        const float *dk = a.dt + tok0 * a.H + h;
        T *yk = Y ? static_cast<T *>(a.y) + (tok0 * a.H + h) * a.P + p0 : nullptr;
        using Raw = typename std::conditional<sizeof(T) == 2, u16x4, float4>::type;  // 4 values
        using RawX = typename std::conditional<sizeof(T) == 2, u16x8, float4>::type;
        constexpr int XL = sizeof(T) == 2 ? 1 : 2;  // 16-byte loads of x per token
        auto raw4 = [](const T *q) { return *reinterpret_cast<const Raw *>(q); };
        auto wide = [](const Raw &v) -> float4 {
            if constexpr (sizeof(T) == 2)
                return make_float4(bf16_to_f32(v[0]), bf16_to_f32(v[1]), bf16_to_f32(v[2]), bf16_to_f32(v[3]));
            else
                return v;
        };
        auto xload = [&](RawX *dst, int64_t k) {
#pragma unroll
            for (int q = 0; q < XL; ++q) dst[q] = *reinterpret_cast<const RawX *>(xk + k * xs + q * 4);
        };
        auto xwide = [&](const RawX *v, int i) -> float {
            if constexpr (sizeof(T) == 2) return bf16_to_f32(v[0][i]);
            else return reinterpret_cast<const float *>(&v[i / 4])[i % 4];
        };
        Raw bq = raw4(bk), cq{};
        if constexpr (Y) cq = raw4(ck);
        RawX xq[XL];
        xload(xq, 0);
        float dt_l = 0.f, av_l = 0.f;  // dt and retention of token k0 + lane
        for (int64_t k = 0; k < a.r; ++k) {
            const int kl = static_cast<int>(k & 63);
            if (kl == 0) {
                const int64_t kk = k + lane;
                dt_l = (kk < a.r) ? dk[kk * a.H] : 0.f;
                av_l = retention(dt_l, Ah);
            }
            const float dtv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dt_l), kl));
            const float av = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(av_l), kl));
            const Raw bc = bq, cc = cq;
            RawX xc[XL];
#pragma unroll
            for (int q = 0; q < XL; ++q) xc[q] = xq[q];
            const int64_t kn = (k + 1 < a.r) ? k + 1 : k;  // the last token re-reads itself
            bq = raw4(bk + kn * bs);
            if constexpr (Y) cq = raw4(ck + kn * bs);
            xload(xq, kn);
            const float4 bdt = scale4(wide(bc), dtv);
            if constexpr (Y) {
                const float4 c = wide(cc);
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    const float xp = xwide(xc, i);
                    float acc = row_step(s[i], av, xp, bdt, c);
                    acc = row_reduce<LPR>(acc);
                    if (rows && (tid % LPR) == 0) IO<T>::st(yk, k * xs + i, fmaf(Dh, xp, acc));
                }
            } else {
#pragma unroll
                for (int i = 0; i < R; ++i) row_update(s[i], av, xwide(xc, i), bdt);
            }
        }
    }
    if (a.state_out != nullptr && rows) {
#pragma unroll
        for (int i = 0; i < R; ++i)
            *reinterpret_cast<float4 *>(a.state_out + bh * PN + static_cast<int64_t>(p0 + i) * N + n0) = s[i];
    }
}

// ---------------------------------------------------------------------------
// Rollback after verification of a draft ("Nemotron 3 Ultra: replaying a rounded
// state", section "Rolling back rejected draft tokens": the selected snapshot is
// the state after the accepted prefix).  A gather copy, 16 bytes per lane: grid
// (chunks of a sequence's state, sequence).  An accepted count outside
// [0, ndraft] writes nothing for that sequence and raises the error flag.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) rollback_kernel(RollbackArgs a) {
    const int64_t b = blockIdx.y;
    const int32_t acc = a.accepted[b];
    if (acc < 0 || acc > a.ndraft) {
        if (a.err != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *a.err = 1;
        return;
    }
    const int64_t n4 = a.per_seq / 4;
    const float *src = a.snap + (static_cast<int64_t>(acc) * a.Bsz + b) * a.per_seq;
    float *dst = a.state_out + b * a.per_seq;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4; i += stride)
        nt_st4(dst + 4 * i, nt_ld4(src + 4 * i));
}

hipError_t launch_rollback(const RollbackArgs &a, hipStream_t s) {
    if (a.Bsz == 0 || a.per_seq == 0) return hipSuccess;
    int64_t chunks = (a.per_seq / 4 + 255) / 256;
    if (chunks > 4096) chunks = 4096;  // grid-stride beyond this
    rollback_kernel<<<dim3(static_cast<unsigned>(chunks), static_cast<unsigned>(a.Bsz)), 256, 0, s>>>(a);
    return hipGetLastError();
}

// Fixed-order reduction of the per-wave drift partials: one thread per step.
__global__ void drift_reduce_kernel(const float *part_max, const float *part_sum, int64_t nwaves,
                                    int64_t r, double inv_count, float *drift_max,
                                    float *drift_mean) {
    const int64_t k = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (k >= r) return;
    float m = 0.f;
    double s = 0.0;
    for (int64_t w = 0; w < nwaves; ++w) {
        m = fmaxf(m, part_max[k * nwaves + w]);
        s += static_cast<double>(part_sum[k * nwaves + w]);
    }
    drift_max[k] = m;
    drift_mean[k] = static_cast<float>(s * inv_count);
}

// ---------------------------------------------------------------------------
// Exact-fp32 reverse sweep, one (batch, head) per workgroup.  Per token, from
// the last to the first ("Nemotron Kernels: From Inference To
// Backpropagation", Kernel 1 backward: output path plus future path; branch
// contributions add):
//   gs += dy (outer) C;  dC_t += dy . s_t;  dx = D dy + dt (gs B);
//   dB_t += dt (gs^T x);  ddt = x.(gs B) + a A <gs, s_{t-1}>;
//   dA += a dt <gs, s_{t-1}>;  dD += dy . x;  gs *= a.
// States of one chunk are rebuilt from chunk_states into a workspace slab.
// dB/dC go to per-head partials that a second kernel sums over the group in
// ascending head order.
// ---------------------------------------------------------------------------
template <int N, int MAXR, typename T>
__global__ void __launch_bounds__(256) scan_bwd_kernel(ScanBwdArgs a) {
    constexpr int LPR = N / 4;
    constexpr int RPW = 256 / LPR;
    __shared__ float red_c[RPW * N];
    __shared__ float red_b[RPW * N];
    __shared__ float red_w[3][4];
    const int bh = blockIdx.x;
    const int b = bh / a.H, h = bh % a.H, g = h / (a.H / a.G);
    const int tid = threadIdx.x;
    const int n0 = (tid % LPR) * 4;
    const int r0 = tid / LPR;
    const int wave = tid / 64, lane = tid % 64;
    const int64_t PN = static_cast<int64_t>(a.P) * N;
    const T *x = static_cast<const T *>(a.x);
    const T *Bm = static_cast<const T *>(a.B);
    const T *Cm = static_cast<const T *>(a.C);
    const T *dy = static_cast<const T *>(a.dy);
    T *dx = static_cast<T *>(a.dx);
    float *slab = a.slab + static_cast<int64_t>(bh) * a.slab_stride;
    const float Ah = a.A[h], Dh = a.D[h];

    float4 gs[MAXR];
#pragma unroll
    for (int i = 0; i < MAXR; ++i) {
        const int p = r0 + i * RPW;
        gs[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (p < a.P && a.dh_final != nullptr)
            gs[i] = *reinterpret_cast<const float4 *>(a.dh_final + bh * PN + static_cast<int64_t>(p) * N + n0);
    }
    double dA_acc = 0.0, dD_acc = 0.0;  // used by thread 0 only

    for (int64_t c = a.nchunks - 1; c >= 0; --c) {
        const int64_t tlo = c * a.L;
        const int64_t thi = (tlo + a.L < a.T) ? tlo + a.L : a.T;
        // rebuild the chunk's states: slab[k] = state after token tlo+k-1
        float4 s[MAXR];
#pragma unroll
        for (int i = 0; i < MAXR; ++i) {
            const int p = r0 + i * RPW;
            if (p < a.P) {
                const int64_t off = static_cast<int64_t>(p) * N + n0;
                s[i] = *reinterpret_cast<const float4 *>(a.chunk_states + (bh * a.nchunks + c) * PN + off);
                *reinterpret_cast<float4 *>(slab + off) = s[i];
            }
        }
        for (int64_t t = tlo; t < thi; ++t) {
            const int64_t bt = static_cast<int64_t>(b) * a.T + t;
            const float dtv = a.dt[bt * a.H + h];
            const float av = retention(dtv, Ah);
            const float4 bdt = scale4(IO<T>::ld4(Bm, (bt * a.G + g) * N + n0), dtv);
#pragma unroll
            for (int i = 0; i < MAXR; ++i) {
                const int p = r0 + i * RPW;
                if (p < a.P) {
                    row_update(s[i], av, IO<T>::ld(x, (bt * a.H + h) * a.P + p), bdt);
                    *reinterpret_cast<float4 *>(slab + (t - tlo + 1) * PN + static_cast<int64_t>(p) * N + n0) = s[i];
                }
            }
        }
        // reverse walk over the chunk (each thread reads only what it wrote)
        for (int64_t t = thi - 1; t >= tlo; --t) {
            const int64_t bt = static_cast<int64_t>(b) * a.T + t;
            const float dtv = a.dt[bt * a.H + h];
            const float av = retention(dtv, Ah);
            const int64_t bgN = (bt * a.G + g) * N + n0;
            const float4 bn = IO<T>::ld4(Bm, bgN);
            const float4 cn = IO<T>::ld4(Cm, bgN);
            const int64_t xrow = (bt * a.H + h) * a.P;
            float4 pc = make_float4(0.f, 0.f, 0.f, 0.f);  // sum_p dy_p s_t[p, n]
            float4 pb = make_float4(0.f, 0.f, 0.f, 0.f);  // sum_p gs[p, n] x_p
            float wsum = 0.f, rsum = 0.f, dsum = 0.f;
#pragma unroll
            for (int i = 0; i < MAXR; ++i) {
                const int p = r0 + i * RPW;
                if (p < a.P) {
                    const int64_t off = static_cast<int64_t>(p) * N + n0;
                    const float4 st = *reinterpret_cast<const float4 *>(slab + (t - tlo + 1) * PN + off);
                    const float4 sp = *reinterpret_cast<const float4 *>(slab + (t - tlo) * PN + off);
                    const float dyp = IO<T>::ld(dy, xrow + p);
                    const float xp = IO<T>::ld(x, xrow + p);
                    gs[i].x = fmaf(dyp, cn.x, gs[i].x);
                    gs[i].y = fmaf(dyp, cn.y, gs[i].y);
                    gs[i].z = fmaf(dyp, cn.z, gs[i].z);
                    gs[i].w = fmaf(dyp, cn.w, gs[i].w);
                    pc.x = fmaf(dyp, st.x, pc.x);
                    pc.y = fmaf(dyp, st.y, pc.y);
                    pc.z = fmaf(dyp, st.z, pc.z);
                    pc.w = fmaf(dyp, st.w, pc.w);
                    pb.x = fmaf(gs[i].x, xp, pb.x);
                    pb.y = fmaf(gs[i].y, xp, pb.y);
                    pb.z = fmaf(gs[i].z, xp, pb.z);
                    pb.w = fmaf(gs[i].w, xp, pb.w);
                    float gb = gs[i].x * bn.x + gs[i].y * bn.y + gs[i].z * bn.z + gs[i].w * bn.w;
                    gb = row_reduce<LPR>(gb);
                    if ((tid % LPR) == 0) {
                        IO<T>::st(dx, xrow + p, fmaf(Dh, dyp, dtv * gb));
                        wsum = fmaf(xp, gb, wsum);
                        dsum = fmaf(dyp, xp, dsum);
                    }
                    rsum += gs[i].x * sp.x + gs[i].y * sp.y + gs[i].z * sp.z + gs[i].w * sp.w;
                }
            }
            // cross-row sums for dC / dB (fixed order over row groups)
            *reinterpret_cast<float4 *>(&red_c[r0 * N + n0]) = pc;
            *reinterpret_cast<float4 *>(&red_b[r0 * N + n0]) = pb;
            wsum = wave_sum(wsum);
            rsum = wave_sum(rsum);
            dsum = wave_sum(dsum);
            if (lane == 0) {
                red_w[0][wave] = wsum;
                red_w[1][wave] = rsum;
                red_w[2][wave] = dsum;
            }
            __syncthreads();
            if (tid < N) {
                float sc = 0.f, sb = 0.f;
                for (int r = 0; r < RPW; ++r) {
                    sc += red_c[r * N + tid];
                    sb += red_b[r * N + tid];
                }
                const int64_t o = (bt * a.H + h) * N + tid;
                a.dC_part[o] = sc;
                a.dB_part[o] = dtv * sb;
            }
            if (tid == 0) {
                const float W = (red_w[0][0] + red_w[0][1]) + (red_w[0][2] + red_w[0][3]);
                const float R = (red_w[1][0] + red_w[1][1]) + (red_w[1][2] + red_w[1][3]);
                const float S = (red_w[2][0] + red_w[2][1]) + (red_w[2][2] + red_w[2][3]);
                a.ddt[bt * a.H + h] = W + R * av * Ah;
                dA_acc += static_cast<double>(R) * av * dtv;
                dD_acc += static_cast<double>(S);
            }
#pragma unroll
            for (int i = 0; i < MAXR; ++i) {
                gs[i].x *= av;
                gs[i].y *= av;
                gs[i].z *= av;
                gs[i].w *= av;
            }
            __syncthreads();
        }
    }
    if (a.dh0 != nullptr) {
#pragma unroll
        for (int i = 0; i < MAXR; ++i) {
            const int p = r0 + i * RPW;
            if (p < a.P)
                *reinterpret_cast<float4 *>(a.dh0 + bh * PN + static_cast<int64_t>(p) * N + n0) = gs[i];
        }
    }
    if (tid == 0) {
        a.dA_part[bh] = dA_acc;
        a.dD_part[bh] = dD_acc;
    }
}

// dB/dC of a group = sum of the per-head partials in ascending head order.
__global__ void group_sum_kernel(const float *part_b, const float *part_c, float *dB, float *dC,
                                 int64_t BT, int H, int G, int N) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = BT * G * N;
    if (i >= total) return;
    const int n = static_cast<int>(i % N);
    const int64_t bg = i / N;
    const int g = static_cast<int>(bg % G);
    const int64_t bt = bg / G;
    const int hpg = H / G;
    float sb = 0.f, sc = 0.f;
    for (int k = 0; k < hpg; ++k) {
        const int64_t o = (bt * H + g * hpg + k) * N + n;
        sb += part_b[o];
        sc += part_c[o];
    }
    dB[i] = sb;
    dC[i] = sc;
}

// dA[h], dD[h] = sums over batch of per-(batch, head) fp64 partials.
__global__ void head_param_sum_kernel(const double *pa, const double *pd, float *dA, float *dD,
                                      int Bsz, int H) {
    const int h = blockIdx.x * blockDim.x + threadIdx.x;
    if (h >= H) return;
    double sa = 0.0, sd = 0.0;
    for (int b = 0; b < Bsz; ++b) {
        sa += pa[static_cast<int64_t>(b) * H + h];
        sd += pd[static_cast<int64_t>(b) * H + h];
    }
    dA[h] = static_cast<float>(sa);
    dD[h] = static_cast<float>(sd);
}

__global__ void fill_kernel(float *p, int64_t n, float v) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}
__global__ void copy_kernel(float *dst, const float *src, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------
hipError_t launch_fill(float *p, int64_t n, float v, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    fill_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(p, n, v);
    return hipGetLastError();
}
hipError_t launch_copy(float *dst, const float *src, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    copy_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(dst, src, n);
    return hipGetLastError();
}

template <typename T, bool SR16>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(a.Bsz * a.H)), block(256);
    switch (a.N) {
        case 16: decode_kernel<16, 8, T, SR16><<<grid, block, 0, s>>>(a); break;
        case 32: decode_kernel<32, 8, T, SR16><<<grid, block, 0, s>>>(a); break;
        case 64: decode_kernel<64, 8, T, SR16><<<grid, block, 0, s>>>(a); break;
        case 128: decode_kernel<128, 8, T, SR16><<<grid, block, 0, s>>>(a); break;
        case 256: decode_kernel<256, 8, T, SR16><<<grid, block, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, bool bf16, hipStream_t s) {
    if (a.state16 != nullptr)
        return bf16 ? launch_decode_t<bf16_t, true>(a, s) : launch_decode_t<float, true>(a, s);
    return bf16 ? launch_decode_t<bf16_t, false>(a, s) : launch_decode_t<float, false>(a, s);
}

template <typename T, typename CK, bool LIVE>
static hipError_t launch_scan_tcl(const ScanArgs &a, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(a.Bsz * a.H)), block(256);
    switch (a.N) {
        case 16: scan_kernel<16, 8, T, CK, LIVE><<<grid, block, 0, s>>>(a); break;
        case 32: scan_kernel<32, 8, T, CK, LIVE><<<grid, block, 0, s>>>(a); break;
        case 64: scan_kernel<64, 8, T, CK, LIVE><<<grid, block, 0, s>>>(a); break;
        case 128: scan_kernel<128, 8, T, CK, LIVE><<<grid, block, 0, s>>>(a); break;
        case 256: scan_kernel<256, 8, T, CK, LIVE><<<grid, block, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, typename CK, bool Y>
static hipError_t launch_replay_tcy(const ScanArgs &a, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(a.Bsz * a.H)), block(256);
    switch (a.N) {
        case 16: replay_kernel<16, T, CK, Y><<<grid, block, 0, s>>>(a); break;
        case 32: replay_kernel<32, T, CK, Y><<<grid, block, 0, s>>>(a); break;
        case 64: replay_kernel<64, T, CK, Y><<<grid, block, 0, s>>>(a); break;
        case 128: replay_kernel<128, T, CK, Y><<<grid, block, 0, s>>>(a); break;
        case 256: replay_kernel<256, T, CK, Y><<<grid, block, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, typename CK>
static hipError_t launch_replay_tc(const ScanArgs &a, hipStream_t s) {
    return a.y ? launch_replay_tcy<T, CK, true>(a, s) : launch_replay_tcy<T, CK, false>(a, s);
}

template <typename T, typename CK>
static hipError_t launch_scan_tc(const ScanArgs &a, hipStream_t s) {
    // the state (and y) alone, x in whole 16-byte pieces per thread: the replay kernel
    const bool plain = a.live == nullptr && a.snap == nullptr && a.chunk_states == nullptr;
    const bool xvec = (reinterpret_cast<uintptr_t>(a.x) % 16) == 0 && (a.P % kReplayRows) == 0;
    if (plain && xvec) return launch_replay_tc<T, CK>(a, s);
    return a.live ? launch_scan_tcl<T, CK, true>(a, s) : launch_scan_tcl<T, CK, false>(a, s);
}

hipError_t launch_scan(const ScanArgs &a, bool bf16, bool ckpt_f16, hipStream_t s) {
    if (bf16) return ckpt_f16 ? launch_scan_tc<bf16_t, uint16_t>(a, s) : launch_scan_tc<bf16_t, float>(a, s);
    return ckpt_f16 ? launch_scan_tc<float, uint16_t>(a, s) : launch_scan_tc<float, float>(a, s);
}

hipError_t launch_drift_reduce(const float *pm, const float *ps, int64_t nwaves, int64_t r,
                               double inv_count, float *dmax, float *dmean, hipStream_t s) {
    const unsigned blocks = static_cast<unsigned>((r + 255) / 256);
    drift_reduce_kernel<<<blocks, 256, 0, s>>>(pm, ps, nwaves, r, inv_count, dmax, dmean);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_scan_bwd_t(const ScanBwdArgs &a, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(a.Bsz * a.H)), block(256);
    switch (a.N) {
        case 16: scan_bwd_kernel<16, 8, T><<<grid, block, 0, s>>>(a); break;
        case 32: scan_bwd_kernel<32, 8, T><<<grid, block, 0, s>>>(a); break;
        case 64: scan_bwd_kernel<64, 8, T><<<grid, block, 0, s>>>(a); break;
        case 128: scan_bwd_kernel<128, 8, T><<<grid, block, 0, s>>>(a); break;
        case 256: scan_bwd_kernel<256, 8, T><<<grid, block, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t total = a.Bsz * a.T * a.G * a.N;
    group_sum_kernel<<<static_cast<unsigned>((total + 255) / 256), 256, 0, s>>>(
        a.dB_part, a.dC_part, a.dB, a.dC, a.Bsz * a.T, a.H, a.G, a.N);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    head_param_sum_kernel<<<static_cast<unsigned>((a.H + 255) / 256), 256, 0, s>>>(
        a.dA_part, a.dD_part, a.dA, a.dD, a.Bsz, a.H);
    return hipGetLastError();
}

hipError_t launch_scan_bwd(const ScanBwdArgs &a, bool bf16, hipStream_t s) {
    return bf16 ? launch_scan_bwd_t<bf16_t>(a, s) : launch_scan_bwd_t<float>(a, s);
}

}  // namespace ssm
