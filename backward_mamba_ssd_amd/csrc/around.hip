// around.hip -- the stages on either side of the scan in a Mamba-2 layer:
//   * the short causal depthwise convolution followed by SiLU (before the scan)
//   * the SiLU-gated group RMSNorm (after the scan)
// with their backward passes.  "Nemotron Kernels: From Inference To
// Backpropagation", Kernel 1 "Forward And Inference" (the pipeline causal
// Conv1D + SiLU -> selective scan -> gated group RMSNorm), section "What Conv1D
// Gives The Mamba Block" (each output gradient reaches the inputs of its window,
// the weights and the bias; overlapping windows add at one input; the SiLU
// derivative comes first) and section "From Classical State Space To A Selective
// Mamba State" (the SiLU gate).
//
// Convolution, per batch b and channel c, K taps, with the K-1 samples before
// token 0 taken from init (zero when absent):
//   ext[j] = init[j] (j < K-1), ext[K-1+t] = u[t]
//   v[t]   = bias[c] + sum_k w[c][k] ext[t+k],   out[t] = v[t] sigmoid(v[t])
// Backward: dv = dout SiLU'(v); du[t] = sum_k w[c][k] dv[t+K-1-k];
//   dw[c][k] = sum_t dv[t] ext[t+k]; dbias[c] = sum_t dv[t];
//   dinit[j] = sum_{k<=j} w[c][k] dv[j-k].
// Gated group RMSNorm over groups of S = C/G consecutive channels:
//   g = y SiLU(z), r = 1/sqrt(mean_group(g^2) + eps), out = g r w[c]
// Backward: n = g r, dn = dout w, dg = r (dn - n mean_group(dn n)),
//   dy = dg SiLU(z), dz = dg y SiLU'(z), dw[c] = sum_rows dout n.
//
// All four kernels are HBM-bound streams.  Each thread owns 4 (convolution) or 8
// (normalisation) consecutive channels, so a wave touches 512 B - 1 KB of one row
// per access.  The parameter gradients are summed deterministically: fp64
// partials per token/row tile, then a second pass adds them in tile order.
#include "common.hpp"
#include "launch.hpp"

namespace ssm {
namespace {

// sigmoid from the hardware exp2 and reciprocal (about 1 ulp each); these
// kernels stream memory, and the library expf and IEEE division would make the
// activation's instruction count, not the bytes, their bound.
__device__ __forceinline__ float sigm(float v) {
    const float e = __expf(-fabsf(v));
    const float s = __builtin_amdgcn_rcpf(1.f + e);
    return v >= 0.f ? s : e * s;
}
__device__ __forceinline__ float silu(float v) { return v * sigm(v); }
__device__ __forceinline__ float silu_grad(float v) {
    const float s = sigm(v);
    return s * (1.f + v * (1.f - s));
}

// 4 consecutive channels of a storage-dtype row as floats, and back
template <typename T> __device__ __forceinline__ float4 ld4(const T *p) { return IO<T>::ld4(p, 0); }
template <typename T> __device__ __forceinline__ void st4(T *p, float4 v);
template <> __device__ __forceinline__ void st4<float>(float *p, float4 v) { *reinterpret_cast<float4 *>(p) = v; }
template <> __device__ __forceinline__ void st4<bf16_t>(bf16_t *p, float4 v) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 w = {pack2_bf16(v.x, v.y), pack2_bf16(v.z, v.w)};
    *reinterpret_cast<u32x2 *>(p) = w;
}

__device__ __forceinline__ float get(const float4 &v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

constexpr int kConvFwdTile = 64;   // tokens per forward thread (window halo K-1)
constexpr int kConvUnroll = 8;     // forward: tokens whose loads are in flight together

// ---------------------------------------------------------------------------
// convolution + SiLU, forward: thread = (batch, 4 channels, token tile)
// ---------------------------------------------------------------------------
template <typename T, int K>
__global__ void __launch_bounds__(256) conv_fwd_kernel(ConvArgs a) {
    const int64_t c0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (c0 >= a.C) return;
    const int64_t b = blockIdx.z;
    const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kConvFwdTile;
    const T *u = static_cast<const T *>(a.u);
    const T *init = static_cast<const T *>(a.init);
    T *out = static_cast<T *>(a.out);
    float4 w[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
        w[k] = make_float4(a.w[(c0 + 0) * K + k], a.w[(c0 + 1) * K + k], a.w[(c0 + 2) * K + k], a.w[(c0 + 3) * K + k]);
    const float4 bias = *reinterpret_cast<const float4 *>(a.bias + c0);
    // ext sample m (m = K-1+t) for t in [t0-K+1, t0): from u, or from init before token 0
    auto sample = [&](int64_t t) -> float4 {
        if (t >= 0) return ld4(u + (b * a.T + t) * a.C + c0);
        if (init != nullptr) return ld4(init + (b * (K - 1) + (K - 1 + t)) * a.C + c0);
        return make_float4(0.f, 0.f, 0.f, 0.f);
    };
    float4 win[K > 1 ? K - 1 : 1];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) win[j] = sample(t0 - (K - 1) + j);
    const int64_t tend = (t0 + kConvFwdTile < a.T) ? t0 + kConvFwdTile : a.T;
    // kConvUnroll tokens at a time: all their loads are issued before the first use
    for (int64_t tb = t0; tb < tend; tb += kConvUnroll) {
        float4 xs[kConvUnroll];
#pragma unroll
        for (int q = 0; q < kConvUnroll; ++q)
            xs[q] = (tb + q < tend) ? ld4(u + (b * a.T + tb + q) * a.C + c0) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int q = 0; q < kConvUnroll; ++q) {
            if (tb + q >= tend) break;  // uniform across the workgroup
            const float4 xv = xs[q];
            float4 v = bias;
#pragma unroll
            for (int k = 0; k < K - 1; ++k) {
                v.x = fmaf(w[k].x, win[k].x, v.x);
                v.y = fmaf(w[k].y, win[k].y, v.y);
                v.z = fmaf(w[k].z, win[k].z, v.z);
                v.w = fmaf(w[k].w, win[k].w, v.w);
            }
            v.x = fmaf(w[K - 1].x, xv.x, v.x);
            v.y = fmaf(w[K - 1].y, xv.y, v.y);
            v.z = fmaf(w[K - 1].z, xv.z, v.z);
            v.w = fmaf(w[K - 1].w, xv.w, v.w);
            st4(out + (b * a.T + tb + q) * a.C + c0, make_float4(silu(v.x), silu(v.y), silu(v.z), silu(v.w)));
#pragma unroll
            for (int j = 0; j + 1 < K - 1; ++j) win[j] = win[j + 1];
            if (K > 1) win[K > 1 ? K - 2 : 0] = xv;
        }
    }
    // the samples the next call needs: ext[T .. T+K-2] (the tile holding the last token,
    // or tile 0 when there are no tokens)
    if (a.final_state != nullptr && ((t0 < a.T && tend == a.T) || (a.T == 0 && t0 == 0))) {
        T *fin = static_cast<T *>(a.final_state);
#pragma unroll
        for (int j = 0; j < K - 1; ++j) st4(fin + (b * (K - 1) + j) * a.C + c0, win[j]);
    }
}

// ---------------------------------------------------------------------------
// convolution + SiLU, backward.  Workgroup = 64 channels x 256 tokens of one
// sequence: thread (4 channels, 16-token sub-tile), so a wave reads 4 tokens x
// 128 contiguous bytes per access and each thread's loop is short.  A sub-tile's
// dv are recomputed with a K-1 token look-ahead so every du of it is complete.
// A thread sums its 16 tokens' weight/bias terms in float32; the 16 sub-tile sums
// are added in fp64 in LDS in sub-tile order and written as one partial per
// (sequence, 256-token tile).
// ---------------------------------------------------------------------------
constexpr int kConvSub = 16;                       // tokens per thread
constexpr int kConvSubs = kConvBwdTile / kConvSub;  // sub-tiles per workgroup (16)

template <typename T, int K>
__global__ void __launch_bounds__(256) conv_bwd_kernel(ConvArgs a) {
    __shared__ double red[kConvSubs][K + 1][64];
    const int cg = threadIdx.x & 15, sub = threadIdx.x >> 4;
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * 64 + cg * 4;
    const bool cvalid = c0 < a.C;
    const int64_t b = blockIdx.z;
    const int64_t tile = blockIdx.y;
    const int64_t t0 = tile * kConvBwdTile + sub * kConvSub;
    const T *u = static_cast<const T *>(a.u);
    const T *init = static_cast<const T *>(a.init);
    const T *dout = static_cast<const T *>(a.dout);
    T *du = static_cast<T *>(a.du);
    float pw[K][4], pb[4];  // float32 over the 16 tokens of the sub-tile, fp64 beyond
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        pb[i] = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) pw[k][i] = 0.f;
    }
    if (cvalid && t0 < a.T) {
        float4 w[K];
#pragma unroll
        for (int k = 0; k < K; ++k)
            w[k] = make_float4(a.w[(c0 + 0) * K + k], a.w[(c0 + 1) * K + k], a.w[(c0 + 2) * K + k], a.w[(c0 + 3) * K + k]);
        const float4 bias = *reinterpret_cast<const float4 *>(a.bias + c0);
        auto sample = [&](int64_t t) -> float4 {
            if (t >= 0) return ld4(u + (b * a.T + t) * a.C + c0);
            if (init != nullptr) return ld4(init + (b * (K - 1) + (K - 1 + t)) * a.C + c0);
            return make_float4(0.f, 0.f, 0.f, 0.f);
        };
        float4 win[K > 1 ? K - 1 : 1];
#pragma unroll
        for (int j = 0; j < K - 1; ++j) win[j] = sample(t0 - (K - 1) + j);
        float4 ring[K];  // ring[j] = dv[m - (K-1) + j] after step m
#pragma unroll
        for (int j = 0; j < K; ++j) ring[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        float4 first[K > 1 ? K - 1 : 1];  // dv[0 .. K-2] (the sub-tile at token 0, for dinit)
#pragma unroll
        for (int j = 0; j < K - 1; ++j) first[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        const int64_t tend = (t0 + kConvSub < a.T) ? t0 + kConvSub : a.T;
        for (int64_t m = t0; m < tend + K - 1; ++m) {
            float4 dv = make_float4(0.f, 0.f, 0.f, 0.f);
            if (m < a.T) {
                const float4 xv = ld4(u + (b * a.T + m) * a.C + c0);
                const float4 go = ld4(dout + (b * a.T + m) * a.C + c0);
                float4 v = bias;
#pragma unroll
                for (int k = 0; k < K - 1; ++k) {
                    v.x = fmaf(w[k].x, win[k].x, v.x);
                    v.y = fmaf(w[k].y, win[k].y, v.y);
                    v.z = fmaf(w[k].z, win[k].z, v.z);
                    v.w = fmaf(w[k].w, win[k].w, v.w);
                }
                v.x = fmaf(w[K - 1].x, xv.x, v.x);
                v.y = fmaf(w[K - 1].y, xv.y, v.y);
                v.z = fmaf(w[K - 1].z, xv.z, v.z);
                v.w = fmaf(w[K - 1].w, xv.w, v.w);
                dv = make_float4(go.x * silu_grad(v.x), go.y * silu_grad(v.y), go.z * silu_grad(v.z), go.w * silu_grad(v.w));
                if (m < tend) {  // the sub-tile's own token: parameter partials
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float d = get(dv, i);
                        pb[i] += d;
#pragma unroll
                        for (int k = 0; k < K - 1; ++k) pw[k][i] = fmaf(d, get(win[k], i), pw[k][i]);
                        pw[K - 1][i] = fmaf(d, get(xv, i), pw[K - 1][i]);
                    }
                }
#pragma unroll
                for (int j = 0; j + 1 < K - 1; ++j) win[j] = win[j + 1];
                if (K > 1) win[K > 1 ? K - 2 : 0] = xv;
            }
            if (t0 == 0 && m < K - 1) {
#pragma unroll
                for (int j = 0; j < K - 1; ++j)
                    if (j == m) first[j] = dv;
            }
#pragma unroll
            for (int j = 0; j + 1 < K; ++j) ring[j] = ring[j + 1];
            ring[K - 1] = dv;
            const int64_t t = m - (K - 1);  // du[t] = sum_j w[K-1-j] dv[t+j] is complete
            if (t >= t0 && t < tend) {
                float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    g.x = fmaf(w[K - 1 - j].x, ring[j].x, g.x);
                    g.y = fmaf(w[K - 1 - j].y, ring[j].y, g.y);
                    g.z = fmaf(w[K - 1 - j].z, ring[j].z, g.z);
                    g.w = fmaf(w[K - 1 - j].w, ring[j].w, g.w);
                }
                st4(du + (b * a.T + t) * a.C + c0, g);
            }
        }
        if (t0 == 0 && a.dinit != nullptr) {
            T *dinit = static_cast<T *>(a.dinit);
#pragma unroll
            for (int j = 0; j < K - 1; ++j) {
                float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int k = 0; k <= j; ++k) {
                    g.x = fmaf(w[k].x, first[j - k].x, g.x);
                    g.y = fmaf(w[k].y, first[j - k].y, g.y);
                    g.z = fmaf(w[k].z, first[j - k].z, g.z);
                    g.w = fmaf(w[k].w, first[j - k].w, g.w);
                }
                st4(dinit + (b * (K - 1) + j) * a.C + c0, g);
            }
        }
    }
    // sub-tile partials meet in LDS; the tile's partial is their sum in sub-tile order
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int k = 0; k < K; ++k) red[sub][k][cg * 4 + i] = static_cast<double>(pw[k][i]);
        red[sub][K][cg * 4 + i] = static_cast<double>(pb[i]);
    }
    __syncthreads();
    // partials [b * ntiles + tile][K + 1][C]: K weight taps, then the bias
    const int64_t pi = (b * a.ntiles + tile) * (K + 1);
    for (int e = threadIdx.x; e < (K + 1) * 64; e += 256) {
        const int k = e / 64, cc = e % 64;
        const int64_t c = static_cast<int64_t>(blockIdx.x) * 64 + cc;
        if (c >= a.C) continue;
        double acc = 0.0;
        for (int sb = 0; sb < kConvSubs; ++sb) acc += red[sb][k][cc];
        a.part[(pi + k) * a.C + c] = acc;
    }
}

// dw[c][k], dbias[c]: thread per (c, tap) adds the partials of all tiles in order
__global__ void __launch_bounds__(256) conv_param_sum_kernel(ConvArgs a) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t n = a.C * (a.K + 1);
    if (i >= n) return;
    const int64_t k = i / a.C, c = i % a.C;
    const int64_t tiles = a.Bsz * a.ntiles;
    double s = 0.0;
    for (int64_t t = 0; t < tiles; ++t) s += a.part[(t * (a.K + 1) + k) * a.C + c];
    if (k < a.K) a.dw[c * a.K + k] = static_cast<float>(s);
    else a.dbias[c] = static_cast<float>(s);
}

// ---------------------------------------------------------------------------
// gated group RMSNorm: a 256-thread workgroup per (row, group) (forward) or per
// (row tile, group) (backward); thread j holds channels 8*(j + 256*q), q < NQ
// ---------------------------------------------------------------------------

template <typename T> __device__ __forceinline__ void ld8(const T *p, float *v);
template <> __device__ __forceinline__ void ld8<float>(const float *p, float *v) {
    const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <> __device__ __forceinline__ void ld8<bf16_t>(const bf16_t *p, float *v) {
    const u16x8 r = *reinterpret_cast<const u16x8 *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = bf16_to_f32(r[i]);
}
template <typename T> __device__ __forceinline__ void st8(T *p, const float *v);
template <> __device__ __forceinline__ void st8<float>(float *p, const float *v) {
    *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
template <> __device__ __forceinline__ void st8<bf16_t>(bf16_t *p, const float *v) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w = {pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]), pack2_bf16(v[4], v[5]), pack2_bf16(v[6], v[7])};
    *reinterpret_cast<u32x4 *>(p) = w;
}

// sum over the workgroup's 256 threads, the same fixed order everywhere
__device__ __forceinline__ float block_sum(float v, float *red) {
    v = wave_total(v);
    const int wave = threadIdx.x >> 6;
    __syncthreads();  // red is free (its previous use has been read)
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

template <typename T, int NQ>
__global__ void __launch_bounds__(256) norm_fwd_kernel(NormArgs a) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x, grp = blockIdx.y;
    const int64_t S = a.C / a.G;
    const int64_t base = row * a.C + grp * S;
    const T *y = static_cast<const T *>(a.y);
    const T *z = static_cast<const T *>(a.z);
    float g[NQ][8];
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int64_t i = 8 * (threadIdx.x + 256 * q);
        if (i < S) {
            float yv[8], zv[8];
            ld8(y + base + i, yv);
            ld8(z + base + i, zv);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                g[q][e] = yv[e] * silu(zv[e]);
                ss = fmaf(g[q][e], g[q][e], ss);
            }
        }
    }
    const float r = rsqrtf(block_sum(ss, red) / static_cast<float>(S) + a.eps);
    T *out = static_cast<T *>(a.out);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int64_t i = 8 * (threadIdx.x + 256 * q);
        if (i < S) {
            float o[8];
            const float *wp = a.w + grp * S + i;
            const float4 w0 = *reinterpret_cast<const float4 *>(wp), w1 = *reinterpret_cast<const float4 *>(wp + 4);
            const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = g[q][e] * r * wv[e];
            st8(out + base + i, o);
        }
    }
}

template <typename T, int NQ>
__global__ void __launch_bounds__(256) norm_bwd_kernel(NormArgs a) {
    __shared__ float red[4];
    const int64_t rt = blockIdx.x, grp = blockIdx.y;
    const int64_t S = a.C / a.G;
    const T *y = static_cast<const T *>(a.y);
    const T *z = static_cast<const T *>(a.z);
    const T *dout = static_cast<const T *>(a.dout);
    T *dy = static_cast<T *>(a.dy);
    T *dz = static_cast<T *>(a.dz);
    float pw[NQ][8];  // float32 over the tile's rows, fp64 across tiles
    float wv[NQ][8];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int64_t i = 8 * (threadIdx.x + 256 * q);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pw[q][e] = 0.f;
            wv[q][e] = (i < S) ? a.w[grp * S + i + e] : 0.f;
        }
    }
    const int64_t r0 = rt * kNormRows;
    const int64_t r1 = (r0 + kNormRows < a.rows) ? r0 + kNormRows : a.rows;
    // Rows alternate between two register sets so the next row's loads are in flight
    // while the current row is reduced (a copy of a loaded register would wait for it).
    struct Row {
        float y[NQ][8], z[NQ][8], g[NQ][8];
    };
    auto load = [&](Row &R, int64_t row) {
        const int64_t base = row * a.C + grp * S;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int64_t i = 8 * (threadIdx.x + 256 * q);
            if (i < S) {
                ld8(y + base + i, R.y[q]);
                ld8(z + base + i, R.z[q]);
                ld8(dout + base + i, R.g[q]);
            }
        }
    };
    auto process = [&](const Row &R, int64_t row) {
        const int64_t base = row * a.C + grp * S;
        float sg[NQ][8], gg[NQ][8];  // sigmoid(z) and the gated value g = y SiLU(z)
        float ss = 0.f;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int64_t i = 8 * (threadIdx.x + 256 * q);
            if (i < S) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sg[q][e] = sigm(R.z[q][e]);
                    gg[q][e] = R.y[q][e] * (R.z[q][e] * sg[q][e]);
                    ss = fmaf(gg[q][e], gg[q][e], ss);
                }
            }
        }
        const float r = rsqrtf(block_sum(ss, red) / static_cast<float>(S) + a.eps);
        float dn_n = 0.f;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int64_t i = 8 * (threadIdx.x + 256 * q);
            if (i < S) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float n = gg[q][e] * r;
                    dn_n = fmaf(R.g[q][e] * wv[q][e], n, dn_n);
                    pw[q][e] = fmaf(R.g[q][e], n, pw[q][e]);
                }
            }
        }
        const float m = block_sum(dn_n, red) / static_cast<float>(S);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int64_t i = 8 * (threadIdx.x + 256 * q);
            if (i < S) {
                float oy[8], oz[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float zv = R.z[q][e], sv = sg[q][e];
                    const float n = gg[q][e] * r;
                    const float dg = r * (R.g[q][e] * wv[q][e] - n * m);
                    oy[e] = dg * (zv * sv);
                    oz[e] = dg * R.y[q][e] * (sv * (1.f + zv * (1.f - sv)));
                }
                st8(dy + base + i, oy);
                st8(dz + base + i, oz);
            }
        }
    };
    Row RA, RB;
    if (r0 < r1) load(RA, r0);
    for (int64_t row = r0; row < r1; row += 2) {
        if (row + 1 < r1) load(RB, row + 1);
        process(RA, row);
        if (row + 1 < r1) {
            if (row + 2 < r1) load(RA, row + 2);
            process(RB, row + 1);
        }
    }
    // partials [row tile][C]
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int64_t i = 8 * (threadIdx.x + 256 * q);
        if (i < S)
#pragma unroll
            for (int e = 0; e < 8; ++e) a.part[rt * a.C + grp * S + i + e] = static_cast<double>(pw[q][e]);
    }
}

// dw[c]: 64 channels per workgroup, four waves each adding every fourth tile's
// partial (tiles ascending), then the four wave sums in wave order
__global__ void __launch_bounds__(256) norm_param_sum_kernel(NormArgs a, int64_t ntiles) {
    __shared__ double red[4][64];
    const int cl = threadIdx.x & 63, qt = threadIdx.x >> 6;
    const int64_t c = static_cast<int64_t>(blockIdx.x) * 64 + cl;
    double s = 0.0;
    if (c < a.C) {
#pragma unroll 8
        for (int64_t t = qt; t < ntiles; t += 4) s += a.part[t * a.C + c];
    }
    red[qt][cl] = s;
    __syncthreads();
    if (qt == 0 && c < a.C) a.dw[c] = static_cast<float>(((red[0][cl] + red[1][cl]) + red[2][cl]) + red[3][cl]);
}

template <typename T, int K>
hipError_t conv_launch(const ConvArgs &a, bool bwd, hipStream_t s) {
    const unsigned cx = static_cast<unsigned>((a.C / 4 + 255) / 256);
    if (!bwd) {
        const int64_t nt = (a.T + kConvFwdTile - 1) / kConvFwdTile;
        conv_fwd_kernel<T, K><<<dim3(cx, static_cast<unsigned>(nt > 0 ? nt : 1), static_cast<unsigned>(a.Bsz)), 256, 0, s>>>(a);
        return hipGetLastError();
    }
    if (a.ntiles > 0) {
        const unsigned cb = static_cast<unsigned>((a.C + 63) / 64);
        conv_bwd_kernel<T, K><<<dim3(cb, static_cast<unsigned>(a.ntiles), static_cast<unsigned>(a.Bsz)), 256, 0, s>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    conv_param_sum_kernel<<<static_cast<unsigned>((a.C * (K + 1) + 255) / 256), 256, 0, s>>>(a);
    return hipGetLastError();
}

template <typename T>
hipError_t conv_dispatch(const ConvArgs &a, bool bwd, hipStream_t s) {
    switch (a.K) {
        case 1: return conv_launch<T, 1>(a, bwd, s);
        case 2: return conv_launch<T, 2>(a, bwd, s);
        case 3: return conv_launch<T, 3>(a, bwd, s);
        case 4: return conv_launch<T, 4>(a, bwd, s);
        case 5: return conv_launch<T, 5>(a, bwd, s);
        case 6: return conv_launch<T, 6>(a, bwd, s);
        case 7: return conv_launch<T, 7>(a, bwd, s);
        case 8: return conv_launch<T, 8>(a, bwd, s);
    }
    return hipErrorInvalidValue;
}

template <typename T, int NQ>
hipError_t norm_launch(const NormArgs &a, bool bwd, hipStream_t s) {
    if (!bwd) {
        norm_fwd_kernel<T, NQ><<<dim3(static_cast<unsigned>(a.rows), static_cast<unsigned>(a.G)), 256, 0, s>>>(a);
        return hipGetLastError();
    }
    const int64_t nt = norm_row_tiles(a.rows);
    if (nt > 0) {
        norm_bwd_kernel<T, NQ><<<dim3(static_cast<unsigned>(nt), static_cast<unsigned>(a.G)), 256, 0, s>>>(a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    norm_param_sum_kernel<<<static_cast<unsigned>((a.C + 63) / 64), 256, 0, s>>>(a, nt);
    return hipGetLastError();
}

template <typename T>
hipError_t norm_dispatch(const NormArgs &a, bool bwd, hipStream_t s) {
    const int64_t q = (a.C / a.G + 2047) / 2048;
    switch (q) {
        case 1: return norm_launch<T, 1>(a, bwd, s);
        case 2: return norm_launch<T, 2>(a, bwd, s);
        case 3: return norm_launch<T, 3>(a, bwd, s);
        case 4: return norm_launch<T, 4>(a, bwd, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace


hipError_t launch_conv(const ConvArgs &a, bool bf16, bool bwd, hipStream_t s) {
    if (a.Bsz == 0 || a.C == 0) return hipSuccess;
    return bf16 ? conv_dispatch<bf16_t>(a, bwd, s) : conv_dispatch<float>(a, bwd, s);
}

hipError_t launch_norm(const NormArgs &a, bool bf16, bool bwd, hipStream_t s) {
    if (a.C == 0) return hipSuccess;
    if (!bwd && a.rows == 0) return hipSuccess;
    return bf16 ? norm_dispatch<bf16_t>(a, bwd, s) : norm_dispatch<float>(a, bwd, s);
}

}  // namespace ssm
