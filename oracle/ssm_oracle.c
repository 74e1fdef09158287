/*
 * ssm_oracle.c -- plain, slow, sequential fp64 CPU reference for the Mamba-2
 * selective state-space recurrence.  TEST INFRASTRUCTURE ONLY: the tests, the
 * smoke check and the CPU-baseline leg of the benchmark load this file's
 * library; the GPU product path never does.  It shares no code, header or
 * constant with the HIP library.
 *
 * What is computed (per batch b, head h, group g = h / (H/G)):
 *
 *   a_t      = exp(dt[b,t,h] * A[h])
 *   s[p][n]  = a_t * s[p][n] + x[b,t,h,p] * (B[b,t,g,n] * dt[b,t,h])
 *   y[b,t,h,p] = sum_n C[b,t,g,n] * s[p][n] + D[h] * x[b,t,h,p]
 *
 * Sources (read as data, restated here in my own words):
 *  - "Nemotron 3 Ultra: replaying a rounded state" (TorchLean Verified
 *    Examples), section "The Mamba state update": the per-coordinate update
 *    of theorem updateHead_apply -- old state times the retention exp(dt*A),
 *    plus value[p] times (B of the head's group [n] times dt); A is a
 *    per-head scalar and B is selected by the head's group.
 *  - same page, section "Recovering the state by replay": the worked SSM.step
 *    example reads the output from the UPDATED state (state 10, write 2,
 *    output 12), so y_t reads s_t, not s_{t-1}.
 *  - "Nemotron Kernels: From Inference To Backpropagation" (shivasnotes),
 *    Kernel 1 "Backpropagation: What Mamba2 Backward Must Do": the reverse
 *    walk goes from the last token to the first; the gradient reaching a state
 *    is the sum of the output path and the future recurrent path; B and C of a
 *    group receive the sum over every head and channel of that group.
 *  - same page, Part I "Branches Copy Forward And Add Backward": where a
 *    forward value is used twice, the reverse contributions are added (dt is
 *    used by the retention and by the write; x by the write and by the D skip).
 *  - "Reverse-mode automatic differentiation" (OneModel docs), section 4
 *    "Arithmetic": sums over many elements are accumulated in double in a
 *    fixed increasing order -- the oracle does every sum in fp64 in a fixed
 *    order (token descending in the reverse sweep, heads ascending, p then n
 *    ascending).
 *
 * Every input, intermediate and output is double (bf16/fp32 inputs are widened
 * exactly by the caller).  No blocking, chunking or
 * reordering of the recurrence: the backward keeps per-token states of one
 * segment at a time and re-derives them from a stored segment-start state by
 * re-running the same forward steps (memory management only; the values are
 * those of the one sequential forward pass, bit for bit).
 *
 * SR16 section: the fp16 stochastic-rounding rule of the same TorchLean page,
 * section "Stochastic rounding and the mean state" (round to the upper grid
 * value when the entropy residue is below the discarded remainder), with the
 * entropy drawn from a counter-based hash built on SplitMix64 (Steele, Lea &
 * Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX4(a, b, c, d, B_, C_, D_) ((((int64_t)(a) * (B_) + (b)) * (C_) + (c)) * (D_) + (d))

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One forward token step on a [P][N] double state (the updateHead_apply
 * coordinate formula), then the read of the updated state. */
static void step_token(double *s, int64_t P, int64_t N, double a, double dtv,
                       const double *xp, const double *Bn, const double *Cn,
                       double Dh, double *y_out /* P values, may be NULL */) {
    for (int64_t p = 0; p < P; ++p) {
        double xv = xp[p];
        double *row = s + p * N;
        for (int64_t n = 0; n < N; ++n)
            row[n] = a * row[n] + xv * (Bn[n] * dtv);
    }
    if (y_out) {
        for (int64_t p = 0; p < P; ++p) {
            const double *row = s + p * N;
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) acc += Cn[n] * row[n];
            y_out[p] = acc + Dh * xp[p];
        }
    }
}

/*
 * Sequential forward.  Shapes (all contiguous):
 *   x [Bsz,T,H,P]  Bm,Cm [Bsz,T,G,N]  dt [Bsz,T,H]  A,D [H]
 *   h0 [Bsz,H,P,N] or NULL (zero initial state)
 *   y [Bsz,T,H,P]  h_final [Bsz,H,P,N] or NULL
 *   chunk_states [Bsz,H,nc,P,N] or NULL, nc = ceil(T/L): entry c is the state
 *   entering chunk c, i.e. before token c*L (entry 0 is the initial state).
 */
void oracle_fwd(int64_t Bsz, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G,
                int64_t L, const double *x, const double *Bm, const double *Cm,
                const double *dt, const double *A, const double *D, const double *h0,
                double *y, double *h_final, double *chunk_states) {
    const int64_t hpg = H / G;
    const int64_t nc = (T + L - 1) / L;
    const int64_t PN = P * N;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < Bsz * H; ++bh) {
        const int64_t b = bh / H, h = bh % H, g = h / hpg;
        double *s = (double *)malloc(sizeof(double) * PN);
        if (h0) memcpy(s, h0 + bh * PN, sizeof(double) * PN);
        else memset(s, 0, sizeof(double) * PN);
        double ybuf[1024];
        double *yb = P <= 1024 ? ybuf : (double *)malloc(sizeof(double) * P);
        for (int64_t t = 0; t < T; ++t) {
            if (chunk_states && t % L == 0)
                memcpy(chunk_states + (bh * nc + t / L) * PN, s, sizeof(double) * PN);
            const double dtv = dt[(b * T + t) * H + h];
            const double a = exp(dtv * A[h]);
            step_token(s, P, N, a, dtv, x + IDX4(b, t, h, 0, T, H, P),
                       Bm + IDX4(b, t, g, 0, T, G, N), Cm + IDX4(b, t, g, 0, T, G, N),
                       D[h], yb);
            memcpy(y + IDX4(b, t, h, 0, T, H, P), yb, sizeof(double) * P);
        }
        if (h_final) memcpy(h_final + bh * PN, s, sizeof(double) * PN);
        if (yb != ybuf) free(yb);
        free(s);
    }
}

/*
 * Reverse sweep.  Given the forward inputs, the upstream dy [Bsz,T,H,P] and
 * optionally dh_final [Bsz,H,P,N] (gradient on the final state), writes
 *   dx [Bsz,T,H,P], dB, dC [Bsz,T,G,N] (summed over the heads of the group),
 *   ddt [Bsz,T,H] (w.r.t. the post-softplus dt input), dA, dD [H] (summed over
 *   batch and tokens), dh0 [Bsz,H,P,N] or NULL.
 *
 * Loss convention: L = sum dy*y + sum dh_final*h_T.  With gs the gradient on
 * the state after token t (gs = dL/ds_t), walking t = T-1 .. 0:
 *   gs     += dy_t (outer) C_t              (output path meets future path)
 *   dC_t[n] = sum_p dy_t[p] * s_t[p][n]
 *   dx_t[p] = D*dy_t[p] + dt * sum_n gs[p][n] * B_t[n]
 *   dB_t[n] = dt * sum_p gs[p][n] * x_t[p]
 *   ddt_t   = sum_{p,n} gs*x_t[p]*B_t[n]    (write branch)
 *           + (sum_{p,n} gs*s_{t-1}) * a_t * A   (retention branch)
 *   dA     += (sum_{p,n} gs*s_{t-1}) * a_t * dt
 *   dD     += sum_p dy_t[p] * x_t[p]
 *   gs      = a_t * gs                      (carry to s_{t-1})
 * and dh0 = gs at the end.
 */
void oracle_bwd(int64_t Bsz, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G,
                const double *x, const double *Bm, const double *Cm, const double *dt,
                const double *A, const double *D, const double *h0, const double *dy,
                const double *dh_final, double *dx, double *dB, double *dC, double *ddt,
                double *dA, double *dD, double *dh0) {
    const int64_t hpg = H / G;
    const int64_t PN = P * N;
    const int64_t SEG = 256; /* states kept per segment (memory only) */
    const int64_t nseg = (T + SEG - 1) / SEG;
    double *dA_part = (double *)calloc((size_t)(Bsz * H), sizeof(double));
    double *dD_part = (double *)calloc((size_t)(Bsz * H), sizeof(double));
    /* dB, dC are accumulated in place: zero them first. */
    memset(dB, 0, sizeof(double) * (size_t)(Bsz * T * G * N));
    memset(dC, 0, sizeof(double) * (size_t)(Bsz * T * G * N));
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bg = 0; bg < Bsz * G; ++bg) {
        const int64_t b = bg / G, g = bg % G;
        double *seg_start = (double *)malloc(sizeof(double) * PN * nseg);
        double *states = (double *)malloc(sizeof(double) * PN * (SEG + 1));
        double *gs = (double *)malloc(sizeof(double) * PN);
        for (int64_t hh = 0; hh < hpg; ++hh) {
            const int64_t h = g * hpg + hh;
            const int64_t bh = b * H + h;
            const double Ah = A[h], Dh = D[h];
            /* forward pass: remember the state entering every segment */
            double *s = states;
            if (h0) memcpy(s, h0 + bh * PN, sizeof(double) * PN);
            else memset(s, 0, sizeof(double) * PN);
            for (int64_t t = 0; t < T; ++t) {
                if (t % SEG == 0) memcpy(seg_start + (t / SEG) * PN, s, sizeof(double) * PN);
                const double dtv = dt[(b * T + t) * H + h];
                step_token(s, P, N, exp(dtv * Ah), dtv, x + IDX4(b, t, h, 0, T, H, P),
                           Bm + IDX4(b, t, g, 0, T, G, N), Cm + IDX4(b, t, g, 0, T, G, N),
                           Dh, NULL);
            }
            /* reverse sweep */
            if (dh_final) memcpy(gs, dh_final + bh * PN, sizeof(double) * PN);
            else memset(gs, 0, sizeof(double) * PN);
            double dA_acc = 0.0, dD_acc = 0.0;
            for (int64_t sg = nseg - 1; sg >= 0; --sg) {
                const int64_t t0 = sg * SEG;
                const int64_t t1 = (t0 + SEG < T) ? t0 + SEG : T;
                /* states[k] = state after token t0+k-1 (states[0] = entering) */
                memcpy(states, seg_start + sg * PN, sizeof(double) * PN);
                for (int64_t t = t0; t < t1; ++t) {
                    double *nx = states + (t - t0 + 1) * PN;
                    memcpy(nx, states + (t - t0) * PN, sizeof(double) * PN);
                    const double dtv = dt[(b * T + t) * H + h];
                    step_token(nx, P, N, exp(dtv * Ah), dtv, x + IDX4(b, t, h, 0, T, H, P),
                               Bm + IDX4(b, t, g, 0, T, G, N),
                               Cm + IDX4(b, t, g, 0, T, G, N), Dh, NULL);
                }
                for (int64_t t = t1 - 1; t >= t0; --t) {
                    const double *s_t = states + (t - t0 + 1) * PN;
                    const double *s_prev = states + (t - t0) * PN;
                    const double *xt = x + IDX4(b, t, h, 0, T, H, P);
                    const double *dyt = dy + IDX4(b, t, h, 0, T, H, P);
                    const double *Bt = Bm + IDX4(b, t, g, 0, T, G, N);
                    const double *Ct = Cm + IDX4(b, t, g, 0, T, G, N);
                    const double dtv = dt[(b * T + t) * H + h];
                    const double a = exp(dtv * Ah);
                    /* output path */
                    for (int64_t p = 0; p < P; ++p) {
                        const double dyp = dyt[p];
                        double *grow = gs + p * N;
                        for (int64_t n = 0; n < N; ++n) grow[n] += dyp * Ct[n];
                    }
                    /* dC: read of s_t by C_t */
                    double *dCt = dC + IDX4(b, t, g, 0, T, G, N);
                    for (int64_t n = 0; n < N; ++n) {
                        double acc = 0.0;
                        for (int64_t p = 0; p < P; ++p) acc += dyt[p] * s_t[p * N + n];
                        dCt[n] += acc;
                    }
                    /* dx: write branch + skip branch */
                    double *dxt = dx + IDX4(b, t, h, 0, T, H, P);
                    double dD_tok = 0.0;
                    for (int64_t p = 0; p < P; ++p) {
                        double acc = 0.0;
                        for (int64_t n = 0; n < N; ++n) acc += gs[p * N + n] * Bt[n];
                        dxt[p] = Dh * dyt[p] + dtv * acc;
                        dD_tok += dyt[p] * xt[p];
                    }
                    dD_acc += dD_tok;
                    /* dB: write branch, summed over p (and over heads by the outer loop) */
                    double *dBt = dB + IDX4(b, t, g, 0, T, G, N);
                    for (int64_t n = 0; n < N; ++n) {
                        double acc = 0.0;
                        for (int64_t p = 0; p < P; ++p) acc += gs[p * N + n] * xt[p];
                        dBt[n] += dtv * acc;
                    }
                    /* dt: write branch + retention branch; A: retention branch */
                    double wsum = 0.0, rsum = 0.0;
                    for (int64_t p = 0; p < P; ++p) {
                        const double xv = xt[p];
                        for (int64_t n = 0; n < N; ++n) {
                            wsum += gs[p * N + n] * xv * Bt[n];
                            rsum += gs[p * N + n] * s_prev[p * N + n];
                        }
                    }
                    ddt[(b * T + t) * H + h] = wsum + rsum * a * Ah;
                    dA_acc += rsum * a * dtv;
                    /* carry to the previous state */
                    for (int64_t k = 0; k < PN; ++k) gs[k] *= a;
                }
            }
            if (dh0) memcpy(dh0 + bh * PN, gs, sizeof(double) * PN);
            dA_part[bh] = dA_acc;
            dD_part[bh] = dD_acc;
        }
        free(gs);
        free(states);
        free(seg_start);
    }
    for (int64_t h = 0; h < H; ++h) {
        double sa = 0.0, sd = 0.0;
        for (int64_t b = 0; b < Bsz; ++b) {
            sa += dA_part[b * H + h];
            sd += dD_part[b * H + h];
        }
        dA[h] = sa;
        dD[h] = sd;
    }
    free(dA_part);
    free(dD_part);
}

/*
 * One decode step: the forward with T = 1 on a state held by the caller.
 *   state [Bsz,H,P,N] in/out, x [Bsz,H,P], Bm/Cm [Bsz,G,N], dt [Bsz,H], y [Bsz,H,P].
 */
void oracle_decode_step(int64_t Bsz, int64_t H, int64_t P, int64_t N, int64_t G,
                        double *state, const double *x, const double *Bm, const double *Cm,
                        const double *dt, const double *A, const double *D, double *y) {
    const int64_t hpg = H / G;
    const int64_t PN = P * N;
#pragma omp parallel for schedule(static)
    for (int64_t bh = 0; bh < Bsz * H; ++bh) {
        const int64_t b = bh / H, h = bh % H, g = h / hpg;
        const double dtv = dt[bh];
        step_token(state + bh * PN, P, N, exp(dtv * A[h]), dtv, x + bh * P,
                   Bm + (b * G + g) * N, Cm + (b * G + g) * N, D[h], y + bh * P);
    }
}

/* ---------------------------------------------------------------------------
 * Counter-based entropy.  SplitMix64 (Steele, Lea & Flood 2014): the state
 * advances by the odd constant gamma and each output is the state passed
 * through the published 64-bit finaliser.  Output k (0-based) of a generator
 * seeded with s is mix(s + (k+1)*gamma).
 * ------------------------------------------------------------------------- */
static uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}
static const uint64_t SM64_GAMMA = 0x9E3779B97F4A7C15ULL;

uint64_t oracle_splitmix64_output(uint64_t seed, uint64_t k) {
    return sm64_mix(seed + (k + 1) * SM64_GAMMA);
}

/* Entropy word of element e of checkpoint j: output floor(e/2) of a SplitMix64
 * stream whose seed is output j of the stream seeded with `seed`, its high 32 bits
 * for even e and its low 32 bits for odd e (one output serves two elements). */
uint32_t oracle_hash32(uint64_t seed, uint64_t ckpt, uint64_t elem) {
    const uint64_t sub = oracle_splitmix64_output(seed, ckpt);
    const uint64_t out = oracle_splitmix64_output(sub, elem / 2);
    return (elem % 2 == 0) ? (uint32_t)(out >> 32) : (uint32_t)(out & 0xFFFFFFFFu);
}

/*
 * Stochastic rounding of one float32 value to binary16 bits, worked in double
 * on the real value (not on bit fields):
 *   q = binary16 spacing at |v|  (2^-24 below 2^-14, else 2^(floor(log2|v|)-10))
 *   k = floor(|v|/q), r = |v|/q - k  (the discarded remainder, in [0,1))
 *   R = floor(r * 2^32); take k+1 when the entropy word u < R
 *   result = sign * k * q; magnitudes >= 65536 become infinity; NaN keeps its
 *   sign and becomes the quiet NaN 0x7E00.
 */
uint16_t oracle_sr16_one(float v, uint32_t u) {
    const uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return (uint16_t)(sign | 0x7E00u);
    if (isinf(v)) return (uint16_t)(sign | 0x7C00u);
    const double m = fabs((double)v);
    if (m == 0.0) return sign;
    if (m >= 65536.0) return (uint16_t)(sign | 0x7C00u);
    int e2;
    (void)frexp(m, &e2);          /* m = f * 2^e2, f in [0.5, 1) */
    const int flo = e2 - 1;       /* floor(log2 m) */
    const int qexp = (flo < -14) ? -24 : flo - 10;
    const double ratio = ldexp(m, -qexp); /* exact: scaling by a power of two */
    double k = floor(ratio);
    const double r = ratio - k;  /* exact */
    const double R = floor(ldexp(r, 32));
    if ((double)u < R) k += 1.0;
    const double val = ldexp(k, qexp);
    if (val >= 65536.0) return (uint16_t)(sign | 0x7C00u);
    /* encode val (a multiple of q, exactly representable) as binary16 */
    if (val < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)ldexp(val, 24));
    int ve;
    (void)frexp(val, &ve);
    const int vflo = ve - 1;
    const double mant = ldexp(val, -vflo) - 1.0; /* in [0,1) */
    const uint16_t bits = (uint16_t)(((vflo + 15) << 10) | (uint16_t)ldexp(mant, 10));
    return (uint16_t)(sign | bits);
}

/* Element e of the array uses key (seed, ckpt, elem_offset + e). */
void oracle_sr16(const float *v, uint16_t *out, int64_t n, uint64_t seed, uint64_t ckpt,
                 uint64_t elem_offset) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_sr16_one(v[i], oracle_hash32(seed, ckpt, elem_offset + (uint64_t)i));
}

/* Exact binary16 -> double widening (used to read stored checkpoints back). */
double oracle_half_to_double(uint16_t hbits) {
    const int sign = (hbits >> 15) & 1;
    const int ex = (hbits >> 10) & 0x1F;
    const int man = hbits & 0x3FF;
    double v;
    if (ex == 0) v = ldexp((double)man, -24);
    else if (ex == 31) v = man ? NAN : INFINITY;
    else v = ldexp(1.0 + ldexp((double)man, -10), ex - 15);
    return sign ? -v : v;
}

void oracle_half_to_double_array(const uint16_t *in, double *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_half_to_double(in[i]);
}

/*
 * Time-step and rate preparation, with gradients.
 *  - "Nemotron Kernels: From Inference To Backpropagation", section "From
 *    Classical State Space To A Selective Mamba State": the time-step stream
 *    goes through softplus and is then clamped to a configured interval; the
 *    local derivative is the sigmoid inside the interval and zero where the
 *    clamp has saturated; the boundary needs a declared convention.
 *  - "Nemotron 3 Ultra: replaying a rounded state", section "The Mamba state
 *    update": the time step is formed from the raw time step and a per-head
 *    bias, and the per-head rate is A = -exp(logA).
 * Readings: the bias is added before the softplus; the interval is closed and
 * a value equal to either end passes its gradient (the clamp is the identity
 * there); the inside/outside decision is taken on the float32 value of the
 * softplus, the precision the time step is stored in.  softplus is the
 * mathematical log(1 + e^v), evaluated as max(v, 0) + log1p(e^-|v|).
 */
static double softplus64(double v) { return (v > 0 ? v : 0.0) + log1p(exp(-fabs(v))); }

static double sigmoid64(double v) {
    if (v >= 0) return 1.0 / (1.0 + exp(-v));
    const double e = exp(v);
    return e / (1.0 + e);
}

static int inside(double sp, float lo, float hi) {
    const float s32 = (float)sp;
    return s32 >= lo && s32 <= hi;
}

/* raw [rows][H], bias [H], logA [H] -> dt [rows][H], A [H] */
void oracle_dt_prep(int64_t rows, int64_t H, const double *raw, const double *bias,
                    const double *logA, float lo, float hi, double *dt, double *A) {
    for (int64_t h = 0; h < H; ++h) A[h] = -exp(logA[h]);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t h = 0; h < H; ++h) {
            const double sp = softplus64(raw[r * H + h] + bias[h]);
            dt[r * H + h] = sp < lo ? (double)lo : (sp > hi ? (double)hi : sp);
        }
}

/* Chain rule back through the preparation: ddt [rows][H] and dA [H] are the
 * gradients with respect to the prepared dt and A.  d_raw = ddt * sigmoid *
 * [inside]; d_bias[h] = sum over rows of d_raw (rows ascending); d_logA = dA * A
 * (the derivative of -exp(logA) is itself). */
void oracle_dt_prep_bwd(int64_t rows, int64_t H, const double *raw, const double *bias,
                        const double *logA, float lo, float hi, const double *ddt,
                        const double *dA, double *d_raw, double *d_bias, double *d_logA) {
    for (int64_t h = 0; h < H; ++h) {
        d_logA[h] = dA[h] * -exp(logA[h]);
        d_bias[h] = 0.0;
    }
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t h = 0; h < H; ++h) {
            const double v = raw[r * H + h] + bias[h];
            const double g = inside(softplus64(v), lo, hi) ? ddt[r * H + h] * sigmoid64(v) : 0.0;
            d_raw[r * H + h] = g;
            d_bias[h] += g;
        }
}

/*
 * Short causal depthwise convolution followed by SiLU, and its backward.
 * "Nemotron Kernels: From Inference To Backpropagation", Kernel 1 "Forward And
 * Inference": the hidden stream passes a causal Conv1D + SiLU before the scan;
 * each output multiplies a short weight vector with the current sample and the
 * ones before it (never a later one) and adds the products; the decode kernel
 * applies SiLU to the convolution sum.  Section "What Conv1D Gives The Mamba
 * Block": in the backward every output gradient reaches the inputs of its window,
 * the weights that touched them and the bias, and overlapping windows add at one
 * input; the SiLU derivative is applied first.
 * Per batch b and channel c, with the K-1 samples before token 0 taken from
 * init [Bsz][K-1][Cch] (zero when init is NULL):
 *   ext[j] = init[j] (j < K-1),  ext[K-1+t] = u[t]
 *   v[t]   = bias[c] + sum_{k=0..K-1} w[c][k] * ext[t+k]      (w[c][K-1] meets u[t])
 *   out[t] = v[t] * sigmoid(v[t])
 * final [Bsz][K-1][Cch] receives ext[T .. T+K-2] (the samples the next call
 * needs).  Layouts: u, out [Bsz][T][Cch]; w [Cch][K]; bias [Cch].
 */
static double silu64(double v) { return v * sigmoid64(v); }
static double silu_grad64(double v) {
    const double s = sigmoid64(v);
    return s * (1.0 + v * (1.0 - s));
}

static void conv_window(int64_t T, int64_t Cch, int64_t K, const double *u, const double *init,
                        int64_t b, int64_t c, double *ext) {
    for (int64_t j = 0; j < K - 1; ++j) ext[j] = init ? init[(b * (K - 1) + j) * Cch + c] : 0.0;
    for (int64_t t = 0; t < T; ++t) ext[K - 1 + t] = u[(b * T + t) * Cch + c];
}

void oracle_conv1d_silu(int64_t Bsz, int64_t T, int64_t Cch, int64_t K, const double *u,
                        const double *w, const double *bias, const double *init, double *out,
                        double *final_state) {
#pragma omp parallel
    {
        double *ext = malloc(sizeof(double) * (size_t)(T + K));
#pragma omp for collapse(2) schedule(static)
        for (int64_t b = 0; b < Bsz; ++b)
            for (int64_t c = 0; c < Cch; ++c) {
                conv_window(T, Cch, K, u, init, b, c, ext);
                for (int64_t t = 0; t < T; ++t) {
                    double v = bias[c];
                    for (int64_t k = 0; k < K; ++k) v += w[c * K + k] * ext[t + k];
                    out[(b * T + t) * Cch + c] = silu64(v);
                }
                if (final_state)
                    for (int64_t j = 0; j < K - 1; ++j) final_state[(b * (K - 1) + j) * Cch + c] = ext[T + j];
            }
        free(ext);
    }
}

/* dv = dout * SiLU'(v); d ext[t+k] += w[c][k] dv[t]; dw[c][k] += dv[t] ext[t+k];
 * dbias[c] += dv[t]; du[t] = d ext[K-1+t]; dinit[j] = d ext[j].  Sums over (b, t)
 * ascending.  dinit may be NULL. */
void oracle_conv1d_silu_bwd(int64_t Bsz, int64_t T, int64_t Cch, int64_t K, const double *u,
                            const double *w, const double *bias, const double *init,
                            const double *dout, double *du, double *dw, double *dbias,
                            double *dinit) {
#pragma omp parallel
    {
        double *ext = malloc(sizeof(double) * (size_t)(T + K));
        double *dext = malloc(sizeof(double) * (size_t)(T + K));
#pragma omp for schedule(static)
        for (int64_t c = 0; c < Cch; ++c) {
            double db = 0.0;
            for (int64_t k = 0; k < K; ++k) dw[c * K + k] = 0.0;
            for (int64_t b = 0; b < Bsz; ++b) {
                conv_window(T, Cch, K, u, init, b, c, ext);
                for (int64_t j = 0; j < T + K - 1; ++j) dext[j] = 0.0;
                for (int64_t t = 0; t < T; ++t) {
                    double v = bias[c];
                    for (int64_t k = 0; k < K; ++k) v += w[c * K + k] * ext[t + k];
                    const double dv = dout[(b * T + t) * Cch + c] * silu_grad64(v);
                    db += dv;
                    for (int64_t k = 0; k < K; ++k) {
                        dext[t + k] += w[c * K + k] * dv;
                        dw[c * K + k] += dv * ext[t + k];
                    }
                }
                for (int64_t t = 0; t < T; ++t) du[(b * T + t) * Cch + c] = dext[K - 1 + t];
                if (dinit)
                    for (int64_t j = 0; j < K - 1; ++j) dinit[(b * (K - 1) + j) * Cch + c] = dext[j];
            }
            dbias[c] = db;
        }
        free(ext);
        free(dext);
    }
}

/*
 * Gated group RMSNorm after the scan, and its backward.  Same page, Kernel 1
 * pipeline "selective scan -> gated group RMSNorm" and section "From Classical
 * State Space To A Selective Mamba State": a learned SiLU gate controls how much
 * signal passes; the page's RMSNorm remark: its backward needs the input, the
 * learned scale, the inverse RMS and the reduction.  Reading: the gate multiplies
 * before the normalisation and the mean square is taken over each group of
 * Cch/G consecutive channels:
 *   g = y * SiLU(z);  r = 1/sqrt(mean_group(g^2) + eps);  out = g * r * w[c]
 * Layouts: y, z, out [rows][Cch]; w [Cch].
 */
void oracle_gated_rmsnorm(int64_t rows, int64_t Cch, int64_t G, const double *y, const double *z,
                          const double *w, double eps, double *out) {
    const int64_t S = Cch / G;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t gi = 0; gi < G; ++gi) {
            const int64_t o = r * Cch + gi * S;
            double ms = 0.0;
            for (int64_t i = 0; i < S; ++i) {
                const double g = y[o + i] * silu64(z[o + i]);
                ms += g * g;
            }
            const double rs = 1.0 / sqrt(ms / (double)S + eps);
            for (int64_t i = 0; i < S; ++i) out[o + i] = y[o + i] * silu64(z[o + i]) * rs * w[gi * S + i];
        }
}

/* n = g r;  dw[c] = sum over rows of dout n;  dn = dout w;
 * dg = r (dn - n mean_group(dn n));  dy = dg SiLU(z);  dz = dg y SiLU'(z). */
void oracle_gated_rmsnorm_bwd(int64_t rows, int64_t Cch, int64_t G, const double *y,
                              const double *z, const double *w, double eps, const double *dout,
                              double *dy, double *dz, double *dw) {
    const int64_t S = Cch / G;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t gi = 0; gi < G; ++gi) {
            const int64_t o = r * Cch + gi * S;
            double ms = 0.0;
            for (int64_t i = 0; i < S; ++i) {
                const double g = y[o + i] * silu64(z[o + i]);
                ms += g * g;
            }
            const double rs = 1.0 / sqrt(ms / (double)S + eps);
            double m = 0.0;
            for (int64_t i = 0; i < S; ++i) {
                const double n = y[o + i] * silu64(z[o + i]) * rs;
                m += dout[o + i] * w[gi * S + i] * n;
            }
            m /= (double)S;
            for (int64_t i = 0; i < S; ++i) {
                const double n = y[o + i] * silu64(z[o + i]) * rs;
                const double dg = rs * (dout[o + i] * w[gi * S + i] - n * m);
                dy[o + i] = dg * silu64(z[o + i]);
                dz[o + i] = dg * y[o + i] * silu_grad64(z[o + i]);
            }
        }
    for (int64_t c = 0; c < Cch; ++c) dw[c] = 0.0;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t gi = 0; gi < G; ++gi) {
            const int64_t o = r * Cch + gi * S;
            double ms = 0.0;
            for (int64_t i = 0; i < S; ++i) {
                const double g = y[o + i] * silu64(z[o + i]);
                ms += g * g;
            }
            const double rs = 1.0 / sqrt(ms / (double)S + eps);
            for (int64_t i = 0; i < S; ++i) dw[gi * S + i] += dout[o + i] * y[o + i] * silu64(z[o + i]) * rs;
        }
}
