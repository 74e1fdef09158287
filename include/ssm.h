/*
 * ssm.h -- C ABI of the MI355X (gfx950) Mamba-2 selective state-space library.
 *
 * The recurrence, per batch b, head h and group g = h / (nheads/ngroups):
 *     a_t      = exp(dt[b,t,h] * A[h])
 *     s[p][n]  = a_t * s[p][n] + x[b,t,h,p] * (B[b,t,g,n] * dt[b,t,h])
 *     y[b,t,h,p] = sum_n C[b,t,g,n] * s[p][n] + D[h] * x[b,t,h,p]
 * "Nemotron 3 Ultra: replaying a rounded state" (TorchLean Verified Examples),
 * section "The Mamba state update" (theorem updateHead_apply: per-coordinate
 * update with the head's group B and a per-head rate), and section "Recovering
 * the state by replay" (the output reads the updated state).
 *
 * Conventions shared by every call
 *  - Layouts are dense row-major:
 *      x, y, dy, dx   [batch, seqlen, nheads, headdim]           (dtype)
 *      B, C           [batch, seqlen, ngroups, dstate]           (dtype)
 *      dB, dC         [batch, seqlen, ngroups, dstate]           float
 *      dt, ddt        [batch, seqlen, nheads]                    float (dt > 0)
 *      A, D, dA, dD   [nheads]                                   float
 *      states         [batch, nheads, headdim, dstate]           float
 *      chunk_states   [batch, nheads, nchunks, headdim, dstate]  float,
 *                     nchunks = ceil(seqlen/chunk); entry c is the state
 *                     ENTERING chunk c (entry 0 is the initial state).
 *  - `dtype` (SSM_F32 or SSM_BF16) is the storage type of x, B, C, dy, y, dx.
 *  - All pointers are device pointers (HBM) owned by the caller.  Alignment:
 *    state-shaped float arrays (states, chunk_states, h0, h_final, dh_final,
 *    dh0, checkpoints) and the workspace: 16 bytes; B, C, dB, dC: 16 bytes on
 *    the MFMA path, else 4 elements; x, y, dy, dx: 16 bytes on the MFMA path,
 *    else one element; dt, A, D, ddt, dA, dD, drift arrays: 4 bytes.
 *    The library never allocates and never synchronises; all work is enqueued
 *    on `stream` (a hipStream_t; NULL means the null stream).
 *  - Outputs are overwritten, never accumulated.
 *  - Every argument is validated before anything is enqueued; on any error
 *    nothing is written ("detected before any work", as in "Reverse-mode
 *    automatic differentiation" (OneModel docs), section 2 "The engine").
 *  - Calls are stateless and reentrant; calls on different streams that
 *    write the same buffers race.
 *  - Results are deterministic: no floating-point atomics; every reduction
 *    has a fixed order.
 */
#ifndef SSM_MI355X_H
#define SSM_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* In C++ the two enums get the fixed underlying type int: a caller in C (or through
 * an FFI) may pass any int, and C++ gives an unfixed enum holding a value outside its
 * enumerators' range undefined behaviour, before the validation could reject it.  The
 * ABI is that of int either way. */
#ifdef __cplusplus
typedef enum ssm_status_e : int {
#else
typedef enum ssm_status_e {
#endif
    SSM_OK = 0,
    SSM_ERR_NULL = 1,        /* a required pointer is NULL */
    SSM_ERR_DIMS = 2,        /* non-positive dim, nheads % ngroups != 0, ... */
    SSM_ERR_UNSUPPORTED = 3, /* a (headdim, dstate, chunk) with no kernel */
    SSM_ERR_DTYPE = 4,       /* unknown dtype */
    SSM_ERR_ALIGN = 5,       /* a pointer is not aligned as required */
    SSM_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required */
    SSM_ERR_HIP = 7          /* a HIP launch reported an error */
} ssm_status;

#ifdef __cplusplus
typedef enum ssm_dtype_e : int { SSM_F32 = 0, SSM_BF16 = 1, SSM_F16 = 2 } ssm_dtype;
#else
typedef enum ssm_dtype_e { SSM_F32 = 0, SSM_BF16 = 1, SSM_F16 = 2 } ssm_dtype;
#endif

typedef struct {
    int64_t batch;
    int64_t seqlen;
    int64_t nheads;
    int64_t headdim;  /* P: value channels per head */
    int64_t dstate;   /* N: state coordinates */
    int64_t ngroups;  /* heads h in [g*nheads/ngroups, (g+1)*nheads/ngroups) share B, C */
    int64_t chunk;    /* L: chunk length (state save interval) */
} ssm_dims;

typedef void *ssm_stream; /* hipStream_t */

/* Workspace kinds for ssm_workspace_bytes. */
enum { SSM_WS_FWD = 0, SSM_WS_BWD = 1, SSM_WS_REPLAY = 2, SSM_WS_DT_PREP_BWD = 3 };

/* Bytes of device workspace a call needs (0 is a valid answer).  `r` is the
 * replay length for SSM_WS_REPLAY and ignored otherwise.  Returns (size_t)-1
 * for invalid or unsupported dims. */
size_t ssm_workspace_bytes(const ssm_dims *d, ssm_dtype dtype, int which, int64_t r);

/* Static human-readable name of a status code. */
const char *ssm_status_string(ssm_status s);

/* 1 when the chunked MFMA kernels serve both the forward and the backward for
 * these dims and dtype: bf16 operands, headdim 64, dstate 128, chunk a multiple
 * of 64, and for the backward also chunk <= 256 and at most 64 heads per group.
 * Otherwise the exact-fp32 sequential kernels run the part the MFMA kernels do
 * not serve (the forward alone still takes the MFMA path whenever its own
 * conditions hold).  Purely informational. */
int ssm_uses_mfma_path(const ssm_dims *d, ssm_dtype dtype);

/*
 * Chunked prefill forward.  "Nemotron Kernels: From Inference To
 * Backpropagation", Kernel 1: the prefill scan walks the whole sequence and
 * returns the outputs and the final state.
 *   h0            initial state or NULL (zero)
 *   y             outputs (dtype)
 *   h_final       final state or NULL
 *   chunk_states  states entering each chunk or NULL (needed by ssm_bwd)
 *   workspace     ssm_workspace_bytes(d, dtype, SSM_WS_FWD, 0) bytes
 */
ssm_status ssm_fwd_chunked(const ssm_dims *d, ssm_dtype dtype, const void *x, const void *B,
                           const void *C, const float *dt, const float *A, const float *D,
                           const float *h0, void *y, float *h_final, float *chunk_states,
                           void *workspace, size_t ws_bytes, ssm_stream stream);

/*
 * Reverse-mode backward.  Same page, Kernel 1 "Backpropagation: What Mamba2
 * Backward Must Do": a reverse walk over the tokens in which the state
 * gradient is the output path plus the future recurrent path, and shared B/C
 * receive the sum over every head and channel of their group.  The loss seen
 * by the backward is sum(dy*y) + sum(dh_final*h_final).
 *   chunk_states  from ssm_fwd_chunked with the same dims (entry 0 = h0); the
 *                 backward recomputes everything else from them
 *   dh_final      gradient on the final state or NULL (zero)
 *   dx            (dtype); dB, dC summed over the group's heads; ddt w.r.t.
 *                 the dt input; dA, dD summed over batch and tokens;
 *   dh0           gradient on the initial state, or NULL
 *   workspace     ssm_workspace_bytes(d, dtype, SSM_WS_BWD, 0) bytes
 */
ssm_status ssm_bwd(const ssm_dims *d, ssm_dtype dtype, const void *x, const void *B,
                   const void *C, const float *dt, const float *A, const float *D,
                   const float *chunk_states, const void *dy, const float *dh_final, void *dx,
                   float *dB, float *dC, float *ddt, float *dA, float *dD, float *dh0,
                   void *workspace, size_t ws_bytes, ssm_stream stream);

/*
 * ssm_bwd with the per-block stage timed (for measurement; the pages print no
 * such call).  Same arguments, results and validation as ssm_bwd, plus
 * block_events: two hipEvent_t handles created by the caller on the current
 * device.  When the chunked MFMA path runs, block_events[0] is recorded on
 * `stream` immediately before the per-block backward kernel and block_events[1]
 * immediately after it, so hipEventElapsedTime gives that kernel's duration;
 * on the other paths both are recorded once at the start of the call.  Both
 * events are first recorded before any work is enqueued, so an unusable event
 * returns SSM_ERR_HIP with nothing written; NULL block_events, or a NULL
 * handle, returns SSM_ERR_NULL.  No state is kept between calls.
 */
ssm_status ssm_bwd_timed(const ssm_dims *d, ssm_dtype dtype, const void *x, const void *B,
                         const void *C, const float *dt, const float *A, const float *D,
                         const float *chunk_states, const void *dy, const float *dh_final,
                         void *dx, float *dB, float *dC, float *ddt, float *dA, float *dD,
                         float *dh0, void *workspace, size_t ws_bytes, void *const *block_events,
                         ssm_stream stream);

/*
 * ssm_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same inputs,
 * outputs, results and validation as ssm_bwd, without the workspace: the
 * kernels use a scratch array the library holds in device memory, one copy per
 * GPU it runs on, from module load until the process ends.  The array holds
 * 65 MiB (SSM_NOALLOC_SCRATCH_BYTES), enough for one 4096-token sequence at
 * 256 heads x 64 x 128 with chunk 256; when ssm_workspace_bytes(d, dtype,
 * SSM_WS_BWD, 0) exceeds it the call returns SSM_ERR_WORKSPACE and does nothing.
 * The call itself allocates nothing and calls no allocating routine; the first
 * call on a device looks up that device's copy of the array (SSM_ERR_HIP if the
 * lookup fails, before any work).  Every call on a GPU shares that GPU's array
 * and leaves its contents behind: calls that overlap on one GPU (on different
 * streams, or from different threads) race and must be serialised by the
 * caller.  Results are bit-identical to ssm_bwd's.
 */
#define SSM_NOALLOC_SCRATCH_BYTES ((size_t)65 << 20)
ssm_status ssm_bwd_noalloc(const ssm_dims *d, ssm_dtype dtype, const void *x, const void *B,
                           const void *C, const float *dt, const float *A, const float *D,
                           const float *chunk_states, const void *dy, const float *dh_final,
                           void *dx, float *dB, float *dC, float *ddt, float *dA, float *dD,
                           float *dh0, ssm_stream stream);

/*
 * One-token decode state update, in place.  Same page, Kernel 1: decode
 * evaluates the same recurrence for one step.  `d->seqlen` and `d->chunk` are
 * ignored.  Shapes: state [batch,nheads,headdim,dstate] float (in/out),
 * x [batch,nheads,headdim], B, C [batch,ngroups,dstate], dt [batch,nheads],
 * y [batch,nheads,headdim] (dtype).  Bit-identical to one step of ssm_replay.
 */
ssm_status ssm_decode_step(const ssm_dims *d, ssm_dtype dtype, float *state, const void *x,
                           const void *B, const void *C, const float *dt, const float *A,
                           const float *D, void *y, ssm_stream stream);

/*
 * One-token decode with a binary16 state cache, in place.  "Nemotron 3 Ultra:
 * replaying a rounded state", introduction (the quantized model keeps the
 * recurrent state cache in FP16 and stores it with stochastic rounding) and
 * section "Counting the state and attention cache" (FP16 halves the state
 * bytes against float32).  state16 [batch,nheads,headdim,dstate] holds binary16
 * bits (8-byte aligned); each element is widened exactly to float32, advanced
 * by the same arithmetic as ssm_decode_step, and stored back with the rounding
 * rule of ssm_checkpoint_sr16 keyed by (seed, step): element i (flat index of
 * state16) uses the entropy word of element i with ckpt_index = step (the high or
 * low half of SM(SM(seed, step), i / 2) for even or odd i).  y is what ssm_decode_step
 * writes from the widened state, bit for bit.  Inputs as for ssm_decode_step;
 * the caller passes a distinct `step` per decode step so rounding choices are
 * independent across steps and reproducible for replay.
 */
ssm_status ssm_decode_step_sr16(const ssm_dims *d, ssm_dtype dtype, uint16_t *state16,
                                const void *x, const void *B, const void *C, const float *dt,
                                const float *A, const float *D, void *y, uint64_t seed,
                                uint64_t step, ssm_stream stream);

/*
 * FP16 stochastically rounded checkpoint of a float32 state.  "Nemotron 3
 * Ultra: replaying a rounded state", sections "Stochastic rounding and the
 * mean state" (round up when the entropy residue is below the discarded
 * remainder) and "Recovering the state by replay" (a random step keeps its
 * random choices, so the entropy is a pure function of a key).
 * Element i of `state` (n_elems of them), e = elem_offset + i, is rounded with
 * the entropy word
 *   u = high32( SM(SM(seed, ckpt_index), e / 2) )  for even e,
 *   u = low32(  SM(SM(seed, ckpt_index), e / 2) )  for odd e,
 * where SM(s, k) is output k (0-based) of a SplitMix64 stream seeded with s
 * (one output serves two elements).
 * With R = floor(remainder * 2^32), the magnitude goes to the upper binary16
 * neighbour iff u < R.  Magnitudes reaching 65536 become infinity; NaN keeps
 * its sign as 0x7E00.  `out` receives binary16 bits and must not alias state.
 */
ssm_status ssm_checkpoint_sr16(const float *state, uint16_t *out, uint64_t n_elems,
                               uint64_t seed, uint64_t ckpt_index, uint64_t elem_offset,
                               ssm_stream stream);

/*
 * Replay r retained tokens from a checkpoint.  Same page, section
 * "Recovering the state by replay": re-applying the retained prepared inputs
 * in order from a saved state recovers the current state.
 *   ckpt        [batch,nheads,headdim,dstate], float (ckpt_dtype SSM_F32) or
 *               binary16 bits (SSM_F16, widened exactly)
 *   state_out   state after the r tokens (float); may alias ckpt if SSM_F32
 *   x, B, C, dt full-length inputs ([batch, seqlen, ...]); tokens
 *               t0 .. t0+r-1 are replayed (t0 + r <= seqlen)
 *   y           NULL, or [batch,seqlen,nheads,headdim] (dtype): the outputs of
 *               the replayed tokens are written at t0 .. t0+r-1
 *   live_ckpt   NULL, or a float state advanced in lockstep with the same
 *               inputs (not written); then drift_max[k] and drift_mean[k]
 *               (k = 0..r-1) receive max and mean over all elements of
 *               |replayed - live| after token t0+k
 *   workspace   ssm_workspace_bytes(d, dtype, SSM_WS_REPLAY, r) bytes (0 when
 *               live_ckpt is NULL)
 * The step arithmetic is the one of ssm_decode_step, bit for bit.
 */
ssm_status ssm_replay(const ssm_dims *d, ssm_dtype dtype, const void *ckpt, ssm_dtype ckpt_dtype,
                      float *state_out, const void *x, const void *B, const void *C,
                      const float *dt, const float *A, const float *D, int64_t t0, int64_t r,
                      void *y, const float *live_ckpt, float *drift_max, float *drift_mean,
                      void *workspace, size_t ws_bytes, ssm_stream stream);

/*
 * Speculative draft with a snapshot after every step.  "Nemotron 3 Ultra:
 * replaying a rounded state", section "Rolling back rejected draft tokens": a
 * Mamba update overwrites its fixed-size state, so a snapshot is kept at every
 * draft step, the initial state included, so that rejecting the whole draft
 * selects it.  d->seqlen is the draft length Dr (d->chunk is ignored).
 *   snapshots  float [Dr+1][batch][nheads][headdim][dstate], 16-byte aligned:
 *              slot 0 holds the state before the draft (read, not written);
 *              slot k (1..Dr) receives the state after draft tokens 0..k-1
 *   x          [batch, Dr, nheads, headdim] (dtype); B, C [batch, Dr, ngroups,
 *              dstate] (dtype); dt [batch, Dr, nheads] float
 *   y          NULL, or [batch, Dr, nheads, headdim] (dtype): the draft outputs
 * Each token is the update of ssm_decode_step, bit for bit: slot k equals the
 * state after k ssm_decode_step calls on the same inputs.  Supported dims and
 * alignment are those of ssm_decode_step.
 */
ssm_status ssm_draft_snapshots(const ssm_dims *d, ssm_dtype dtype, float *snapshots,
                               const void *x, const void *B, const void *C, const float *dt,
                               const float *A, const float *D, void *y, ssm_stream stream);

/*
 * Rollback after verification (same section): the state to continue from is
 * the snapshot after the accepted prefix, per sequence.
 *   snapshots  from ssm_draft_snapshots with the same dims (d->seqlen = Dr)
 *   accepted   device int32 [batch], each in [0, Dr]: the number of accepted
 *              draft tokens of that sequence
 *   state_out  float [batch][nheads][headdim][dstate], 16-byte aligned;
 *              state_out[b] <- snapshots[accepted[b]][b] (a copy, bit for bit).
 *              It may be one of the snapshot slots (for example slot 0, so the
 *              next draft starts from it); otherwise it must not overlap them.
 *   err        NULL, or a device int32 set to 1 when some accepted[b] lies
 *              outside [0, Dr]; that sequence's state_out is then not written
 *              (the value is only known on the device, so it cannot be rejected
 *              before the launch).  The flag is never cleared by the call.
 */
ssm_status ssm_rollback(const ssm_dims *d, const float *snapshots, const int32_t *accepted,
                        float *state_out, int32_t *err, ssm_stream stream);

/*
 * Short causal depthwise convolution followed by SiLU, the stage before the
 * scan.  "Nemotron Kernels: From Inference To Backpropagation", Kernel 1
 * "Forward And Inference" (the hidden stream passes a causal Conv1D + SiLU; an
 * output reads the present and past samples of its channel, never a future
 * one; the decode kernel applies SiLU to the convolution sum).  Per batch b and
 * channel c with `width` = K taps and the K-1 samples before token 0 taken from
 * conv_init (zero when NULL):
 *   v[t]   = bias[c] + sum_{k<K} w[c][k] * ext[t+k],  ext = (conv_init, u)
 *   out[t] = v[t] * sigmoid(v[t])
 * Layouts: u, out [batch][seqlen][channels] (dtype); w [channels][K] float;
 * bias [channels] float; conv_init, conv_final [batch][K-1][channels] (dtype).
 * conv_final (may be NULL) receives the last K-1 samples of (conv_init, u): the
 * conv_init of the next call (seqlen = 1 is the decode step).
 * Constraints: 1 <= width <= 8; channels a positive multiple of 4; batch <=
 * 65535; u, out, bias, conv_init, conv_final 16-byte aligned, w 4-byte aligned.
 * out must not overlap u or conv_init.
 */
ssm_status ssm_conv1d_silu(int64_t batch, int64_t seqlen, int64_t channels, int64_t width,
                           ssm_dtype dtype, const void *u, const float *w, const float *bias,
                           const void *conv_init, void *out, void *conv_final,
                           ssm_stream stream);

/* Workspace bytes of ssm_conv1d_silu_bwd ((size_t)-1 for invalid sizes). */
size_t ssm_conv1d_silu_workspace_bytes(int64_t batch, int64_t seqlen, int64_t channels,
                                       int64_t width);

/*
 * Backward of ssm_conv1d_silu (same page, section "What Conv1D Gives The Mamba
 * Block": the SiLU derivative first, then each output gradient reaches the
 * inputs of its window, the weights that touched them and the bias; overlapping
 * windows add at one input).  With dv = dout * SiLU'(v):
 *   du[t] = sum_k w[c][k] dv[t+K-1-k];  dw[c][k] = sum_{b,t} dv[t] ext[t+k];
 *   dbias[c] = sum_{b,t} dv[t];  dconv_init[j] = sum_{k<=j} w[c][k] dv[j-k]
 * du, dconv_init (NULL to skip) in dtype; dw [channels][K], dbias float (fp64
 * partial sums in a fixed order).  Same layouts and constraints as the forward.
 */
ssm_status ssm_conv1d_silu_bwd(int64_t batch, int64_t seqlen, int64_t channels, int64_t width,
                               ssm_dtype dtype, const void *u, const float *w, const float *bias,
                               const void *conv_init, const void *dout, void *du, float *dw,
                               float *dbias, void *dconv_init, void *workspace, size_t ws_bytes,
                               ssm_stream stream);

/*
 * SiLU-gated group RMSNorm, the stage after the scan.  Same page, Kernel 1
 * pipeline ("selective scan -> gated group RMSNorm") and section "From
 * Classical State Space To A Selective Mamba State" (a learned SiLU gate
 * controls how much signal passes).  Over groups of S = channels/ngroups
 * consecutive channels of each row:
 *   g = y * SiLU(z);  out = g / sqrt(mean_group(g^2) + eps) * w[c]
 * Layouts: y, z, out [rows][channels] (dtype); w [channels] float.
 * Constraints: S a multiple of 8 and at most 8192; rows < 2^31; ngroups <=
 * 65535; eps >= 0 and finite (with eps = 0 an all-zero group divides by zero);
 * all pointers 16-byte aligned.
 */
ssm_status ssm_gated_rmsnorm(int64_t rows, int64_t channels, int64_t ngroups, ssm_dtype dtype,
                             const void *y, const void *z, const float *w, float eps, void *out,
                             ssm_stream stream);

/* Workspace bytes of ssm_gated_rmsnorm_bwd ((size_t)-1 for invalid sizes). */
size_t ssm_gated_rmsnorm_workspace_bytes(int64_t rows, int64_t channels, int64_t ngroups);

/*
 * Backward of ssm_gated_rmsnorm (the page's RMSNorm remark: the backward needs
 * the input, the learned scale, the inverse RMS and the reduction).  With
 * r = 1/sqrt(mean_group(g^2) + eps), n = g r, dn = dout w:
 *   dg = r (dn - n mean_group(dn n));  dy = dg SiLU(z);  dz = dg y SiLU'(z)
 *   dw[c] = sum over rows of dout n   (fp64 partial sums, fixed order)
 * dy, dz in dtype; dw float.  The inverse RMS is recomputed from y and z.
 */
ssm_status ssm_gated_rmsnorm_bwd(int64_t rows, int64_t channels, int64_t ngroups,
                                 ssm_dtype dtype, const void *y, const void *z, const float *w,
                                 float eps, const void *dout, void *dy, void *dz, float *dw,
                                 void *workspace, size_t ws_bytes, ssm_stream stream);

/*
 * Time-step and rate preparation.  "Nemotron Kernels: From Inference To
 * Backpropagation", section "From Classical State Space To A Selective Mamba
 * State" (the time step goes through softplus and is clamped to a configured
 * interval); "Nemotron 3 Ultra: replaying a rounded state", section "The Mamba
 * state update" (the time step is built from the raw value and a per-head
 * bias; the rate is A = -exp(logA)).
 *   dt[r,h] = min(max(softplus(dt_raw[r,h] + dt_bias[h]), dt_lo), dt_hi)
 *   A[h]    = -exp(logA[h])
 * Only d->batch, d->seqlen and d->nheads are read: rows r = batch * seqlen,
 * layouts dt_raw, dt [batch, seqlen, nheads] and dt_bias, logA, A [nheads],
 * all float32, 4-byte aligned, device memory.  dt_lo <= dt_hi (dt_hi may be
 * +inf; neither may be NaN), else SSM_ERR_DIMS.  softplus is evaluated in
 * float32 without a threshold branch (log(1+e^v) computed as
 * max(v,0) + log1p(e^-|v|)).  dt may alias dt_raw.
 */
ssm_status ssm_dt_prep(const ssm_dims *d, const float *dt_raw, const float *dt_bias,
                       const float *logA, float dt_lo, float dt_hi, float *dt, float *A,
                       ssm_stream stream);

/*
 * Chain rule back through ssm_dt_prep (same passages: the derivative of the
 * softplus is the sigmoid inside the interval and zero where the clamp
 * saturates; the interval is closed, so a softplus equal to dt_lo or dt_hi
 * passes its gradient).  ddt [batch, seqlen, nheads] and dA [nheads] are the
 * gradients on the prepared dt and A (as returned by ssm_bwd).
 *   d_raw[r,h]  = ddt[r,h] * sigmoid(dt_raw[r,h] + dt_bias[h]) * [inside]
 *   d_bias[h]   = sum over r of d_raw[r,h]   (fp64 partial sums, fixed order)
 *   d_logA[h]   = dA[h] * A[h] = -dA[h] * exp(logA[h])
 * The inside test is taken on the float32 softplus that ssm_dt_prep stores.
 *   workspace   ssm_workspace_bytes(d, SSM_F32, SSM_WS_DT_PREP_BWD, 0) bytes
 * Same dims, layouts and alignment as ssm_dt_prep; d_raw may alias ddt.
 */
ssm_status ssm_dt_prep_bwd(const ssm_dims *d, const float *dt_raw, const float *dt_bias,
                           const float *logA, float dt_lo, float dt_hi, const float *ddt,
                           const float *dA, float *d_raw, float *d_bias, float *d_logA,
                           void *workspace, size_t ws_bytes, ssm_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_MI355X_H */
