/*
 * selscan.h -- C ABI of libselscan, the selective state-space scan of Mamba
 * on AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For every batch b, channel d, state index n and token t
 * (Mamba-1 form):
 *
 *     Delta_t  = softplus(delta_t + delta_bias_d)      (or delta_t + bias if softplus == 0)
 *     h_t[n]   = exp(Delta_t * A[d,n]) * h_{t-1}[n] + Delta_t * B_t[n] * u_t,   h_{-1} = 0
 *     y_t      = (sum_n C_t[n] * h_t[n] + D_d * u_t) * silu(z_t)             (gate optional)
 *
 * Sources: the "Understanding Mamba and Selective State Space Models (SSMs)"
 * blog, section 2.2 (the selective update with exp(Delta A), the recurrent
 * scan from a zero state, softplus keeping Delta positive) and section 2.1
 * (the read-out y = C h + D x); the Mamba README on the gittoolsai page for
 * state-spaces/mamba, sections "Selective SSM" (the layer), "Mamba-2" and
 * "Initialization" (the Delta bias); the "model-architecture-mamba" skill
 * page (Mamba-2: multi-head, d_state 128, headdim 64).  Where the pages are
 * silent the plainest reading is taken: the read-out sums over n, the gate
 * multiplies the D term too, the initial state is zero, A is stored negative.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller, dense and
 *    row-major in the layouts given below.  The library keeps no pointer after
 *    a call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *    is enqueued on it and the call returns without synchronising.  Faults
 *    inside a kernel surface at the caller's next synchronisation.
 *  - Argument errors are detected on the host before any device work and
 *    return SELSCAN_ERR_INVALID_ARG / SELSCAN_ERR_UNSUPPORTED with a message
 *    available from selscan_last_error() on the calling thread.  No C++
 *    exception crosses this interface; the library never aborts the process.
 *  - NaN and Inf in the inputs propagate to the outputs; nothing is clamped.
 *  - Calls on distinct streams may run concurrently.
 */
#ifndef SELSCAN_H
#define SELSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SELSCAN_OK = 0,
    SELSCAN_ERR_INVALID_ARG = 1,  /* null required pointer, bad size, overflow */
    SELSCAN_ERR_UNSUPPORTED = 2,  /* valid but not implemented (dtype, d_state) */
    SELSCAN_ERR_NO_DEVICE = 3,    /* no usable gfx950 device */
    SELSCAN_ERR_LAUNCH = 4,       /* the HIP runtime refused a launch or an allocation */
    SELSCAN_ERR_WORKSPACE = 5     /* caller workspace smaller than selscan_*_workspace_bytes */
} selscan_status_t;

typedef enum {
    SELSCAN_F32 = 0,   /* IEEE binary32 */
    SELSCAN_BF16 = 1   /* bfloat16 (upper half of a binary32); stores round to nearest even */
} selscan_dtype_t;

/*
 * Mamba-1 problem description.
 *   batch  B >= 1, dim D >= 1 (channels, d_inner), dstate N in {1..16},
 *   1 <= seqlen L < 16777216 (2^24; UNSUPPORTED from 2^24 on).
 *   in_dtype : dtype of u, delta, z, B, C.
 *   out_dtype: dtype of y.
 *   workspace: optional device scratch of at least selscan_workspace_bytes()
 *              bytes, 256-byte aligned.  NULL: the library allocates what it
 *              needs with stream-ordered hipMallocAsync / hipFreeAsync on the
 *              call's stream.
 */
typedef struct {
    int64_t batch, dim, dstate, seqlen;
    int32_t in_dtype;
    int32_t out_dtype;
    void* workspace;
    size_t workspace_bytes;
} selscan_shape_t;

/* Bytes of workspace selscan_fwd needs for `shape` (0 if none). */
size_t selscan_workspace_bytes(const selscan_shape_t* shape);

/*
 * Mamba-1 selective scan (the selective SSM layer of the Mamba README; the
 * update of section 2.2 of the "Understanding Mamba ..." blog).
 *
 *   u          [B, D, L]  in_dtype   input x_t of each channel
 *   delta      [B, D, L]  in_dtype   Delta pre-activation
 *   A          [D, N]     fp32       state matrix diagonal (normally < 0)
 *   B          [B, N, L]  in_dtype   input projection, shared by all channels
 *   C          [B, N, L]  in_dtype   output projection, shared by all channels
 *   D          [D]        fp32       skip weight; NULL = no skip term
 *   z          [B, D, L]  in_dtype   gate; NULL = no silu(z) gating
 *   delta_bias [D]        fp32       added to delta before softplus; NULL = 0
 *   softplus   0 or 1     apply softplus to delta + bias
 *   y          [B, D, L]  out_dtype  output (written)
 *   last_state [B, D, N]  fp32       h after the last token (written); NULL = skip
 *
 * Returns SELSCAN_OK once the work is enqueued.
 */
selscan_status_t selscan_fwd(const selscan_shape_t* shape,
                             const void* u, const void* delta, const float* A,
                             const void* B, const void* C, const float* D,
                             const void* z, const float* delta_bias, int softplus,
                             void* y, float* last_state, void* stream);

/*
 * selscan_fwd from a given initial state instead of zero: the scan continues
 * a sequence whose state after its previous part is h0 (the recurrence of
 * section 2.2 of the "Understanding Mamba ..." blog, resumed; the streaming
 * use on the tutorial and skill pages).
 *   h0 [B, D, N] fp32 device memory, read only; NULL = zero state (then
 *      identical to selscan_fwd).  h0 and last_state must not alias: chunks
 *      of one channel run concurrently.
 * Other arguments, errors and workspace as for selscan_fwd.
 */
selscan_status_t selscan_fwd_h0(const selscan_shape_t* shape,
                                const void* u, const void* delta, const float* A,
                                const void* B, const void* C, const float* D,
                                const void* z, const float* delta_bias, int softplus,
                                const float* h0, void* y, float* last_state, void* stream);

/*
 * selscan_fwd_h0 for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It allocates nothing (no hipMalloc, hipFree or allocating library call):
 * its scratch is a file-scope device array of SELSCAN_NOALLOC_SCRATCH_BYTES
 * (64 MiB) that each GPU the library runs on holds until the process ends.
 *   shape      as for selscan_fwd; its workspace fields are ignored.
 *   other arguments as for selscan_fwd_h0 (h0 NULL = zero state).
 * Errors as for selscan_fwd_h0, plus SELSCAN_ERR_WORKSPACE when the shape
 * needs more scratch than the maximum (selscan_workspace_bytes(shape) >
 * SELSCAN_NOALLOC_SCRATCH_BYTES; e.g. batch 1, dim 2048, L 2^20 needs
 * ~137 MB), before any device work.  Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (concurrent streams without ordering
 * between them) race and must not be issued.  Device ids >= 64 are
 * UNSUPPORTED.
 */
#define SELSCAN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
selscan_status_t selscan_fwd_noalloc(const selscan_shape_t* shape,
                                     const void* u, const void* delta, const float* A,
                                     const void* B, const void* C, const float* D,
                                     const void* z, const float* delta_bias, int softplus,
                                     const float* h0, void* y, float* last_state, void* stream);

/*
 * One-token state update (decoding; the recurrent view of section 2.2 of the
 * "Understanding Mamba ..." blog, one token at a time as the tutorial and
 * skill pages use it for generation).  shape: batch, dim, dstate N (1..16),
 * in_dtype, out_dtype; seqlen, workspace and workspace_bytes are ignored.
 *   state      [B, D, N] fp32  h before the token on entry, after it on
 *                              return (updated in place); 16-byte aligned
 *                              when N is a multiple of 4
 *   u, delta   [B, D]    in_dtype
 *   A          [D, N]    fp32
 *   B, C       [B, N]    in_dtype   this token's projections
 *   D, delta_bias [D]    fp32       NULL = 0
 *   z          [B, D]    in_dtype   NULL = no gate
 *   y          [B, D]    out_dtype  (written)
 * No workspace.  Errors as for selscan_fwd; UNSUPPORTED for N > 16.
 */
selscan_status_t selscan_step(const selscan_shape_t* shape, float* state,
                              const void* u, const void* delta, const float* A,
                              const void* B, const void* C, const float* D,
                              const void* z, const float* delta_bias, int softplus,
                              void* y, void* stream);

/* Bytes of workspace selscan_bwd needs for `shape` (0 on a bad shape). */
size_t selscan_bwd_workspace_bytes(const selscan_shape_t* shape);

/*
 * Gradients of the Mamba-1 scan (training; reverse mode through the
 * recurrence of section 2.2 of the "Understanding Mamba ..." blog, the layer
 * the Mamba README trains end to end).  For out = selscan_fwd_h0(...) and
 * dout = d loss / d out, writes the gradient of the loss with respect to
 * every input.  The states are recomputed from the inputs (nothing from the
 * forward call is needed).
 *   u .. softplus, h0   as for selscan_fwd_h0 (h0 NULL = zero state)
 *   dout        [B, D, L]  out_dtype   gradient of the output
 *   du, ddelta  [B, D, L]  fp32        (written); ddelta is with respect to
 *                                      delta itself (before bias/softplus)
 *   dA          [D, N]     fp32        (written)
 *   dB, dC      [B, N, L]  fp32        (written)
 *   dD          [D]        fp32        (written; NULL = skip; 0 when D is NULL)
 *   dz          [B, D, L]  fp32        (written; required when z is given,
 *                                      ignored otherwise)
 *   ddelta_bias [D]        fp32        (written; NULL = skip)
 *   dh0         [B, D, N]  fp32        (written; NULL = skip)
 * seqlen <= 4194304 (2^22; UNSUPPORTED above).
 * Gradients must not alias inputs or each other.  Sums over channels,
 * batches and time are taken in a fixed order: results are reproducible
 * bit for bit.  shape->workspace as for selscan_fwd, sized by
 * selscan_bwd_workspace_bytes.  Errors as for selscan_fwd, plus
 * SELSCAN_ERR_INVALID_ARG for a NULL required gradient.
 */
selscan_status_t selscan_bwd(const selscan_shape_t* shape,
                             const void* u, const void* delta, const float* A,
                             const void* B, const void* C, const float* D,
                             const void* z, const float* delta_bias, int softplus,
                             const float* h0, const void* dout,
                             float* du, float* ddelta, float* dA, float* dB, float* dC,
                             float* dD, float* dz, float* ddelta_bias, float* dh0,
                             void* stream);

/*
 * Mamba-2 problem description.
 *   batch >= 1, seqlen >= 1, nheads H >= 1, headdim P >= 1, ngroups G >= 1
 *   with H % G == 0, dstate N in {16, 32, 64, 128}.
 *   in_dtype: dtype of x, dt, z, B, C; out_dtype: dtype of y.
 *   workspace: as for selscan_shape_t.
 */
typedef struct {
    int64_t batch, seqlen, nheads, headdim, ngroups, dstate;
    int32_t in_dtype;
    int32_t out_dtype;
    void* workspace;
    size_t workspace_bytes;
} selscan_m2_shape_t;

size_t selscan_mamba2_workspace_bytes(const selscan_m2_shape_t* shape);

/*
 * Mamba-2 multi-head selective scan (the Mamba-2 block of the Mamba README;
 * the "model-architecture-mamba" page's multi-head Mamba-2): a scalar A per
 * head, one Delta per (batch, token, head) shared by the head's P channels,
 * B and C shared by the heads of a group; head h reads group h / (H / G).
 *
 *   x          [B, L, H, P]  in_dtype
 *   dt         [B, L, H]     in_dtype   Delta pre-activation
 *   A          [H]           fp32
 *   B, C       [B, L, G, N]  in_dtype
 *   D          [H]           fp32       NULL = no skip
 *   z          [B, L, H, P]  in_dtype   NULL = no gate
 *   dt_bias    [H]           fp32       NULL = 0
 *   y          [B, L, H, P]  out_dtype  (written)
 *   last_state [B, H, P, N]  fp32       (written); NULL = skip
 *
 * Two forms compute it.  bf16 inputs with P = 64, N in {64, 128} and x, B, C
 * on 16-byte boundaries take the chunked matrix form named in the README's
 * Mamba-2 section (64-token chunks, the products on the matrix cores in bf16
 * with fp32 accumulation; the fp32 operands -- the intra-chunk matrix, the
 * state and the weighted x -- enter as bf16 pairs, relative error near
 * 2^-16, and sums run in another order than the recurrence's); every other
 * shape takes the recurrent form in fp32 (whose chunk carries on long
 * sequences are what selscan_mamba2_workspace_bytes sizes).
 */
selscan_status_t selscan_mamba2_fwd(const selscan_m2_shape_t* shape,
                                    const void* x, const void* dt, const float* A,
                                    const void* B, const void* C, const float* D,
                                    const void* z, const float* dt_bias, int softplus,
                                    void* y, float* last_state, void* stream);

/* selscan_mamba2_fwd from an initial state h0 [B, H, P, N] fp32 (NULL =
 * zero); h0 and last_state must not alias. */
selscan_status_t selscan_mamba2_fwd_h0(const selscan_m2_shape_t* shape,
                                       const void* x, const void* dt, const float* A,
                                       const void* B, const void* C, const float* D,
                                       const void* z, const float* dt_bias, int softplus,
                                       const float* h0, void* y, float* last_state, void* stream);

/* Bytes of workspace selscan_mamba2_bwd needs for `shape` (0 on a bad
 * shape): per (batch, head) the state entering every 8-token tile
 * (64 x N fp32 each, i.e. 4 KiB per token and head at N = 128; the chunked
 * form below uses one state per 32 tokens of this space) and the head's
 * share of dB and dC (2 x L x N fp32).  It grows with batch x seqlen x
 * nheads: 5.4 GB for batch 8, seqlen 4096, 32 heads. */
size_t selscan_mamba2_bwd_workspace_bytes(const selscan_m2_shape_t* shape);

/*
 * Gradients of the Mamba-2 scan (training; reverse mode through the
 * multi-head recurrence of the README's "Mamba-2" section: one scalar decay
 * per token and head, B and C shared by the heads of a group).  For
 * out = selscan_mamba2_fwd_h0(...) and dout = d loss / d out, writes the
 * gradient of the loss with respect to every input; the states are
 * recomputed from the inputs.  bf16 inputs with N >= 32 and 16-byte aligned
 * x, z, dout, B, C take the chunked matrix form (32-token chunks, products
 * on the matrix cores with fp32 operands split into bf16 hi + lo pairs, the
 * state entering each chunk kept in the workspace; the environment variable
 * SELSCAN_M2_BWD_SSD=0 turns it off); other calls take the recurrent form
 * (fp32, the state entering every 8-token tile kept).
 *   x .. softplus, h0   as for selscan_mamba2_fwd_h0 (h0 NULL = zero state)
 *   dout        [B, L, H, P]  out_dtype   gradient of the output
 *   dx          [B, L, H, P]  fp32        (written)
 *   ddt         [B, L, H]     fp32        (written; with respect to dt itself,
 *                                         before bias and softplus)
 *   dA          [H]           fp32        (written)
 *   dB, dC      [B, L, G, N]  fp32        (written; summed over the heads of
 *                                         each group and their channels)
 *   dD          [H]           fp32        (written; NULL = skip; 0 when D is NULL)
 *   dz          [B, L, H, P]  fp32        (written; required when z is given,
 *                                         ignored otherwise)
 *   ddt_bias    [H]           fp32        (written; NULL = skip; 0 when dt_bias
 *                                         is NULL)
 *   dh0         [B, H, P, N]  fp32        (written; NULL = skip)
 * headdim P = 64 only (SELSCAN_ERR_UNSUPPORTED otherwise); N in
 * {16, 32, 64, 128}.  One workgroup per (batch, head) walks the whole
 * sequence: time is not split, so few (batch, head) units leave most of the
 * GPU idle.  Gradients must not alias inputs or each other.  Sums
 * over heads, channels, batches and time run in a fixed order: results are
 * reproducible bit for bit.  shape->workspace as for selscan_mamba2_fwd,
 * sized by selscan_mamba2_bwd_workspace_bytes.  Errors as for
 * selscan_mamba2_fwd, plus SELSCAN_ERR_INVALID_ARG for a NULL required
 * gradient.
 */
selscan_status_t selscan_mamba2_bwd(const selscan_m2_shape_t* shape,
                                    const void* x, const void* dt, const float* A,
                                    const void* B, const void* C, const float* D,
                                    const void* z, const float* dt_bias, int softplus,
                                    const float* h0, const void* dout,
                                    float* dx, float* ddt, float* dA, float* dB, float* dC,
                                    float* dD, float* dz, float* ddt_bias, float* dh0,
                                    void* stream);

/*
 * Mamba-2 one-token update.  shape: batch, nheads H, headdim P, ngroups G,
 * dstate N in {16, 32, 64, 128}, dtypes; seqlen and workspace ignored.
 *   state   [B, H, P, N] fp32  updated in place, 16-byte aligned
 *   x, z    [B, H, P]    in_dtype (z NULL = no gate)
 *   dt      [B, H]       in_dtype
 *   A, D, dt_bias [H]    fp32 (D, dt_bias NULL = 0)
 *   B, C    [B, G, N]    in_dtype
 *   y       [B, H, P]    out_dtype (written)
 */
selscan_status_t selscan_mamba2_step(const selscan_m2_shape_t* shape, float* state,
                                     const void* x, const void* dt, const float* A,
                                     const void* B, const void* C, const float* D,
                                     const void* z, const float* dt_bias, int softplus,
                                     void* y, void* stream);

/*
 * Causal depthwise convolution ahead of the scan (section 3.3 of the
 * "Understanding Mamba ..." blog: a width-4 convolution whose output at a
 * token sees it and the three before it; the README's causal-conv1d layer):
 *   out[b,d,t] = act(bias[d] + sum_{k<K} weight[d,k] x[b,d,t-(K-1)+k]),
 * x before the first token taken as zero, act = silu when silu == 1, else
 * identity.  weight[d, K-1] multiplies the current token.
 *   x       [B, D, L]  in_dtype
 *   weight  [D, K]     fp32
 *   bias    [D]        fp32, NULL = 0
 *   out     [B, D, L]  out_dtype (written; must not alias x)
 * width K in 1..64 (UNSUPPORTED above); no workspace; asynchronous on stream.
 */
typedef struct {
    int64_t batch, dim, seqlen, width;
    int32_t in_dtype, out_dtype;
} selscan_conv_shape_t;

selscan_status_t selscan_conv1d(const selscan_conv_shape_t* shape, const void* x,
                                const float* weight, const float* bias, int silu,
                                void* out, void* stream);

/* Message for the last failed call on this thread ("" after a success).
 * The string stays valid until the next call on the same thread. */
const char* selscan_last_error(void);

/* Library version string, e.g. "libselscan 0.1 gfx950". */
const char* selscan_version(void);

/* ---- Kernel timing (instrumentation for benchmarks) ---------------------
 * selscan_timing_enable(1) makes every later kernel launch of the entry
 * points, on any thread, record a HIP event before and after the kernel on
 * the call's own stream.  selscan_timing_collect waits for all events
 * recorded so far, writes at most max_entries per-kernel aggregates to `out`
 * (host memory owned by the caller; `name` points to a static string of the
 * library) in order of first launch, forgets those events and returns the
 * number of distinct kernels (which may exceed max_entries), or a negative
 * value on a bad argument (-1) or an event failure (-2).  Enabling adds two
 * event records per launch to the stream; leave it off for end-to-end
 * timing.  selscan_timing_enable returns SELSCAN_ERR_INVALID_ARG for values
 * other than 0 and 1. */
typedef struct {
    const char* name;   /* e.g. "m1_scan_output" */
    int64_t launches;
    double total_ms, min_ms, max_ms;
} selscan_kernel_time_t;

selscan_status_t selscan_timing_enable(int on);
int selscan_timing_collect(selscan_kernel_time_t* out, int max_entries);

#ifdef __cplusplus
}
#endif

#endif /* SELSCAN_H */
