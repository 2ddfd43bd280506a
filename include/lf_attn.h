/*
 * lf_attn.h — C ABI of the MI355X (gfx950) Longformer attention layer.
 *
 * The forward pass of Longformer's combined attention layer (lf_attn_forward,
 * lf_attn_forward_lse), its gradients (lf_attn_backward) and the layer's
 * input projections (lf_attn_project).  The forward is a sliding window
 * over a fixed number of diagonals of QK^T (optionally dilated per head,
 * optionally causal) merged with symmetric global
 * attention on a few selected tokens that uses its own Q_g/K_g/V_g
 * projections.  Sources for the definition:
 *   - sliding window, dilation, global attention, separate global
 *     projections, banded QK^T: segmentfault.com Longformer summary,
 *     sections "Sliding window", "Dilated sliding window", "Global
 *     attention", "Linear projections for global attention",
 *     "Implementation";
 *   - 256 tokens per side, inclusive |i-j| <= window/2, global row and
 *     column set in a boolean mask (a set union): ultralytics glossary
 *     "Longformer", section "How Longformer attention works" and its worked
 *     mask-count example;
 *   - mask values 0 = no attention, 1 = local, 2 = global, sequence padded
 *     to a multiple of the window: allenai/longformer README, "Usage".
 *
 * Definition computed, for every batch row b and head h (d = dilation[h],
 * s = scale, D the head dim), with W(i) = { i + k*d : -w <= k <= (causal ? 0 : w),
 * 0 <= i + k*d < n }, Valid = { j : mask[b,j] != 0 }, G = { j : mask[b,j] == 2 }:
 *   mask[b,i] == 1 (local row):  S(i) = (W(i) u G) n Valid,
 *       out[b,i,h] = sum_{j in S(i)} softmax_j(s <q[b,i,h], k[b,j,h]>) v[b,j,h]
 *   mask[b,i] == 2 (global row): S(i) = Valid,
 *       out[b,i,h] = sum_{j in S(i)} softmax_j(s <q_g[b,i,h], k_g[b,j,h]>) v_g[b,j,h]
 *   mask[b,i] == 0 (padding):    out[b,i,h] = 0, S(i) = {}
 *   row_nnz[b,h,i] = |S(i)|.
 * A global key inside a row's window is counted once.  Keys outside S(i)
 * never influence out[b,i,h], whatever values they hold.
 *
 * Conventions of every entry point:
 *   - All tensors are contiguous.  q, k, v, q_g, k_g, v_g and out are
 *     [B, n, H, D] (token-major: element (b,i,h,d) at ((b*n + i)*H + h)*D + d),
 *     of the dtype in the parameters.  mask is int8 [B, n].  row_nnz is
 *     int32 [B, H, n].
 *   - Device pointers are HIP device memory of the current device.  The
 *     caller owns every buffer; the library allocates and frees nothing in
 *     lf_attn_forward and never synchronises the stream there.
 *   - Every argument is validated on the host before any HIP call, so every
 *     error code below is returned without touching the GPU.
 *   - Mask contents are not read on the host.  Under causal = 1 a mask
 *     value 2 acts as 1 (global attention is not defined for the
 *     autoregressive case).  Mask values other than 0/1/2 act as 0.
 */
#ifndef LF_ATTN_H
#define LF_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LF_OK = 0,
  LF_ERR_INVALID_ARG = 1, /* NULL pointer, bad size, bad window/dilation/scale, aliasing */
  LF_ERR_UNSUPPORTED = 2, /* D not a supported head dim, unknown dtype, a size above the limits below */
  LF_ERR_WORKSPACE = 3,   /* workspace missing or smaller than lf_attn_workspace_bytes */
  LF_ERR_HIP = 4          /* the HIP runtime refused the launch */
} lf_status;

/* Element type of q, k, v, q_g, k_g, v_g and out.  Scores, softmax state
 * and P V accumulate in fp32 in every case; the probabilities enter P V in
 * the element type (fp32, bf16 or f16). */
typedef enum { LF_F32 = 0, LF_BF16 = 1, LF_F16 = 2 } lf_dtype;

/* Limits of this build.  The forward takes head dims D = 32, 64 and 128 (a
 * kernel build each).  The pages print no head size: they name the
 * longformer-base and led-base checkpoints (allenai/longformer README,
 * "Usage"; segmentfault summary, the LED models), whose heads are 64 wide,
 * and the window and global pattern never depend on D.  The backward takes
 * D = LF_BWD_HEAD_DIM only. */
#define LF_HEAD_DIM 64       /* the default head dim (longformer-base) */
#define LF_BWD_HEAD_DIM 64
#define LF_MAX_HEADS 64
#define LF_MAX_GLOBAL 1024   /* global tokens per batch row */
#define LF_MAX_SEQ (1 << 24)
#define LF_MAX_ROW_BYTES 0x7fffffff /* n * H * D * element size of one batch row */

/* Bits of the device status word (lf_attn_device_status). */
#define LF_DEV_TOO_MANY_GLOBALS 1 /* a batch row held more than max_global tokens with mask 2 */

typedef struct {
  int32_t B, n, H, D;        /* B, n, H >= 1; D is 32, 64 or 128 */
  int32_t window;            /* one-sided w >= 0; the pages' attention_window is 2w */
  const int32_t* dilation;   /* HOST array [H], each >= 1; NULL means all 1 */
  int32_t causal;            /* 0 or 1 */
  float scale;               /* score scale > 0; 0 means 1/sqrt(D) */
  int32_t max_global;        /* upper bound on mask==2 tokens per batch row, 0..LF_MAX_GLOBAL */
  int32_t dtype;             /* lf_dtype of q, k, v, q_g, k_g, v_g and out */
} lf_attn_params;

/* Bytes of device workspace lf_attn_forward needs for these parameters
 * (status word, per-(b,h) arrival counters, split-sequence partial results
 * of the global rows).  Returns 0 if the parameters are invalid. */
size_t lf_attn_workspace_bytes(const lf_attn_params* p);

/* Zero a freshly allocated workspace on `stream` (a hipStream_t; NULL is
 * the default stream).  Needed once per allocation: every lf_attn_forward
 * leaves the counters it uses back at zero when its kernel completes.
 * Also clears the status word. */
lf_status lf_attn_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Enqueue the forward on `stream` and return.  q_g, k_g, v_g may be NULL,
 * meaning "the same as q, k, v" (the initial state of the global
 * projections), and may alias q, k, v.  out must not overlap any input.
 * row_nnz may be NULL.  out is fully overwritten, and so is row_nnz when
 * given.  workspace must hold lf_attn_workspace_bytes(p) bytes initialised
 * by lf_attn_workspace_init; two calls in flight at once must not share a
 * workspace.  LF_OK means the arguments were valid and the launch was
 * accepted; faults during execution surface at the caller's next
 * synchronisation.  The first call on a device also asks the runtime for
 * that device's compute-unit count and the kernel's occupancy (no
 * allocation, no synchronisation); they set how the global rows are split. */
lf_status lf_attn_forward(const lf_attn_params* p,
                          const void* q, const void* k, const void* v,
                          const void* q_g, const void* k_g, const void* v_g,
                          const int8_t* mask, void* out, int32_t* row_nnz,
                          void* workspace, size_t workspace_bytes, void* stream);

/* lf_attn_forward that also writes lse[b,h,i] (fp32 [B, H, n], caller-owned,
 * must not overlap any other buffer): the natural log of the row's softmax
 * denominator, log sum_{j in S(i)} exp(s <q, k_j>) with the projections of
 * the row's kind, and -inf for mask-0 rows.  It is the row statistic
 * lf_attn_backward takes.  lse must not be NULL. */
lf_status lf_attn_forward_lse(const lf_attn_params* p,
                              const void* q, const void* k, const void* v,
                              const void* q_g, const void* k_g, const void* v_g,
                              const int8_t* mask, void* out, int32_t* row_nnz, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace lf_attn_backward needs (status word, the global
 * token list of each batch row, two fp32 per row: <dout, out> and the row's
 * lse in base 2).  Returns
 * 0 if the parameters are invalid. */
size_t lf_attn_backward_workspace_bytes(const lf_attn_params* p);

/* Enqueue the backward on `stream` and return: the gradients of the forward
 * above with respect to q, k, v, q_g, k_g, v_g for the upstream gradient
 * dout of out.  The pages train the layer (segmentfault Longformer summary,
 * "Training" and "Pre-training"; gittoolsai page, the gradient-checkpointing
 * note) but print no formula for its gradient; what is computed is
 * the chain rule through each row's softmax over S(i):
 *   P_ij = exp(s <q_i, k_j> - lse_i) for j in S(i), D_i = <dout_i, out_i>,
 *   dS_ij = P_ij (<dout_i, v_j> - D_i),
 *   dq_i = s sum_j dS_ij k_j,  dk_j = s sum_i dS_ij q_i,  dv_j = sum_i P_ij dout_i,
 * with (q, k, v) for local rows and (q_g, k_g, v_g) for global rows.
 *   - D must be LF_BWD_HEAD_DIM and dtype LF_BF16 or LF_F16
 *     (LF_ERR_UNSUPPORTED otherwise, and lf_attn_backward_workspace_bytes
 *     returns 0); q..v_g,
 *     out and dout are [B, n, H, D] of that type; out and lse are what
 *     lf_attn_forward_lse wrote for the same inputs and parameters.
 *   - dq, dk, dv, dq_g, dk_g, dv_g are fp32 [B, n, H, D], caller-owned, each
 *     fully overwritten, none overlapping another buffer.  Rows that take no
 *     part get zeros (mask-0 rows and keys; dq of global rows; dq_g of local
 *     rows).  When q_g, k_g, v_g are NULL (aliasing q, k, v), the gradient of
 *     a shared tensor is the sum of its two results.
 *   - workspace holds lf_attn_backward_workspace_bytes(p) bytes; its first
 *     256 bytes are the device status word (lf_attn_workspace_init clears
 *     it, lf_attn_device_status reads it); the rest needs no initialisation.
 *   - A batch row with more than max_global mask-2 tokens sets
 *     LF_DEV_TOO_MANY_GLOBALS in this status word, and that row's gradients
 *     are then incomplete: the tokens past the first max_global get no dk
 *     and dv from the local rows and no global-row work (the forward drops
 *     them likewise and flags its own status word).  Size max_global to the
 *     mask (the Python binding derives it when validating).
 *   - Asynchronous like lf_attn_forward; the same argument errors.  With
 *     global tokens, the global-token work runs on a second stream of the
 *     library (one per device, created at the first such call made outside
 *     graph capture, kept until the process ends, default priority), forked
 *     from `stream` after the preparation and joined back into it before
 *     the call returns, so `stream` orders everything as usual and a graph
 *     captured from `stream` holds both branches.  Concurrent calls on one
 *     device take turns enqueueing on that stream.  While a graph capture
 *     that holds such a call is open, no other thread may make such a call
 *     on the same device (its work would join the capture).  If the second
 *     stream is unavailable, or the first such call is made under capture,
 *     the work runs on `stream`. */
lf_status lf_attn_backward(const lf_attn_params* p,
                           const void* q, const void* k, const void* v,
                           const void* q_g, const void* k_g, const void* v_g,
                           const int8_t* mask, const void* out, const void* dout, const float* lse,
                           float* dq, float* dk, float* dv, float* dq_g, float* dk_g, float* dv_g,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Most projections lf_attn_project computes in one launch. */
#define LF_MAX_PROJ 6

/* Enqueue the layer's input projections on `stream` and return: P stacked
 * linear maps of the hidden states x [M, C] (M = B*n tokens, C = H*D
 * features, token-major, dtype LF_BF16 or LF_F16),
 *   out[p][m][c] = sum_k x[m][k] w[p*C + c][k] + bias[p*C + c],
 * with w [P*C, C] in the [out features, in features] layout and bias fp32
 * [P*C] or NULL.  out is [P, M, C] of the same dtype; each out[p], viewed as
 * [B, n, H, D], is one input of lf_attn_forward.  With P = 6 and the
 * weights stacked as Q_s, K_s, V_s, Q_g, K_g, V_g these are the layer's
 * sliding-window and separate global projections (segmentfault Longformer
 * summary, "Linear projections for global attention"; the global weights
 * start as copies of the local ones).  fp32 accumulation, the bias added in
 * fp32, the result rounded to nearest even.  Errors: LF_ERR_INVALID_ARG for
 * M, C or P < 1, a NULL x, w or out, or out overlapping an input;
 * LF_ERR_UNSUPPORTED for another dtype, C not a multiple of 64, P > 6, x or
 * w larger than 2^31 - 1 bytes, or x, w, out or bias not 16-byte aligned.
 * Allocates nothing, needs no workspace. */
lf_status lf_attn_project(int32_t M, int32_t C, int32_t P, int32_t dtype,
                          const void* x, const void* w, const float* bias, void* out, void* stream);

/* lf_attn_project with some of the P projections needed at the global
 * tokens only.  The separate global projections score global attention
 * (segmentfault Longformer summary, "Linear projections for global
 * attention"): of them Q_g enters only the rows of global tokens, while
 * K_g and V_g are read at every token.  For each set bit p of global_only,
 * out[p][m] is computed as in lf_attn_project where mask[m] == 2 and is
 * written as zero at every other token m; the other projections are exactly
 * those of lf_attn_project.  mask: int8 [M], the attention's [B, n] mask
 * (M = B*n, token-major), read on the device only; tiles of global-only
 * features with no global token skip their reduction.  With the weights
 * stacked Q_s, K_s, V_s, Q_g, K_g, V_g, global_only = 1 << 3 gives the
 * attention all it reads.  Errors: those of lf_attn_project, and
 * LF_ERR_INVALID_ARG for a bit at p >= P, a NULL mask with global_only != 0,
 * or out overlapping the mask. */
lf_status lf_attn_project_global_only(int32_t M, int32_t C, int32_t P, int32_t dtype, const void* x,
                                      const void* w, const float* bias, const int8_t* mask,
                                      uint32_t global_only, void* out, void* stream);

/* Size of the device scratch that lf_attn_forward_noalloc uses instead of a
 * workspace (one copy per device, held until the process ends). */
#define LF_NOALLOC_SCRATCH_BYTES (8u << 20)

/* lf_attn_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and outputs without the workspace, which
 * lives in a static device array of this library instead.  Allocates and
 * frees nothing.  Each call enqueues a small clearing kernel and then the
 * forward on `stream`.  Every call on one GPU shares that GPU's scratch:
 * calls that overlap in time on one GPU (other streams, other threads) race
 * and must be ordered by the caller.  Returns LF_ERR_WORKSPACE when
 * lf_attn_workspace_bytes(p) exceeds LF_NOALLOC_SCRATCH_BYTES (the global
 * rows' partial records grow with B * H * max_global * ceil(n / 512)), and
 * otherwise the errors of lf_attn_forward.  The too-many-globals condition
 * is not reported by this variant: size max_global to the mask. */
lf_status lf_attn_forward_noalloc(const lf_attn_params* p,
                                  const void* q, const void* k, const void* v,
                                  const void* q_g, const void* k_g, const void* v_g,
                                  const int8_t* mask, void* out, int32_t* row_nnz, void* stream);

/* Debug helper: synchronise `stream`, then read the device status word of
 * `workspace` into *status (LF_DEV_* bits; 0 = no condition seen). */
lf_status lf_attn_device_status(const void* workspace, void* stream, int32_t* status);

/* Static description of a status code. */
const char* lf_status_str(int32_t s);

#ifdef __cplusplus
}
#endif

#endif /* LF_ATTN_H */
