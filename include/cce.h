/*
 * cce.h -- C ABI of libcce, the MI355X (gfx950) flash cut-cross-entropy head.
 *
 * The operation (page "mlx-bun 0.0.4 -> 0.0.6", src/train/flash-cce.ts, header
 * comment and flashCceForward / flashCceBackward): for hidden states h [M, H]
 * and a frozen affine-quantized LM head W [V, H], compute per token
 *
 *     y_v   = c(h_t . W_v),  c(z) = cap * tanh(z / cap) if cap > 0 else z
 *     lse_t = log sum_v exp(y_v)
 *     logp_t = y_{target_t} - lse_t
 *
 * and, for an upstream cotangent g_t = d loss / d logp_t, the gradient
 *
 *     dh_t = g_t * d logp_t / d h_t
 *          = g_t * sum_v (1[v = target_t] - exp(y_v - lse_t)) * c'(z_v) * W_v
 *
 * The [M, V] logits and a dequantized head are never written to memory.  The
 * coefficients g * (1[v = target] - exp(y - lse)) * c' are: the backward stages
 * them in bf16 in the caller's workspace one vocabulary chunk at a time (at
 * most 1 GiB per chunk; 4 chunks of 8192 x 65536 at M = 8192, V = 262144).
 *
 * Conventions shared by every call:
 *  - Pointers named "device" are HIP device (or managed) memory on the current
 *    device; the caller allocates and owns every buffer.  The library keeps no
 *    pointer after a call returns and never allocates device memory.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  Buffers must stay valid until the stream has passed the work.
 *    Nothing synchronizes with the host.  A call only enqueues kernels (no
 *    allocation, memset or host synchronization), so it can be captured in a
 *    HIP graph and replayed with the same buffers.
 *  - The library holds no state; calls on different streams are independent
 *    provided each has its own workspace.  Two calls in flight that share a
 *    workspace race.
 *  - On any error return nothing has been enqueued and no output written,
 *    except CCE_ERR_HIP, which is reported after a failed launch.
 *  - Masked tokens (mask[t] == 0) get logp = lse = 0 and a zero dh row.
 *  - A target outside [0, V) matches no vocabulary row: its target term is 0
 *    (logp = -lse) and it adds no one-hot term to dh.
 */
#ifndef LIBCCE_CCE_H
#define LIBCCE_CCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CCE_ABI_VERSION 8

/* Vocabulary rows per block of block_max, and supervised tokens per token
 * tile of the backward skips (both are the kernels' tile sizes). */
#define CCE_BLOCK_V 256
#define CCE_TOKEN_TILE 256

typedef enum cce_status {
  CCE_OK = 0,
  CCE_ERR_INVALID_ARG = 1, /* null pointer, negative size, H % group != 0,
                              softcap < 0 or not finite, misaligned pointer */
  CCE_ERR_UNSUPPORTED = 2, /* bits not 4 or 8, group not 32/64/128, scale
                              dtype unknown, H or V too large */
  CCE_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than required */
  CCE_ERR_HIP = 4          /* a HIP launch failed; see cce_status_str */
} cce_status;

/* Storage type of the per-group scales and biases. */
typedef enum cce_sb_dtype {
  CCE_SB_F32 = 0,
  CCE_SB_BF16 = 1,
  CCE_SB_F16 = 2
} cce_sb_dtype;

/*
 * The frozen quantized head (page "mlx-bun 0.0.4 -> 0.0.6",
 * src/train/flash-cce.ts, the FlashCceHead interface; packing as read by the
 * forward kernels there).  All pointers are device memory, row-major:
 *   wq      uint32 [V][H*bits/32]; element d of row v is the unsigned code
 *           (wq[v][d / (32/bits)] >> (bits * (d % (32/bits)))) & (2^bits - 1),
 *           i.e. little-endian within each word.  16-byte aligned.
 *   scales  [V][H/group] of sb_dtype (aligned to its size)
 *   biases  [V][H/group] of sb_dtype (aligned to its size)
 * The dequantized element is w[v][d] = scales[v][d/group] * q + biases[v][d/group],
 * with the stored scale and bias widened exactly to fp32.
 *   bits    4 or 8;  group  32, 64 or 128 (the group sizes of MLX's affine
 *           quantizer, which the page's kernels accept);  H a multiple of
 *           group and of 64, at most 16384;  V in [1, 2^31 - 1];
 *   softcap >= 0 (0 = no softcap);
 *   sb_dtype  CCE_SB_F32 (what the page's host casts to), CCE_SB_BF16 or
 *           CCE_SB_F16 (the model-dtype storage of MLX heads, read as is).
 */
typedef struct cce_head {
  const uint32_t *wq;
  const void *scales;
  const void *biases;
  int64_t V;
  int64_t H;
  int32_t bits;
  int32_t group;
  float softcap;
  int32_t sb_dtype;
  /* Optional: the head's preparation, or NULL.  Every call first derives
   * per-row data from the scales and biases (the fold ratios s_{g-1} / s_g,
   * the last scale, the fixed-point digits of b + z s and their block
   * maxima).  A frozen head can have that written once by cce_head_prepare
   * into a device buffer of prep_bytes (256-byte aligned); a call given it
   * skips that work and needs a smaller workspace.  The caller keeps it in
   * step with wq, scales and biases (the library cannot tell). */
  const void *prep;
  size_t prep_bytes;
} cce_head;

/*
 * The head is frozen while the caller trains (page "mlx-bun 0.0.4 -> 0.0.6",
 * src/train/flash-cce.ts, the FlashCceHead interface), so its preparation can
 * be made once for many calls.  Bytes of the prepared buffer for this head
 * (its prep fields ignored), 0 when the head is invalid.  Depends on V, H,
 * bits and group only.
 */
size_t cce_head_prepare_bytes(const cce_head *head);

/*
 * Writes the head's preparation into `prep` (device, 256-byte aligned, at
 * least cce_head_prepare_bytes), asynchronously on `stream`; the head's own
 * prep fields are ignored.  Set head->prep / prep_bytes to it for later calls.
 * Errors: those of the head (CCE_ERR_INVALID_ARG, CCE_ERR_UNSUPPORTED),
 * CCE_ERR_INVALID_ARG for a NULL or misaligned prep, CCE_ERR_WORKSPACE when
 * prep_bytes is too small, CCE_ERR_HIP after a failed launch.
 */
cce_status cce_head_prepare(const cce_head *head, void *prep, size_t prep_bytes, void *stream);

/*
 * Bytes of device workspace that cce_forward / cce_backward need for this head
 * and M tokens.  Returns 0 when the head or M is invalid (cce_forward then
 * reports why).  The value depends only on (V, H, bits, group, M, whether
 * head->prep is set) and the compute unit count of the current device (the
 * launch plan fills whole rounds).
 */
size_t cce_forward_workspace_bytes(const cce_head *head, int64_t M);
size_t cce_backward_workspace_bytes(const cce_head *head, int64_t M);

/*
 * Forward (page "mlx-bun 0.0.4 -> 0.0.6", src/train/flash-cce.ts,
 * flashCceForward: vocab-parallel online-softmax partials merged across vocab
 * blocks into lse, then logp = target logit - lse).
 *   h          device bf16 [M][H] row-major (raw bf16 bits, 16-byte aligned)
 *   targets    device int32 [M]
 *   mask       device uint8 [M] (nonzero = supervised token) or NULL = all
 *   logp, lse  device float [M], written for every token
 *   workspace  device, 256-byte aligned, >= cce_forward_workspace_bytes
 */
cce_status cce_forward(const cce_head *head, const void *h, int64_t M,
                       const int32_t *targets, const uint8_t *mask,
                       float *logp, float *lse, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * Backward (same file, flashCceBackward: recompute the logits, form the
 * coefficient g * (onehot - softmax) * c', contract it with W, summing over
 * vocabulary blocks).
 *   lse        device float [M], as written by cce_forward for these inputs
 *   g          device float [M] cotangent of logp, or NULL = all ones
 *              (for a loss of -sum_t logp_t pass g = -1)
 *   dh         device float [M][H], fully overwritten
 *   workspace  device, 256-byte aligned, >= cce_backward_workspace_bytes
 * Other arguments as for cce_forward.
 */
cce_status cce_backward(const cce_head *head, const void *h, int64_t M,
                        const int32_t *targets, const uint8_t *mask,
                        const float *lse, const float *g, float *dh,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * Forward that also writes the per-block maxima the backward's block skip
 * reads (page "mlx-bun 0.0.4 -> 0.0.6", src/train/flash-cce.ts, the notes on
 * the blockMax vocabulary-block early exit of the backward).
 *   block_max  device float [M][ceil(V / CCE_BLOCK_V)] (4-byte aligned) or
 *              NULL, which makes the call cce_forward.  block_max[t][b] is the
 *              largest softcapped logit y_v over the rows v in
 *              [CCE_BLOCK_V*b, min(V, CCE_BLOCK_V*(b+1))); rows of masked
 *              tokens are 0.
 * Other arguments, the workspace size and the errors are those of cce_forward.
 */
cce_status cce_forward_ex(const cce_head *head, const void *h, int64_t M,
                          const int32_t *targets, const uint8_t *mask,
                          float *logp, float *lse, float *block_max,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Opt-in approximations of the backward (same file: the coefficient filter
 * and the block early exit of the backward kernels; both default to off).
 * Token tiles are runs of CCE_TOKEN_TILE consecutive supervised tokens (in
 * index order), vocabulary blocks those of block_max.  For a (token tile,
 * block) pair:
 *   block_eps   > 0: the pair is left out when, for every token of the tile,
 *               block_max - lse < log(block_eps) (its largest probability in
 *               the block is below block_eps) and its target is outside the
 *               block.  Needs block_max.
 *   filter_eps  > 0: the pair is left out when every non-target coefficient
 *               g * p_v * c'(z_v) in it is below filter_eps in magnitude.
 * "Left out" drops the pair's non-target coefficients; every target's term
 * g * (1 - p) * c' * w_target is always kept.  0 turns a skip off; both on:
 * the block rule first, then the filter on the pairs that remain.
 */
typedef struct cce_skip {
  float block_eps;
  float filter_eps;
} cce_skip;

/* Element type of the dh written by cce_backward_ex. */
typedef enum cce_dh_dtype {
  CCE_DH_F32 = 0,
  CCE_DH_BF16 = 1 /* the fp32 sum rounded to nearest, ties to even */
} cce_dh_dtype;

/*
 * Backward with the skips of `skip` (NULL or both eps 0: exactly cce_backward)
 * and a choice of output type (the page's training loop keeps dh in the
 * model's dtype; this saves the caller a conversion pass).
 *   block_max  as written by cce_forward_ex for these inputs; needed (non-NULL)
 *              when skip->block_eps > 0, else ignored
 *   dh         device [M][H] of dh_dtype (aligned to its size), fully
 *              overwritten; every element is the fp32 value cce_backward
 *              would write, rounded once when dh_dtype is CCE_DH_BF16
 * Other arguments and the workspace size are those of cce_backward.  Errors
 * as cce_backward, plus CCE_ERR_INVALID_ARG for a negative or non-finite eps,
 * block_eps > 0 without block_max, or an unknown dh_dtype.
 */
cce_status cce_backward_ex(const cce_head *head, const void *h, int64_t M,
                           const int32_t *targets, const uint8_t *mask,
                           const float *lse, const float *g,
                           const float *block_max, const cce_skip *skip,
                           void *dh, int32_t dh_dtype, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * Forward and backward in one call, for a caller that has g before the
 * forward (a loss linear in logp, e.g. g = -1/N for the mean cross entropy),
 * or that wants d logp_t / d h_t itself (g = NULL) and scales it by its g
 * later: dh is linear in g, row by row.  Same operation as cce_forward
 * followed by cce_backward (page "mlx-bun 0.0.4 -> 0.0.6",
 * src/train/flash-cce.ts, flashCceForward and flashCceBackward), outputs as
 * there: logp, lse [M] and dh [M][H] of dh_dtype.
 *
 * With a softcap in (0, 40] the logits are computed once: the forward sums
 * e^{y - cap} against the fixed reference cap (every term <= 1, the largest
 * one >= e^{-2 cap}), and the same epilogue writes every coefficient up to
 * the token's factor g e^{cap - lse}, which the split reduce applies once
 * lse is known.  Other heads run the forward, then the backward, in this call.
 *   workspace  device, 256-byte aligned, >= cce_forward_backward_workspace_bytes
 * Errors as cce_forward and cce_backward_ex.
 */
size_t cce_forward_backward_workspace_bytes(const cce_head *head, int64_t M);
cce_status cce_forward_backward(const cce_head *head, const void *h, int64_t M,
                                const int32_t *targets, const uint8_t *mask,
                                const float *g, float *logp, float *lse,
                                void *dh, int32_t dh_dtype, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * Trainable dense head (the original cut-cross-entropy setting, which the
 * page's frozen quantized head specializes; same page, the note that the head
 * is frozen so no weight gradient is formed).  Same operation as above with
 * W a bf16 matrix, plus the weight gradient
 *
 *     dW_v = sum_t g_t * (1[v = target_t] - exp(y_v - lse_t)) * c'(z_v) * h_t
 *
 *   w        device bf16 [V][H] row-major (raw bf16 bits), 16-byte aligned;
 *            H a multiple of 64, at most 16384;  V in [1, 2^31 - 257]
 *   softcap  as cce_head.softcap
 */
typedef struct cce_dense_head {
  const void *w;
  int64_t V;
  int64_t H;
  float softcap;
} cce_dense_head;

size_t cce_dense_forward_workspace_bytes(const cce_dense_head *head, int64_t M);
size_t cce_dense_backward_workspace_bytes(const cce_dense_head *head, int64_t M);

/* Forward on a dense head: arguments, outputs and errors as cce_forward. */
cce_status cce_dense_forward(const cce_dense_head *head, const void *h, int64_t M,
                             const int32_t *targets, const uint8_t *mask,
                             float *logp, float *lse, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * Backward on a dense head: dh as cce_backward, and
 *   dw   device float [V][H] (4-byte aligned), fully overwritten with dW, or
 *        NULL to skip it.  Every coefficient, the target's included, enters
 *        dW rounded to bf16 (dh adds the target's term in fp32).  Needs
 *        M <= 2^21; larger M with dw is CCE_ERR_UNSUPPORTED.  M = 0 enqueues
 *        nothing and leaves dw untouched.
 * Errors as cce_backward.
 */
cce_status cce_dense_backward(const cce_dense_head *head, const void *h, int64_t M,
                              const int32_t *targets, const uint8_t *mask,
                              const float *lse, const float *g, float *dh, float *dw,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * Forward and backward of a dense head in one call (the two passes of page
 * "mlx-bun 0.0.4 -> 0.0.6", src/train/flash-cce.ts, flashCceForward and
 * flashCceBackward, with g known up front).  Outputs: logp and lse as
 * cce_dense_forward, dh (fp32) and dw as cce_dense_backward, with g as there
 * (NULL = all ones).  With 0 < softcap <= 40 the logits are computed once:
 * the forward's fixed reference e^{y - cap} gives each coefficient up to the
 * token's factor g e^{cap - lse}, every coefficient chunk is kept until lse is
 * known, and dW is formed from them last; the workspace then holds all the
 * chunks (about 2 M V bytes).  Without a softcap likewise, the coefficients
 * taken against each 32-row vocabulary block's largest logit and brought to
 * the token's largest one before the dh and dW contractions (as
 * cce_forward_backward does for a quantized head).  Softcaps above 40 run
 * cce_dense_forward and then cce_dense_backward on the same workspace.  dW
 * takes every coefficient rounded to bf16 and, in the single pass, each h row
 * times its factor rounded to bf16.  Errors as cce_dense_backward.
 */
size_t cce_dense_forward_backward_workspace_bytes(const cce_dense_head *head, int64_t M);
cce_status cce_dense_forward_backward(const cce_dense_head *head, const void *h, int64_t M,
                                      const int32_t *targets, const uint8_t *mask,
                                      const float *g, float *logp, float *lse, float *dh,
                                      float *dw, void *workspace, size_t workspace_bytes,
                                      void *stream);

/*
 * The forward without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  The library's own buffer of CCE_STATIC_SCRATCH_BYTES per
 * device (a file-scope device array, held by every device the library runs
 * on until the process ends) serves as the workspace; the caller still passes
 * inputs and outputs, as for cce_forward.  Every call on one device shares
 * that device's buffer: calls that overlap on one device (other streams,
 * other threads) race, and must be ordered by the caller.  The buffer keeps
 * the last call's contents; nothing in it needs to start at zero.
 * Arguments, results and errors are those of cce_forward, plus
 * CCE_ERR_WORKSPACE when cce_forward_workspace_bytes(head, M) exceeds
 * CCE_STATIC_SCRATCH_BYTES and CCE_ERR_HIP when the buffer's device address
 * cannot be found.
 */
#define CCE_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
cce_status cce_forward_static(const cce_head *head, const void *h, int64_t M,
                              const int32_t *targets, const uint8_t *mask,
                              float *logp, float *lse, void *stream);

/* Human-readable text of a status (for CCE_ERR_HIP, of the last HIP error
 * seen by this thread).  The pointer stays valid until the thread's next call. */
const char *cce_status_str(cce_status status);

/* CCE_ABI_VERSION of the loaded library. */
int cce_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBCCE_CCE_H */
