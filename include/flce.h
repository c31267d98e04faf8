/*
 * flce.h -- fused linear cross-entropy for AMD MI355X (gfx950), C ABI.
 *
 * The operation (fused-linear-ce README, "Usage" and "Algorithm"; quack-kernels
 * 0.2.0 quack/linear_cross_entropy.py, linear_cross_entropy_func_ref):
 *
 *   u_ij = sum_k hidden_ik * weight_jk + bias_j          (bias optional)
 *   z_ij = softcap(logit_scale * u_ij)                   softcap(v) = cap*tanh(v/cap), off if cap <= 0
 *   LSE_i = log sum_j exp(z_ij)
 *   loss_i = LSE_i - z_{i,t_i} + z_loss * LSE_i^2        for rows with t_i != ignore_index, else 0
 *   loss = loss_i (none) | sum_i loss_i (sum) | sum_i loss_i / n_valid (mean)
 *
 * The (N, V) logits are never written to device memory: the forward pass tiles
 * the vocabulary and merges each logit tile into a running log-sum-exp, and the
 * backward pass recomputes the tiles ("Algorithm" section of the README).  The
 * z-loss term follows the z_loss_multiplier option of the greyhound "Chunked
 * Linear Cross-Entropy" page ("Usage"); "mean" is one global mean over valid
 * tokens ("Chunked Linear Loss", "Reduction semantics").
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers, row-major and contiguous, 16-byte
 *    aligned.  hidden is (N, H), weight (V, H), bias (V) or NULL, targets (N)
 *    int64, or int32 with FLCE_TARGETS_INT32.  Floating inputs are all of
 *    params->dtype: fp32, bf16 or fp16 (fused-linear-ce README, "Usage": the
 *    signature's hidden/weight dtypes; quack's linear_cross_entropy_func takes
 *    int or long targets).
 *  - The caller owns every buffer, including the workspace, which it sizes with
 *    flce_workspace_size.  The library allocates no device memory and keeps no
 *    mutable global state; calls on different streams with different
 *    workspaces may run concurrently.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = default stream).
 *    flce_forward and flce_backward never synchronise the host.
 *  - Every output is overwritten, except grad_weight / grad_bias when
 *    params->flags asks the backward pass to accumulate into them.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    non-zero status means nothing was launched.
 *  - Results are deterministic: the same inputs give the same bits, run to run.
 */
#ifndef FLCE_H
#define FLCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FLCE_OK = 0,
  FLCE_ERR_INVALID_ARG = -1,          /* NULL required pointer, negative size, bad enum      */
  FLCE_ERR_UNSUPPORTED = -2,          /* H % 8 != 0, misaligned pointer, or too large: the
                                         kernels use 32-bit offsets, so N*H*elem and the
                                         backward's (vocabulary chunk, <= 32768 rows) x H
                                         and N x chunk must stay under 2^31 bytes, N and V
                                         under 2^30, H under 2^20                             */
  FLCE_ERR_WORKSPACE_TOO_SMALL = -3,
  FLCE_ERR_HIP = -4,                  /* a HIP runtime call failed                           */
  FLCE_ERR_TARGET_OUT_OF_RANGE = -5,  /* reported by flce_get_status only                    */
  FLCE_ERR_CALLBACK = -6              /* a chunk loss function returned non-zero             */
} flce_status;

typedef enum { FLCE_F32 = 0, FLCE_BF16 = 1, FLCE_F16 = 2 } flce_dtype;

typedef enum {
  FLCE_REDUCTION_NONE = 0,
  FLCE_REDUCTION_SUM = 1,
  FLCE_REDUCTION_MEAN = 2
} flce_reduction;

typedef enum { FLCE_PASS_FORWARD = 0, FLCE_PASS_BACKWARD = 1 } flce_pass;

/* flce_params.flags.
 * FLCE_ACCUMULATE_GRAD_WEIGHT / _BIAS (backward): add the result to what the
 * output buffer already holds instead of overwriting it, e.g. to accumulate
 * the weight gradient over micro-batches without a separate add ("Chunked
 * Linear Loss" page, "Weight-gradient accumulation dtype": accumulate in the
 * weight dtype, or in fp32 with grad_weight_dtype = FLCE_F32).  The sum is
 * formed in fp32 and rounded once to the buffer's dtype.
 * FLCE_TARGETS_INT32 (both passes): `targets` points to int32 values.
 * FLCE_GRAD_WEIGHT_ACCUM_IN_OUTPUT (flce_forward_backward): sum grad_weight
 * over the row blocks in grad_weight's own dtype, rounding after every block,
 * instead of in an fp32 workspace accumulator rounded once ("Chunked Linear
 * Cross-Entropy" page, "Usage": grad_weight_accum_dtype="weight"; "Chunked
 * Linear Loss" page, "Weight-gradient accumulation dtype": less memory and
 * faster, rounds between chunks).  No effect when grad_weight is fp32 or the
 * call has one block, nor on flce_backward, which writes each grad_weight row
 * once. */
typedef enum {
  FLCE_ACCUMULATE_GRAD_WEIGHT = 1,
  FLCE_ACCUMULATE_GRAD_BIAS = 2,
  FLCE_TARGETS_INT32 = 4,
  FLCE_GRAD_WEIGHT_ACCUM_IN_OUTPUT = 8
} flce_flags;

typedef struct {
  int64_t n_tokens;           /* N >= 0 (N = 0 is an empty batch)                        */
  int64_t hidden;             /* H >= 8, H % 8 == 0                                      */
  int64_t vocab;              /* V >= 1                                                  */
  int64_t ignore_index;       /* rows whose target equals this are ignored (-100)       */
  int32_t dtype;              /* flce_dtype of hidden, weight and bias                   */
  int32_t grad_weight_dtype;  /* flce_dtype of grad_weight; accumulated in fp32 always   */
  int32_t reduction;          /* flce_reduction                                          */
  int32_t flags;              /* flce_flags bits; 0 = int64 targets, overwrite outputs   */
  float logit_scale;          /* multiplies (x.W^T + b); 1.0 = off                       */
  float softcap;              /* cap of cap*tanh(v/cap); <= 0 = off                      */
  float z_loss;               /* z-loss multiplier lambda >= 0; 0 = off                  */
  float reserved_f;           /* must be 0                                               */
  int64_t vocab_chunk;        /* flce_backward: at most this many vocabulary rows per
                                 chunk of the logit gradient scratch (N x chunk in the
                                 input dtype; the chunks are balanced over the
                                 vocabulary), a multiple of 256, or 0 for the
                                 library's choice; the
                                 chunk trades scratch size (which decides whether it
                                 stays in the last-level cache) against one more fp32
                                 pass over grad_hidden per chunk ("Chunked Linear Loss",
                                 "Chunk size")                                          */
} flce_params;

/* Bytes of device workspace one call of `pass` needs (flce_pass).  Host only. */
int flce_workspace_size(const flce_params* p, int pass, size_t* bytes);

/*
 * Forward pass.
 *  loss:        device fp32, 1 element (sum, mean) or N (none).  Required.
 *               mean with no valid row gives NaN.
 *  lse:         device fp32 (N), the per-row log-sum-exp of z, every row
 *               (ignored rows included).  Required: the backward pass needs it.
 *  num_correct: device int64 scalar, #valid rows with argmax_j z_ij == t_i
 *               (ties -> lowest index), or NULL.   (README, "Metrics for free")
 *  entropy_sum: device fp32 scalar, sum over valid rows of the softmax entropy
 *               of z in nats, or NULL.
 * The metrics are always carried through the vocabulary sweep; asking for them
 * leaves loss and lse bit-identical.
 * A valid target outside [0, V) is treated as ignored and flags the workspace
 * status word (see flce_get_status).
 */
int flce_forward(const flce_params* p, const void* hidden, const void* weight, const void* bias,
                 const void* targets, float* loss, float* lse, int64_t* num_correct,
                 float* entropy_sum, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass: gradients of  sum_i g_i * loss_i  (none) or  g * loss  (sum, mean),
 * recomputing the logit tiles (README, "Algorithm").
 *  lse:         device fp32 (N) from flce_forward with the same inputs.
 *  grad_loss:   device fp32, 1 element (sum, mean) or N (none).
 *  grad_hidden: device (N, H) in params->dtype.  Required.
 *  grad_weight: device (V, H) in params->grad_weight_dtype, accumulated in fp32.  Required.
 *  grad_bias:   device (V) in params->dtype, or NULL; must be NULL when bias is NULL.
 * Rows whose target is ignored (or out of range) get zero gradient.
 * The logit gradient feeding the two contractions is held in the input dtype;
 * for fp16 it is scaled by a power of two chosen per call (so that the small
 * probabilities of a large vocabulary stay in fp16's normal range) and the
 * factor is divided out exactly in fp32.
 */
int flce_backward(const flce_params* p, const void* hidden, const void* weight, const void* bias,
                  const void* targets, const float* lse, const float* grad_loss,
                  void* grad_hidden, void* grad_weight, void* grad_bias, void* workspace,
                  size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * One-pass forward + backward (the row-chunked schedule of the "Chunked Linear
 * Cross-Entropy" page, "Kernel design", and of quack-kernels'
 * chunked_linear_cross_entropy: the gradients are formed while the logits of a
 * block of rows exist, instead of recomputing them in a later backward call).
 * For callers that know the upstream gradient before the forward pass (the
 * loss is the last node: grad_loss = 1, or a loss scale).
 * ------------------------------------------------------------------------- */

/* Bytes of device workspace flce_forward_backward needs.  block_rows: rows per
 * block, a multiple of 256, or 0 for the library's choice (the most rows whose
 * logits, block_rows x V in the input dtype, fit in 1 GiB).  Host only. */
int flce_forward_backward_workspace_size(const flce_params* p, int64_t block_rows, size_t* bytes);

/*
 * The outputs of flce_forward followed by flce_backward with the same
 * grad_loss, in one call: loss, lse, num_correct, entropy_sum (as flce_forward)
 * and grad_hidden, grad_weight, grad_bias (as flce_backward; grad_loss is a
 * device fp32 scalar for sum / mean, N values for none).  Per block of rows the
 * logit tiles are computed once and written to the workspace in the input
 * dtype; loss, LSE and metrics come from their fp32 values, the logit gradient
 * from the stored ones (as the pages' chunked paths keep logits in the logits
 * dtype), so results agree with the two-call path to rounding, not bitwise.
 * grad_weight is summed over the blocks in fp32 and rounded once.  Costs
 * 3 x 2NHV flop instead of 4 x 2NHV.  Argument rules, flags and status codes
 * are those of flce_forward and flce_backward.
 */
int flce_forward_backward(const flce_params* p, int64_t block_rows, const void* hidden, const void* weight,
                          const void* bias, const void* targets, const float* grad_loss, float* loss, float* lse,
                          int64_t* num_correct, float* entropy_sum, void* grad_hidden, void* grad_weight,
                          void* grad_bias, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Multiplies the gradients flce_forward_backward wrote, in place, by the device
 * fp32 scalar g: the upstream gradient of a "sum" or "mean" loss that arrives
 * after the call (which then ran with grad_loss = 1), as the chunked pages do it
 * ("Chunked Linear Loss" page, "Gradient handling": gradients precomputed in
 * the forward pass, scaled by the upstream scalar in the backward).
 * grad_hidden (N x H, params->dtype), grad_weight (V x H,
 * params->grad_weight_dtype), grad_bias (V, params->dtype) or NULL; each
 * element is rounded once more to its dtype.  g == 1 changes nothing.  Not for
 * "none" (the per-row upstream gradient must go into flce_forward_backward).
 */
int flce_scale_gradients(const flce_params* p, const float* g, void* grad_hidden, void* grad_weight,
                         void* grad_bias, void* stream);

/* ---------------------------------------------------------------------------
 * Launch timing, for benchmarks and profilers: flce_forward_timed and
 * flce_backward_timed are flce_forward and flce_backward that also record a pair
 * of caller-owned HIP events on `stream` right before and right after each
 * launch of a matrix-core kernel, so that one kernel's time can be read inside
 * a call that launches several.  The events never change what is computed.
 * ------------------------------------------------------------------------- */
typedef enum {
  FLCE_KERNEL_FORWARD_TILES = 1,    /* logit tiles + online softmax (flce_forward)              */
  FLCE_KERNEL_DLOGITS = 2,          /* recomputed tiles -> logit gradient of a vocabulary chunk */
  FLCE_KERNEL_GRAD_WEIGHT = 3,      /* grad_weight contraction of a chunk                       */
  FLCE_KERNEL_GRAD_HIDDEN = 4       /* grad_hidden contraction of a chunk                       */
} flce_kernel;

typedef struct {
  void* const* events;   /* 2 * capacity hipEvent_t, created by the caller: pair k is
                            events[2k] (before the launch) and events[2k+1] (after)   */
  int32_t* kernel;       /* capacity entries; receives the flce_kernel of each pair    */
  int32_t capacity;      /* pairs available                                             */
  int32_t count;         /* in: pairs already used (a call appends after them);
                            out: pairs used.  Launches past capacity are not timed.   */
} flce_launch_timer;

/* As flce_forward / flce_backward; `timer` may be NULL (no events).  A failed
 * event record returns FLCE_ERR_HIP. */
int flce_forward_timed(const flce_params* p, const void* hidden, const void* weight, const void* bias,
                       const void* targets, float* loss, float* lse, int64_t* num_correct, float* entropy_sum,
                       void* workspace, size_t workspace_bytes, void* stream, flce_launch_timer* timer);
int flce_backward_timed(const flce_params* p, const void* hidden, const void* weight, const void* bias,
                        const void* targets, const float* lse, const float* grad_loss, void* grad_hidden,
                        void* grad_weight, void* grad_bias, void* workspace, size_t workspace_bytes, void* stream,
                        flce_launch_timer* timer);

/*
 * flce_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments as flce_forward without the workspace, same kernels and results.
 * The scratch flce_forward keeps in its workspace (status word, per-split
 * softmax partials, per-block sums) lives in a fixed 8 MiB device array inside
 * the library, one copy per GPU, held until the process ends; the call itself
 * allocates nothing.  Limit: problems whose forward workspace
 * (flce_workspace_size, FLCE_PASS_FORWARD) exceeds 8 MiB -- roughly N above
 * 400k tokens -- return FLCE_ERR_UNSUPPORTED before anything is enqueued.
 * `stream` must belong to the current device (else FLCE_ERR_INVALID_ARG).
 * Every call on a GPU uses that GPU's one array: calls that overlap on one GPU
 * (other streams, other host threads) race and must be serialised by the
 * caller.  Out-of-range targets are treated as ignored, as in flce_forward, but
 * there is no workspace whose status word flce_get_status could read.
 */
int flce_forward_no_alloc(const flce_params* p, const void* hidden, const void* weight, const void* bias,
                          const void* targets, float* loss, float* lse, int64_t* num_correct, float* entropy_sum,
                          void* stream);

/*
 * Synchronises `stream`, then reads the status word that the last forward,
 * backward or forward-backward call on this workspace left: FLCE_OK, FLCE_ERR_TARGET_OUT_OF_RANGE,
 * or FLCE_ERR_HIP if the stream reports an error.
 */
int flce_get_status(const void* workspace, void* stream);

/* Static text for a status code. */
const char* flce_status_string(int status);

/* ---------------------------------------------------------------------------
 * Generic chunked linear loss ("Chunked Linear Loss" page: the per-chunk steps
 * of "Why chunk the projection?" and the "Loss function contract").  The
 * projection logits = inputs . weight^T is formed one block of rows at a time;
 * a loss function supplied by the caller turns each block of logits into its
 * loss and its logits gradient G; the library then adds G . weight to
 * grad_inputs and G^T . inputs to grad_weight.  No bias, scale or cap: those
 * belong to the loss function.  At most one block of logits exists at a time.
 * ------------------------------------------------------------------------- */

/* Called on the host once per block, in row order.  `logits` is device memory
 * holding the block's (rows, vocab) logits in `dtype` (flce_dtype), row stride
 * `ld` elements, rows row0 .. row0+rows-1 of inputs.  The function must enqueue
 * on `stream` work that overwrites logits[i][j] (i < rows, j < vocab) with
 * d loss / d logits[i][j] in the same dtype, leaves the rest of the buffer as it
 * is, and adds the block's loss to *loss (device fp32).  Return 0, or non-zero
 * to stop: flce_chunked_linear_loss then returns FLCE_ERR_CALLBACK and the
 * outputs are undefined. */
typedef int (*flce_chunk_loss_fn)(void* user, int64_t row0, int64_t rows, int64_t vocab, void* logits,
                                  int64_t ld, int32_t dtype, float* loss, void* stream);

typedef struct {
  int64_t n_tokens;           /* N >= 0                                                  */
  int64_t hidden;             /* H >= 8, H % 8 == 0                                      */
  int64_t vocab;              /* V >= 1                                                  */
  int64_t chunk_rows;         /* rows per block, a multiple of 256; 0 = library choice   */
  int32_t dtype;              /* flce_dtype of inputs, weight, logits and grad_inputs    */
  int32_t grad_weight_dtype;  /* flce_dtype of grad_weight                               */
  int32_t accum_dtype;        /* grad_weight summed over the blocks in FLCE_F32 (rounded
                                 once) or in grad_weight_dtype (rounded per block):
                                 "Chunked Linear Loss", "Weight-gradient accumulation
                                 dtype", its "fp32" and "weight" modes                   */
  int32_t flags;              /* FLCE_ACCUMULATE_GRAD_WEIGHT or 0                        */
} flce_chunked_params;

/* Bytes of device workspace flce_chunked_linear_loss needs.  Host only. */
int flce_chunked_workspace_size(const flce_chunked_params* p, size_t* bytes);

/*
 *  inputs:      device (N, H), weight: device (V, H), both in p->dtype.
 *  loss:        device fp32 scalar: the sum of the blocks' losses.  Required.
 *  grad_inputs: device (N, H) in p->dtype (fp32 accumulation, one rounding).
 *  grad_weight: device (V, H) in p->grad_weight_dtype.
 * The loss function runs between launches on `stream`; with a deterministic
 * loss function the results are deterministic.
 */
int flce_chunked_linear_loss(const flce_chunked_params* p, const void* inputs, const void* weight,
                             flce_chunk_loss_fn fn, void* user, float* loss, void* grad_inputs,
                             void* grad_weight, void* workspace, size_t workspace_bytes, void* stream);

/* Built-in loss function for flce_chunked_linear_loss: weighted squared error,
 * the "Direct logits gradients" example of the "Chunked Linear Loss" page:
 *   loss = sum_ij (z_ij - y_ij)^2 r_i f_j,   d loss / d z_ij = 2 (z_ij - y_ij) r_i f_j,
 * with z the logits (read in their dtype, math in fp32) and the gradient
 * rounded to the logits' dtype.  `user` points to an flce_wmse_args. */
typedef struct {
  const float* target;          /* device (N, vocab) fp32, row stride ld_target >= vocab   */
  int64_t ld_target;
  const float* row_weight;      /* device (N) fp32 (r)                                     */
  const float* feature_weight;  /* device (vocab) fp32 (f)                                 */
  float* row_loss;              /* device (N) fp32: receives each row's loss               */
} flce_wmse_args;

int flce_weighted_mse_chunk(void* user, int64_t row0, int64_t rows, int64_t vocab, void* logits, int64_t ld,
                            int32_t dtype, float* loss, void* stream);

/* Library version, major*10000 + minor*100 + patch. */
int flce_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H */
