/*
 * flce.h - chunked fused linear cross-entropy / selective log-softmax on
 * AMD Instinct MI355X (gfx950).  C ABI; plain pointers and sizes only.
 *
 * What the library computes
 * -------------------------
 * Given flattened hidden states H [T x D] and an lm_head W [V x D] (both
 * bfloat16, row-major), labels y [T] and an ignore index, the logits are
 * z_t = W h_t (bf16 x bf16 products accumulated in fp32, never rounded back to
 * bf16) and for every token
 *     lse_t = log sum_v exp(z_tv),
 *     NLL_t = lse_t - z_{t,y_t}            (mode FLCE_MODE_NLL),
 *     log p_t = z_{t,y_t} - lse_t          (mode FLCE_MODE_LOGPROB).
 * The full [T x V] logit matrix never exists in device memory.
 *
 * Sources on the pages:
 *  - Unsloth, "Reinforcement Learning GRPO mit 7x laengerem Kontext", section
 *    "Chunking der abgeflachten Sequenzlaenge": the flattened (batch x context)
 *    rows are processed in chunks so that the logits are never materialised in
 *    full (Equations 1-3 give their memory); the chunk logits are handled in
 *    float32; the call returns the selective log-softmax at the completion ids.
 *  - same page, section "Auslagern von Aktivierungen fuer Log-Softmax": the
 *    forward runs without autograd state, the backward recomputes the chunked
 *    logits and back-propagates a per-token grad_output.
 *  - TRL v1.13 article (arex-research.com), section on the four hurdles:
 *    loss_type "chunked_nll" computes the loss 256 rows at a time and sums;
 *    section on the chunked loss returning to tensor cores: the GEMM operands
 *    stay bf16 (no float32 copy of the lm_head), forward plus backward.
 *
 * Conventions common to every entry point
 * ---------------------------------------
 *  - Every pointer argument is DEVICE memory owned by the caller; the library
 *    never allocates, frees or synchronises.  Work is enqueued on `stream`
 *    (a hipStream_t; NULL = the default stream); buffers must stay alive until
 *    the stream has passed the call.  One workspace must not be used by two
 *    calls that can run at the same time.
 *  - Layouts: hidden [T x D] and weight [V x D] bf16 row-major, rows 16-byte
 *    aligned (D a multiple of 8, base pointers 16-byte aligned); labels int64
 *    [T]; per-token outputs fp32 [T].
 *  - Arguments are checked on the host before anything is enqueued; a failed
 *    check returns a status and enqueues nothing.  The library never aborts.
 *    The last failure's text is available from flce_last_error() (per thread).
 *  - A label outside [0, V) that is not ignore_index is a caller error: that
 *    token's output is NaN (so is the mean) and its gradient row is zero.
 *    Tokens whose label equals ignore_index output 0, get a zero gradient row
 *    and are left out of the mean's denominator.
 *  - Results are deterministic: repeated calls with the same inputs give the
 *    same bits (no floating-point atomics).
 *  - The host pointers are the optional logit transform and the policy
 *    losses' parameter struct (read during the call, not retained).
 *  - A call only launches kernels on `stream` (no allocation, memset, copy or
 *    synchronisation), so it may be recorded into a HIP graph by stream
 *    capture; a replay repeats the work with the captured pointers and sizes.
 */
#ifndef FLCE_H
#define FLCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum flce_status {
  FLCE_OK = 0,
  FLCE_ERR_ARG = 1,          /* NULL or misaligned pointer, unknown mode, both/neither grad */
  FLCE_ERR_SHAPE = 2,        /* T < 0, D/V/chunk_rows < 1, or sizes too large for the ABI */
  FLCE_ERR_WORKSPACE = 3,    /* workspace smaller than flce_workspace_bytes() */
  FLCE_ERR_UNSUPPORTED = 4,  /* D not a multiple of 8, or the device is not gfx950 */
  FLCE_ERR_HIP = 5           /* a HIP runtime call or kernel launch failed */
} flce_status;

enum { FLCE_MODE_NLL = 0, FLCE_MODE_LOGPROB = 1 };

/*
 * Optional per-logit transform applied before the log-softmax: the chunked
 * call on the Unsloth GRPO page (section "Chunking der abgeflachten
 * Sequenzlaenge") takes logit_scale_multiply, logit_scale_divide,
 * logit_softcapping and temperature, and the page says softcapping and
 * temperature scaling are supported; it prints no formula.  This library
 * applies them in that order to each raw logit z:
 *     z' = z * scale_multiply                 (skipped when scale_multiply == 0)
 *     z' = z' / scale_divide                  (skipped when scale_divide == 0)
 *     z' = softcap * tanh(z' / softcap)       (skipped when softcap == 0)
 *     z' = z' / temperature
 * and every output (lse, NLL, log p) refers to z'.  The backward takes the
 * chain rule through the transform.  scale_multiply, scale_divide and softcap
 * must be >= 0 and finite, temperature > 0 and finite; otherwise the call
 * fails with FLCE_ERR_ARG.  A NULL pointer means no transform.  Passed by
 * host pointer; forward and backward must be given the same values.
 */
typedef struct flce_logit_transform {
  float scale_multiply;
  float scale_divide;
  float softcap;
  float temperature;
} flce_logit_transform;

/*
 * Bytes of device workspace that flce_forward and flce_backward need for this
 * shape (one size serves both).  It does not grow with T x V.  The backward
 * stages the softmax gradient of a block of R rows x Vc vocabulary entries in
 * bf16, R * Vc * 2 <= chunk_rows * V * 4 bytes (the fp32 logits of one chunk,
 * the pages' Equation 3; at least one 256 x 256 tile), next to the fp32 dH
 * sums of the row block (R * D * 4 per split of the vocabulary chunk), a bf16
 * copy of the row block's hidden states transposed (R * D * 2) and O(T)
 * per-token values; R <= 8192.  Returns 0 when the arguments are invalid
 * (same rules as the entry points) or overflow.
 */
size_t flce_workspace_bytes(int64_t T, int64_t D, int64_t V, int64_t chunk_rows);

/*
 * Forward.  Writes, for t < T:
 *   out[t]  = NLL_t or log p_t (mode), 0 where labels[t] == ignore_index;
 *   lse[t]  = log-sum-exp of the logit row (written for ignored rows too;
 *             the backward takes it back);
 *   *mean_out (if mean_out != NULL; one fp32 in device memory)
 *           = sum of out over non-ignored tokens / their number (0 if none).
 * chunk_rows only bounds the workspace (see flce_workspace_bytes); the
 * results do not depend on it beyond fp32 rounding order.  T == 0 is valid:
 * nothing is written except *mean_out = 0.
 */
flce_status flce_forward(const void *hidden, const void *weight, const int64_t *labels,
                         int64_t T, int64_t D, int64_t V, int64_t ignore_index,
                         int64_t chunk_rows, int mode, const flce_logit_transform *transform,
                         float *out, float *lse, float *mean_out,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * flce_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation and outputs, with the forward's partial results kept in a
 * fixed array inside the library instead of a caller workspace.  The array
 * holds FLCE_FORWARD_SCRATCH_BYTES (16 MiB); the library reserves one per GPU
 * when its code is loaded there and keeps it until the process ends.  The
 * forward uses at most about 8 * max(T_pad, 524288) + 4 * T_pad bytes of it
 * (T_pad = T rounded up to 256; 4.7 MB at 131,072 tokens, 12.6 MB at 1,048,576),
 * so T up to about 1.39 million tokens fits; beyond the limit the call returns
 * FLCE_ERR_WORKSPACE and enqueues nothing.
 * Nothing in the array needs clearing between calls (every value a call reads
 * was written by that call).  All calls on one GPU share its array: calls that
 * can overlap on one GPU (two streams, two threads) race, so serialise them.
 * Same arguments, conventions and errors as flce_forward otherwise.
 */
#define FLCE_FORWARD_SCRATCH_BYTES ((size_t)16 << 20)

flce_status flce_forward_noalloc(const void *hidden, const void *weight, const int64_t *labels,
                                 int64_t T, int64_t D, int64_t V, int64_t ignore_index,
                                 int64_t chunk_rows, int mode,
                                 const flce_logit_transform *transform, float *out, float *lse,
                                 float *mean_out, void *stream);

/*
 * Backward.  Recomputes the logits chunk by chunk and writes
 *   grad_hidden [T x D] bf16  = G W,
 *   grad_weight [V x D] fp32  = G^T H      (added to the existing contents if
 *                                           accumulate_grad_weight != 0),
 * with G_tv = c_t (softmax(z'_t)_v - [v == y_t]) dz'_tv/dz_tv (z' = z without a
 * transform) and
 *   c_t = s * grad_out[t]            if grad_out != NULL (dL/d out_t),
 *   c_t = s * (*grad_mean) / N_valid if grad_out == NULL (dL/d mean; device scalar),
 * s = +1 for FLCE_MODE_NLL and -1 for FLCE_MODE_LOGPROB, c_t = 0 for ignored
 * (and out-of-range) labels, N_valid = number of tokens whose label is not
 * ignore_index (c_t = 0 for all t if N_valid == 0).  Exactly one of grad_out
 * and grad_mean must be non-NULL.  Either gradient output may be NULL: a NULL
 * grad_hidden skips the dH products, a NULL grad_weight skips the dW products
 * (a frozen lm_head); both NULL is FLCE_ERR_ARG.  lse must be the forward's
 * output for the same inputs and transform.  T == 0 is valid: grad_weight (if
 * given) is zeroed unless accumulating.  A tile of 256 consecutive tokens in
 * which every c_t is 0 (prompt tokens of a policy loss, say) is left out of the
 * GEMMs (the other tiles are packed into the leading row blocks): its
 * grad_hidden rows are written as zeros and it adds nothing to grad_weight,
 * exactly what computing it gives.
 */
flce_status flce_backward(const void *hidden, const void *weight, const int64_t *labels,
                          const float *lse, int64_t T, int64_t D, int64_t V,
                          int64_t ignore_index, int64_t chunk_rows, int mode,
                          const flce_logit_transform *transform,
                          const float *grad_out, const float *grad_mean,
                          void *grad_hidden, float *grad_weight, int accumulate_grad_weight,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Distillation through two LM heads over one vocabulary (TRL v1.13 article,
 * speed section: the distillation trainer computes every chunk twice, for the
 * student and for the teacher).  The pages define no divergence; this call
 * computes the forward Kullback-Leibler divergence of the student from the
 * teacher per token,
 *     kl_t = sum_v p_t,v (log p_t,v - log p_s,v),
 * p_s = softmax(W_s h_s,t), p_t = softmax(W_t h_t,t) (each head's logits through
 * the same optional logit transform), and, if asked, the student's gradients
 * of L = sum_t c_t kl_t:
 *   grad_student_hidden [T x Ds] bf16 = G W_s,
 *   grad_student_weight [V x Ds] fp32 = G^T H_s (added if accumulate_grad_weight),
 *   G_tv = c_t (p_s,tv - p_t,tv) dz'_tv/dz_tv.
 * The teacher gets no gradient.  Inputs: student_hidden [T x Ds],
 * student_weight [V x Ds], teacher_hidden [T x Dt], teacher_weight [V x Dt],
 * all bf16 row-major (Ds, Dt multiples of 8).  labels is an optional int64 [T]
 * mask: tokens whose label equals ignore_index are left out (kl = 0, no
 * gradient, not counted in the mean); other label values are not used; NULL
 * keeps every token.  Outputs (each optional): kl_out [T] fp32, *mean_out =
 * mean of kl over kept tokens (0 if none).  Gradients are computed when
 * grad_out (dL/d kl_t, [T]) or grad_mean (dL/d mean, device scalar) is given
 * (at most one): c_t = grad_out[t], or *grad_mean / N_kept; at least one of
 * grad_student_hidden and grad_student_weight must then be non-NULL (a NULL one
 * is not computed).  The forward values and the
 * gradients come from one call: the logits of both heads are recomputed per
 * block (the two log-sum-exps first), nothing of size T x V is stored, and
 * the workspace is bounded like that of the cross-entropy path.  T == 0 is
 * valid.  Same conventions (device pointers, stream, errors, determinism) as
 * above.
 */
size_t flce_distill_workspace_bytes(int64_t T, int64_t Ds, int64_t Dt, int64_t V,
                                    int64_t chunk_rows);

flce_status flce_distill(const void *student_hidden, const void *student_weight, int64_t Ds,
                         const void *teacher_hidden, const void *teacher_weight, int64_t Dt,
                         const int64_t *labels, int64_t ignore_index, int64_t T, int64_t V,
                         int64_t chunk_rows, const flce_logit_transform *transform,
                         float *kl_out, float *mean_out, const float *grad_out,
                         const float *grad_mean, void *grad_student_hidden,
                         float *grad_student_weight, int accumulate_grad_weight,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * The same call with the generalized Jensen-Shannon divergence in place of the
 * KL (the TRL v1.13 article names a fused linear JSD loss among the losses
 * built on the chunked LM head, without defining it; this is the textbook
 * skewed form): with weight beta in (0, 1) and M = beta p_t + (1 - beta) p_s,
 *     jsd_t = beta KL(p_t || M) + (1 - beta) KL(p_s || M)
 * (beta = 1/2: the symmetric JSD, at most ln 2), and the student's gradient
 *     G_tv = c_t p_s,tv (g_tv - sum_u p_s,tu g_tu) dz'_tv/dz_tv,
 *     g = (1 - beta) log(p_s / M).
 * jsd_out [T] replaces kl_out; every other argument, the workspace size
 * (flce_distill_workspace_bytes) and the error conventions are those of
 * flce_distill.  beta outside (0, 1) gives FLCE_ERR_ARG.  The gradient needs
 * each token's full-vocabulary sum before any G value exists, so with a
 * gradient the call recomputes both heads' logits once more than the KL does.
 */
flce_status flce_distill_jsd(const void *student_hidden, const void *student_weight, int64_t Ds,
                             const void *teacher_hidden, const void *teacher_weight, int64_t Dt,
                             const int64_t *labels, int64_t ignore_index, int64_t T, int64_t V,
                             int64_t chunk_rows, const flce_logit_transform *transform,
                             float beta, float *jsd_out, float *mean_out, const float *grad_out,
                             const float *grad_mean, void *grad_student_hidden,
                             float *grad_student_weight, int accumulate_grad_weight,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * Policy-optimisation losses on the selective log-softmax.  The TRL v1.13
 * article (section on the other v1.13 changes) names fused linear GRPO, DPO
 * and KTO losses built on the chunked LM head, and the Unsloth GRPO
 * long-context page feeds the chunked selective log-softmax into GRPO; neither
 * defines the losses, so these calls compute the published objectives:
 *
 *   GRPO (DeepSeekMath's group relative policy optimisation with its unbiased
 *   KL estimator):  r_t = exp(logp_t - old_t),
 *     s_t = min(r_t A_b, clip(r_t, 1 - eps_low, 1 + eps_high) A_b),
 *     k_t = exp(ref_t - logp_t) - (ref_t - logp_t) - 1,
 *     L = -(1/B') sum_{b: n_b > 0} (1/n_b) sum_{t in b} (s_t - beta k_t);
 *   DPO (direct preference optimisation): pi_b = sum_{t in b} logp_t, the first
 *     P = n_seq/2 sequences chosen and the last P rejected (pair i = (i, P+i)),
 *     Delta_i = beta ((pi_i - ref_i) - (pi_{P+i} - ref_{P+i})),
 *     L = (1/P) sum_i log(1 + exp(-Delta_i));
 *   KTO (Kahneman-Tversky optimisation): r_b = pi_b - ref_b, z0 = max(*kl_ref, 0),
 *     v_b = desirable_weight sigmoid(beta (r_b - z0)) for desirable sequences,
 *           undesirable_weight sigmoid(beta (z0 - r_b)) otherwise,
 *     L = (1/n_seq) sum_b (lambda_b - v_b).
 *
 * logp_t is log softmax(W h_t)[labels_t] (through the optional logit transform),
 * as flce_forward computes it in FLCE_MODE_LOGPROB.  The T = n_seq * S tokens
 * are n_seq sequences of S consecutive rows; tokens whose label is ignore_index
 * are not completion tokens (no term, no gradient); n_b counts the completion
 * tokens of sequence b and B' the sequences with at least one.  Inputs besides
 * those of flce_forward, all device memory: GRPO advantages [n_seq] fp32,
 * old_logp [T] fp32 (NULL: old = logp, ratio 1), ref_logp [T] fp32 (NULL: no
 * KL term); DPO/KTO ref_seq_logp [n_seq] fp32 (the reference model's summed
 * completion log-probs); KTO desirable [n_seq] uint8 (nonzero = desirable) and
 * kl_ref (device scalar z0 estimate, NULL = 0).  old, ref, advantages and z0
 * are constants.  params is a host pointer: beta (GRPO: KL weight >= 0;
 * DPO/KTO: > 0), eps_low in [0, 1) and eps_high >= 0 (GRPO), the KTO weights
 * (>= 0).  Outputs: *loss_out (device scalar, required), logp_out [T] (optional:
 * the per-token log-probs, 0 off the completions).  If grad_loss (device scalar
 * dTotal/dL) is given, grad_hidden [T x D] bf16 and grad_weight [V x D] fp32
 * (added if accumulate_grad_weight) receive grad_loss * dL/dH and dL/dW through
 * the log-prob backward (recompute), with grad_out_t = grad_loss * dL/dlogp_t;
 * either may be NULL (not computed), not both.
 * At a clipping kink GRPO takes the unclipped derivative.  Errors: n_seq must
 * divide T (FLCE_ERR_SHAPE), DPO needs an even n_seq, parameters out of range
 * give FLCE_ERR_ARG; otherwise the conventions of flce_forward (T == 0 gives
 * *loss_out = 0 and, unless accumulating, a zero grad_weight).  The workspace,
 * flce_policy_workspace_bytes(...), holds the cross-entropy workspace plus
 * 12 T + 16 n_seq bytes (rounded).
 */
typedef struct flce_policy_params {
  float beta;
  float eps_low, eps_high;  /* GRPO */
  float desirable_weight, undesirable_weight;  /* KTO */
} flce_policy_params;

size_t flce_policy_workspace_bytes(int64_t T, int64_t D, int64_t V, int64_t chunk_rows,
                                   int64_t n_seq);

flce_status flce_grpo_loss(const void *hidden, const void *weight, const int64_t *labels,
                           int64_t ignore_index, int64_t T, int64_t D, int64_t V,
                           int64_t chunk_rows, const flce_logit_transform *transform,
                           int64_t n_seq, const float *advantages, const float *old_logp,
                           const float *ref_logp, const flce_policy_params *params,
                           float *loss_out, float *logp_out, const float *grad_loss,
                           void *grad_hidden, float *grad_weight, int accumulate_grad_weight,
                           void *workspace, size_t workspace_bytes, void *stream);

flce_status flce_dpo_loss(const void *hidden, const void *weight, const int64_t *labels,
                          int64_t ignore_index, int64_t T, int64_t D, int64_t V,
                          int64_t chunk_rows, const flce_logit_transform *transform,
                          int64_t n_seq, const float *ref_seq_logp,
                          const flce_policy_params *params, float *loss_out, float *logp_out,
                          const float *grad_loss, void *grad_hidden, float *grad_weight,
                          int accumulate_grad_weight, void *workspace, size_t workspace_bytes,
                          void *stream);

flce_status flce_kto_loss(const void *hidden, const void *weight, const int64_t *labels,
                          int64_t ignore_index, int64_t T, int64_t D, int64_t V,
                          int64_t chunk_rows, const flce_logit_transform *transform,
                          int64_t n_seq, const float *ref_seq_logp, const uint8_t *desirable,
                          const float *kl_ref, const flce_policy_params *params,
                          float *loss_out, float *logp_out, const float *grad_loss,
                          void *grad_hidden, float *grad_weight, int accumulate_grad_weight,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Host policy (no device call).  The Unsloth GRPO page (section "Chunking der
 * abgeflachten Sequenzlaenge" and the configuration section after it) cuts
 * each sequence of the flattened batch into `multiplier` chunks, with the
 * default multiplier max(4, context_length // 4096), i.e. batch * multiplier
 * chunks of context_length / multiplier rows each.
 *
 * flce_chunk_rows_for: rows per chunk, ceil(context_length / multiplier), for
 * that multiplier (<= 0 selects the default).  Returns 0 if context_length < 1.
 */
int64_t flce_chunk_rows_for(int64_t context_length, int64_t multiplier);

/*
 * flce_tune: the page lets both the hidden-state mini-batching (its
 * unsloth_grpo_mini_batch: the batch is processed in that many groups of
 * sequences) and the chunk multiplier be chosen automatically from the free
 * device memory, without giving the rule.  This one: the fewest mini-batches,
 * then the smallest multiplier not below the default, such that one
 * mini-batch's device memory
 *     flce_workspace_bytes(T_mb, D, V, chunk_rows)
 *   + T_mb * D * 2 (its hidden states) + T_mb * D * 2 (their gradient)
 *   + T_mb * 16 (labels, output, lse)
 * fits in budget_bytes, with T_mb = ceil(batch / mini_batches) * context_length.
 * Writes *mini_batches, *chunk_rows and, if bytes_needed != NULL, the memory
 * above.  FLCE_ERR_WORKSPACE if nothing fits; FLCE_ERR_ARG / FLCE_ERR_SHAPE
 * for invalid arguments.  The gradient of the lm_head (V * D * 4 bytes, fp32)
 * is the caller's and is not counted.
 */
flce_status flce_tune(int64_t batch, int64_t context_length, int64_t D, int64_t V,
                      size_t budget_bytes, int64_t *mini_batches, int64_t *chunk_rows,
                      size_t *bytes_needed);

/*
 * The schedule the library would use for this shape, for inspection and
 * tests (host only, no device call).  Fills info[0..11] with:
 *   0 token tiles of 256 rows     1 vocabulary tiles of 256 rows
 *   2 forward vocabulary splits   3 backward row block (tokens)
 *   4 number of row blocks        5 backward vocabulary chunk
 *   6 number of vocabulary chunks 7 split-K factor of the grad_hidden GEMM
 *   8 forward workspace bytes     9 backward workspace bytes
 *  10 bf16 gradient-tile bytes   11 chunk-logit bound chunk_rows*V*4
 * Returns FLCE_OK or the status flce_workspace_bytes would fail with.
 */
flce_status flce_describe_plan(int64_t T, int64_t D, int64_t V, int64_t chunk_rows,
                               int64_t *info);

/*
 * Per-launch kernel timing, a profiling aid (no page defines it; it is how the
 * time of each GEMM kernel inside one call is measured).  The exceptions to the
 * conventions above: flce_timing_begin creates HIP events and flce_timing_end
 * waits for them; while timing is on, the entry points also record events on
 * their stream (do not turn it on around stream capture).
 *
 * flce_timing_begin(capacity): creates `capacity` (1 .. 1,048,576) events on the
 * current device and turns timing on for the whole process.  From then on each
 * entry point records one event on its stream before its first launch and one
 * after every kernel it launches, tagged with that kernel's FLCE_KERNEL_* code,
 * until the events run out (later marks are dropped and counted).  Timing must
 * be off (FLCE_ERR_ARG otherwise).
 *
 * flce_timing_end(ids, ms, capacity, count, dropped): waits for the recorded
 * events, turns timing off, destroys the events and writes, in launch order,
 * one (id, milliseconds) pair per recorded kernel: ids[i] its FLCE_KERNEL_*
 * code, ms[i] the time between the event before it on the same stream and the
 * event after it (-1 when the mark before it was recorded on another stream or
 * none exists).  At most `capacity` pairs are written; *count receives the
 * number recorded, *dropped (if not NULL) the marks dropped for lack of events.
 * ids and ms are host arrays.  FLCE_ERR_ARG if timing is off or an argument is
 * NULL.  Calls on several streams at once interleave their marks; time one
 * stream at a time.
 */
enum {
  FLCE_KERNEL_FWD_LSE = 1,        /* forward: fused logit GEMM + running log-sum-exp */
  FLCE_KERNEL_FWD_COMBINE = 2,    /* forward: combine of the vocabulary splits */
  FLCE_KERNEL_FWD_MEAN = 3,       /* forward: the mean over kept tokens */
  FLCE_KERNEL_BWD_PREP = 4,       /* backward: per-token scale c_t */
  FLCE_KERNEL_BWD_HT = 5,         /* backward: H^T of a row block */
  FLCE_KERNEL_BWD_GRAD = 6,       /* backward: logit recompute + bf16 gradient block G */
  FLCE_KERNEL_BWD_DH = 7,         /* backward: dH partial sums G W */
  FLCE_KERNEL_BWD_DW = 8,         /* backward: dW update G^T H */
  FLCE_KERNEL_BWD_DH_OUT = 9,     /* backward: dH partials summed and rounded to bf16 */
  FLCE_KERNEL_FILL = 10,          /* a constant fill (T == 0 paths) */
  FLCE_KERNEL_DST_LSE = 11,       /* distillation: combine of one head's log-sum-exp */
  FLCE_KERNEL_DST_PREP = 12,      /* distillation: per-token scale */
  FLCE_KERNEL_DST_TEACHER = 13,   /* distillation: teacher logits -> probabilities */
  FLCE_KERNEL_DST_STUDENT = 14,   /* distillation: student logits -> sums and G */
  FLCE_KERNEL_DST_REDUCE = 15,    /* distillation: per-token sums of a row block */
  FLCE_KERNEL_DST_DH = 16,        /* distillation: dH partial sums */
  FLCE_KERNEL_DST_DW = 17,        /* distillation: dW update */
  FLCE_KERNEL_DST_COMBINE = 18,   /* distillation: per-token divergence */
  FLCE_KERNEL_POLICY = 19,        /* policy losses: the loss kernels (2 or 3 launches) */
  FLCE_KERNEL_FWD_SKIP_PREP = 20, /* policy losses: list of the token tiles with a label */
  FLCE_KERNEL_BWD_ZERO_ROWS = 21, /* backward: dH rows of token tiles without gradient */
  FLCE_KERNEL_COUNT = 22
};

flce_status flce_timing_begin(int32_t capacity);
flce_status flce_timing_end(int32_t *ids, float *ms, int32_t capacity, int32_t *count,
                            int32_t *dropped);

/* Static name of a FLCE_KERNEL_* code ("?" for other values). */
const char *flce_kernel_name(int32_t id);

/* Static text for a status code. */
const char *flce_status_string(int status);

/* Text of the last failure on the calling thread ("" if none). */
const char *flce_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H */
