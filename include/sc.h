/*
 * sc.h -- C ABI of the score-centering (SC) correction library for AMD
 * Instinct MI355X (gfx950).
 *
 * The method: "Score Centering" example page of Agent Lightning
 * (microsoft.github.io/agent-lightning), section "Score Centering".  For each
 * generated position the rollout recorded the top-K candidate ids H with their
 * behaviour probabilities q, plus the sampled token a and its log-probability.
 * The trainer scores its policy p over the full vocabulary at the rollout
 * temperature T, gathers p at H and at a, sets P_H = sum_H p, Q_H = sum_H q,
 * rho = max(1 - Q_H, 1e-6) / max(1 - P_H, 1e-6), and trains on the token loss
 * -sg(A) [log p_a - sum_H sg(q_v - rho p_v) log p_v], the unrecorded tail of
 * the behaviour policy being taken proportional to p.  Advantages come from
 * group standard-deviation normalisation of the rewards (same page, section
 * "Training"), the loss is reduced over all generated tokens of the step with
 * padding masked, and rollout_corr/k3_kl is the masked mean of
 * exp(d) - 1 - d with d = train logprob - rollout logprob.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named as device pointers address GPU memory owned by the caller.
 *   The library allocates nothing and keeps no state besides a cached query of
 *   the device's compute-unit count.
 * - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default
 *   stream) and never synchronises.  Calls are thread-safe.
 * - Argument errors are returned as a negative sc_status BEFORE any HIP call is
 *   made, so they can be exercised on a host without a GPU.  A failed kernel
 *   launch returns SC_ERR_HIP.  No exception crosses the ABI.
 * - Data errors found on the device (see SC_DEV_*) are OR-ed into the optional
 *   `dev_status` word; every float output of the affected row is then NaN,
 *   its integer outputs are -1 and its full-vocabulary output row is NaN.
 * - Padding rows (resp_idx < 0) are never read: their outputs are 0, their
 *   integer outputs -1 and their full-vocabulary output row is all zero.
 * - Per-id outputs keep the caller's slot order of head_ids.
 * - Logits rows: `row_stride` elements apart, row_stride >= vocab.  The
 *   16-byte vector path is taken when the logits pointer is 16-byte aligned
 *   and row_stride * element size is a multiple of 16; otherwise a scalar path
 *   gives the same results.
 * - Preconditions checked on the host: 1 <= k <= min(vocab, 1024),
 *   1 <= vocab < 2^31, 0 <= n_rows < 2^31, temperature finite and > 0.
 */
#ifndef SC_H
#define SC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
enum sc_status {
  SC_OK = 0,
  SC_ERR_ARG = -1,          /* invalid argument (checked before any HIP call) */
  SC_ERR_UNSUPPORTED = -2,  /* valid but outside what the library supports    */
  SC_ERR_HIP = -3,          /* a HIP runtime call or kernel launch failed       */
  SC_ERR_TOO_LARGE = -4     /* beyond the static workspace of an entry point    */
};                          /* that allocates nothing (see below)              */

/* Element types of logits and of the full-vocabulary output row. */
enum sc_dtype { SC_F32 = 0, SC_BF16 = 1 };

/* Device data-error bits OR-ed into *dev_status. */
enum sc_dev_flag {
  SC_DEV_BAD_ID = 1,       /* a head id outside [0, vocab)                     */
  SC_DEV_DUP_ID = 2,       /* the same id recorded twice in one row            */
  SC_DEV_BAD_SAMPLED = 4,  /* sampled id outside [0, vocab)                    */
  SC_DEV_NONFINITE = 8,    /* NaN or +inf logit, -inf at a head or sampled id  */
  SC_DEV_BAD_RESP = 16     /* resp_idx >= n_responses                          */
};

/* Full-vocabulary output row selected by `row_mode`. */
enum sc_row_mode {
  SC_ROW_DLOGITS = 0,    /* d(step loss)/dz = -A / (T * N_valid) * g          */
  SC_ROW_SCORE = 1,      /* centered score g = e_a - mu_hat - (1 - S) p       */
  SC_ROW_CORRECTION = 2  /* correction mu_hat - p                             */
};

/* Importance weighting of the token loss (Score Centering page, SC settings:
 * is_mode none / tis / mis; lecture notes "RL systems for agents", section 1,
 * truncated importance sampling).  w = p(a) / mu(a) from the recorded
 * rollout log-probability; the weight is a stop-gradient factor:
 *   SC_IS_NONE  1
 *   SC_IS_TIS   min(w, is_hi)                      (tis_max, default 2.0)
 *   SC_IS_MIS   w if is_lo <= w <= is_hi, else 0   (mis_min 0.5, mis_max 5.0) */
enum sc_is_mode { SC_IS_NONE = 0, SC_IS_TIS = 1, SC_IS_MIS = 2 };

/* Columns of the per-row statistics array row_stats[n_rows][SC_NSTATS]. */
enum sc_stat {
  SC_STAT_LSE = 0,      /* log sum_v exp(z_v / T)                              */
  SC_STAT_LOGP_A = 1,   /* log p(a) of the sampled token                       */
  SC_STAT_TAIL = 2,     /* tau = sum of p over ids outside H (= 1 - P_H)       */
  SC_STAT_P_H = 3,      /* trainer mass on the recorded ids                    */
  SC_STAT_Q_H = 4,      /* recorded behaviour mass (coverage)                  */
  SC_STAT_RHO = 5,      /* tail scale rho, both clamps applied                 */
  SC_STAT_S = 6,        /* sum of mu_hat = Q_H + rho * tau                     */
  SC_STAT_LOSS = 7,     /* token loss -A wt [log p_a - centering sum_H c log p] */
  SC_STAT_TV = 8,       /* 1/2 sum_v |mu_hat_v - p_v|                          */
  SC_STAT_KL = 9,       /* KL(mu_hat || p)                                     */
  SC_STAT_K3 = 10,      /* exp(d) - 1 - d, d = log p(a) - rollout log mu(a)    */
  SC_STAT_ENTROPY = 11, /* -sum_v p_v log p_v of the trainer policy            */
  SC_STAT_W = 12,       /* importance ratio w = p(a) / mu(a)                   */
  SC_STAT_WEIGHT = 13,  /* stop-gradient weight wt applied (sc_is_mode)        */
  SC_STAT_REV_KL = 14,  /* KL(p || mu_hat)                                     */
  SC_STAT_LSE_LO = 15,  /* LSE's float64 value minus its fp32 value: the two
                           columns together carry the log-sum-exp to sc_center
                           at double precision                               */
  SC_NSTATS = 16
};

/* Columns of the per-row integer array row_idx[n_rows][2]. */
enum sc_idx { SC_IDX_ARGMAX = 0, SC_IDX_A_SLOT = 1, SC_NIDX = 2 };

/* Sums and means written by sc_batch_sums, batch[SC_NBATCH] (float64). */
enum sc_batch {
  SC_SUM_LOSS = 0, SC_SUM_K3 = 1, SC_SUM_TV = 2, SC_SUM_KL = 3,
  SC_SUM_Q_H = 4, SC_SUM_P_H = 5, SC_SUM_ENTROPY = 6, SC_SUM_REV_KL = 7,
  SC_SUM_ROWS = 8, SC_SUM_FLAGGED = 9, SC_MAX_W = 10,
  SC_MEAN_LOSS = 11, SC_MEAN_K3 = 12, SC_MEAN_TV = 13, SC_MEAN_KL = 14,
  SC_MEAN_Q_H = 15, SC_MEAN_P_H = 16, SC_MEAN_ENTROPY = 17, SC_MEAN_REV_KL = 18,
  SC_NBATCH = 19
};

/*
 * sc_logprobs -- trainer log-probabilities at the recorded and sampled ids.
 *
 * Score Centering page, section "Score Centering": the trainer evaluates its
 * policy on the whole vocabulary at the temperature the rollout used and
 * reads off the log-probabilities of the recorded candidates and of the
 * sampled token.  One HBM pass over each valid row of logits.
 *
 *   logits        device, [n_rows, row_stride] of logits_dtype (SC_F32/SC_BF16)
 *   head_ids      device int32 [n_rows, k]: recorded ids H, distinct, in [0,V)
 *   sampled       device int32 [n_rows]: sampled token a
 *   resp_idx      device int32 [n_rows] or NULL: response of each row, < 0 for
 *                 padding; NULL means every row is valid
 *   temperature   T > 0; p = softmax(z / T)
 * Outputs (device, written for every row):
 *   row_stats     float [n_rows, SC_NSTATS]: columns LSE, LSE_LO, LOGP_A, TAIL,
 *                 P_H, ENTROPY (the other columns are left untouched)
 *   row_idx       int32 [n_rows, SC_NIDX]: argmax of the raw logits (lowest
 *                 index among equal maxima) and the slot k with H_k = a (-1 if
 *                 a is not recorded)
 *   head_logp     float [n_rows, k]: log p at H, in slot order
 *   dev_status    uint32 or NULL: data-error bits OR-ed in
 */
int sc_logprobs(const void* logits, int logits_dtype, int64_t n_rows,
                int64_t vocab, int64_t row_stride, const int32_t* head_ids,
                int32_t k, const int32_t* sampled, const int32_t* resp_idx,
                float temperature, float* row_stats, int32_t* row_idx,
                float* head_logp, uint32_t* dev_status, void* stream);

/*
 * sc_center -- the SC token loss, rho, coefficients, diagnostics and
 * (optionally) one full-vocabulary row per position, from sc_logprobs' output.
 *
 * Score Centering section: P_H, Q_H, rho, the token loss with stop-gradient
 * coefficients c = q - rho p on H, the tail proportional to p, global
 * generated-token reduction with padding masked; rollout_corr/k3_kl.
 * Reads row_stats columns LSE, LSE_LO, LOGP_A, TAIL and row_idx / head_logp as
 * written by sc_logprobs (or sc_logprobs_lmhead) on the same rows; writes
 * columns P_H .. K3 and W .. REV_KL.  When logits are given, log p and p at
 * the recorded ids and log p(a) are formed in float64 from the logits at
 * those ids and LSE + LSE_LO (head_logp and LOGP_A then serve only where an
 * id is out of range); without logits they come from head_logp and LOGP_A,
 * fp32 numbers, whose rounding c = q - rho p carries times rho p where rho is
 * large.  With row_out, the row maximum is read back from the logits at the
 * recorded argmax.
 * When row_out is not NULL the logits are streamed once more to write it.
 *
 *   logits, logits_dtype, row_stride   as for sc_logprobs; may be NULL when
 *                 row_out is NULL
 *   head_ids      device int32 [n_rows, k]
 *   head_probs    device float [n_rows, k]: recorded q (their sum may be < 1)
 *   sampled       device int32 [n_rows]
 *   rollout_logp  device float [n_rows] or NULL: recorded log mu(a); NULL
 *                 leaves the K3 column NaN
 *   resp_idx      device int32 [n_rows]: response of each row, < 0 = padding
 *   advantages    device float [n_responses]: A of each response
 *   n_valid       device int64 [1]: valid positions of the WHOLE step (all
 *                 chunks); read only for SC_ROW_DLOGITS with row_out
 *   row_out       device [n_rows, out_stride] of out_dtype, or NULL
 *   row_mode      sc_row_mode; SC_ROW_DLOGITS and SC_ROW_SCORE carry the
 *                 importance weight, SC_ROW_CORRECTION does not
 *   coef          device float [n_rows, k]: c_k = q_k - rho p_k, or NULL
 *   is_mode       sc_is_mode; TIS and MIS need rollout_logp
 *   is_lo, is_hi  MIS acceptance interval [is_lo, is_hi]; TIS cap is_hi
 *                 (finite, 0 <= is_lo <= is_hi, is_hi > 0)
 *   centering     non-zero: the SC loss; zero: the centering term is dropped
 *                 (loss -A wt log p_a, score wt (e_a - p)), the ablation of
 *                 the Score Centering page that turns centering off
 */
int sc_center(const void* logits, int logits_dtype, int64_t n_rows,
              int64_t vocab, int64_t row_stride, const int32_t* head_ids,
              const float* head_probs, int32_t k, const int32_t* sampled,
              const float* rollout_logp, const int32_t* resp_idx,
              const float* advantages, int32_t n_responses, float temperature,
              const int64_t* n_valid, float* row_stats, int32_t* row_idx,
              const float* head_logp, float* coef, void* row_out,
              int out_dtype, int64_t out_stride, int row_mode, int is_mode,
              float is_lo, float is_hi, int centering, uint32_t* dev_status,
              void* stream);

/*
 * sc_correct -- sc_logprobs followed by sc_center in one kernel: every output
 * of both, with each logits row brought from HBM once for the statistics and
 * re-read from the on-chip caches for row_out.  Same arguments and outputs as
 * the two calls together; row_stats, row_idx and head_logp are written, not
 * read.  head_logp and coef may be NULL.
 */
int sc_correct(const void* logits, int logits_dtype, int64_t n_rows,
               int64_t vocab, int64_t row_stride, const int32_t* head_ids,
               const float* head_probs, int32_t k, const int32_t* sampled,
               const float* rollout_logp, const int32_t* resp_idx,
               const float* advantages, int32_t n_responses, float temperature,
               const int64_t* n_valid, float* row_stats, int32_t* row_idx,
               float* head_logp, float* coef, void* row_out, int out_dtype,
               int64_t out_stride, int row_mode, int is_mode, float is_lo,
               float is_hi, int centering, uint32_t* dev_status, void* stream);

/*
 * sc_group_norm -- rollout-level advantages by group normalisation.
 *
 * Score Centering page, section "Training": both algorithms normalise the
 * advantages by the group's standard deviation; Agent Lightning v1.0.3 release note,
 * section 4: rewards stay fractional (no bf16 cast first) and the normaliser
 * must not overflow -- the kernel accumulates in float64.
 *
 *   rewards     device float [n_groups * group_size]; group j holds entries
 *               j*group_size .. j*group_size + group_size - 1
 *   mode        0: (R - mean) / (unbiased std + eps); 1: population std;
 *               2: R - mean (mean only).  A group of one gets 0 in modes 0-1.
 *   advantages  device float [n_groups * group_size] (output)
 * Preconditions: n_groups >= 0, 1 <= group_size <= 4096, eps >= 0 finite.
 */
int sc_group_norm(const float* rewards, int32_t n_groups, int32_t group_size,
                  int32_t mode, float eps, float* advantages, void* stream);

/*
 * sc_count_valid -- the exact number of non-padding positions (resp_idx >= 0)
 * as int64 (release note, section 4: token counts are not rounded).
 *   out         device int64 [1]; overwritten, or incremented when
 *               accumulate != 0 (for steps processed in chunks)
 */
int sc_count_valid(const int32_t* resp_idx, int64_t n_rows, int64_t* out,
                   int32_t accumulate, void* stream);

/*
 * sc_batch_sums -- step-level reductions in a fixed order (deterministic):
 * float64 sums over the valid rows of loss, K3, TV, KL, Q_H, P_H, entropy and
 * KL(p || mu_hat), the number of valid rows and of rows whose statistics are
 * NaN, the largest importance ratio w (lecture notes, section 7, debugging signals),
 * then the means over n_valid (global generated-token reduction, Score
 * Centering section).
 *   row_stats   device float [n_rows, SC_NSTATS] from sc_center / sc_correct
 *   resp_idx    device int32 [n_rows]
 *   n_valid     device int64 [1]
 *   batch       device double [SC_NBATCH]; sums overwritten, or added to when
 *               accumulate != 0; means recomputed from the sums every call
 */
int sc_batch_sums(const float* row_stats, const int32_t* resp_idx,
                  int64_t n_rows, const int64_t* n_valid, double* batch,
                  int32_t accumulate, void* stream);

/*
 * sc_reference_copy -- copies `bytes` bytes from src to dst with the plain
 * streaming kernel that serves as the measured bandwidth reference of the
 * roofline figures (a read-once / write-once stream with no arithmetic:
 * 16-byte nontemporal loads and stores, one workgroup per 512 KiB).  Not
 * part of the SC computation.
 *   src, dst   device, 16-byte aligned, not overlapping
 *   bytes      a multiple of 16, at most 2^40; 0 is a no-op
 * Returns SC_ERR_ARG for a bad argument before any HIP call.
 */
int sc_reference_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* Human-readable name of a status code (static storage). */
const char* sc_status_string(int status);

/*
 * Fused LM-head statistics.
 *
 * Score Centering page, section "Score Centering": the trainer scores the
 * current policy over the full vocabulary at the rollout temperature and
 * gathers the log-probabilities of the recorded ids and of the sampled token
 * (the page's SC worker does this on materialised logits and has no fused
 * LM-head path).  sc_logprobs_lmhead produces exactly the outputs of
 * sc_logprobs for logits z = X W^T / T without writing the [n_rows, vocab]
 * logits anywhere: z is computed tile by tile with bf16 matrix cores (fp32
 * accumulation over d) and folded into the running row statistics on chip.
 * sc_center (with logits = NULL and no full-vocabulary row) completes the
 * correction from these outputs.
 *
 *   hidden         device bf16 [n_rows, d], row stride hidden_stride elements
 *                  (16-byte aligned, stride a multiple of 8, <= 4,194,303)
 *   d              hidden size, a multiple of 64 (else SC_ERR_UNSUPPORTED)
 *   weight         device bf16 [vocab, d] (vocabulary projection, one row per
 *                  id), row stride weight_stride (same rules as hidden)
 *   head_ids .. dev_status   as sc_logprobs (row_stats columns LSE, LOGP_A,
 *                  TAIL, P_H and ENTROPY are written; head_logp may be NULL)
 *   workspace      device memory of at least sc_lmhead_workspace_size(n_rows,
 *                  vocab, k) bytes, 256-byte aligned, owned by the caller; its
 *                  contents need no initialisation and are scratch afterwards
 * A NaN or infinite logit (from non-finite inputs or overflow) flags the row
 * SC_DEV_NONFINITE.  Argmax is over the fp32 logits, lowest id on ties.
 */
int64_t sc_lmhead_workspace_size(int64_t n_rows, int64_t vocab, int32_t k);

int sc_logprobs_lmhead(const void* hidden, int64_t n_rows, int32_t d,
                       int64_t hidden_stride, const void* weight, int64_t vocab,
                       int64_t weight_stride, const int32_t* head_ids, int32_t k,
                       const int32_t* sampled, const int32_t* resp_idx,
                       float temperature, float* row_stats, int32_t* row_idx,
                       float* head_logp, void* workspace, int64_t workspace_bytes,
                       uint32_t* dev_status, void* stream);

/*
 * sc_logprobs_lmhead_static -- sc_logprobs_lmhead for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same arguments without the workspace, the same
 * kernels and bit-identical outputs.  Its workspace is a static device array
 * of SC_STATIC_SCRATCH_BYTES per GPU, held until the process ends; the call
 * allocates nothing.  Requests whose sc_lmhead_workspace_size exceeds it
 * return SC_ERR_TOO_LARGE before any HIP call (at vocab = 248,320 and
 * k = 128 that is more than 11,881 rows: call it on chunks of rows).  Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (concurrent streams or threads) race and must be serialised by the caller.
 */
#define SC_STATIC_SCRATCH_BYTES ((int64_t)64 << 20)

int sc_logprobs_lmhead_static(const void* hidden, int64_t n_rows, int32_t d,
                              int64_t hidden_stride, const void* weight,
                              int64_t vocab, int64_t weight_stride,
                              const int32_t* head_ids, int32_t k,
                              const int32_t* sampled, const int32_t* resp_idx,
                              float temperature, float* row_stats,
                              int32_t* row_idx, float* head_logp,
                              uint32_t* dev_status, void* stream);

/*
 * sc_lmhead_logits -- the logits X W^T of the fused kernel's GEMM, written as
 * fp32 [n_rows, logits_stride >= vocab] (the same tiles and accumulation
 * order, so its values are bit-identical to the ones sc_logprobs_lmhead
 * consumes).  Meant for checking; it writes n_rows * vocab floats.
 */
int sc_lmhead_logits(const void* hidden, int64_t n_rows, int32_t d,
                     int64_t hidden_stride, const void* weight, int64_t vocab,
                     int64_t weight_stride, float* logits, int64_t logits_stride,
                     void* stream);

/*
 * LM-head backward.
 *
 * The gradient of the SC step loss (Score Centering page, section "Score
 * Centering": the token loss, reduced over all generated tokens of the step)
 * with respect to the logits is dZ = -A wt / (T N_valid) g per row (the
 * SC_ROW_DLOGITS row of sc_center); through the LM head z = X W^T it gives
 * dHidden = dZ W and dW = dZ^T X.  The logits are recomputed from X and W
 * with the matrix cores of sc_logprobs_lmhead, so the [n_rows, vocab] logits
 * are never stored; the statistics come from sc_logprobs_lmhead followed by
 * sc_center (same head_ids, head_probs, sampled, resp_idx, advantages,
 * temperature, n_valid; centering as given to sc_center, the importance
 * weight read from row_stats).
 *
 * sc_lmhead_dlogits writes the bf16 dLogits rows themselves (round to
 * nearest even), dlogits_stride >= vocab, a multiple of 4, 8-byte aligned;
 * padding rows are zero, rows with NaN statistics NaN.
 *
 * sc_lmhead_backward processes chunk_rows rows at a time: their bf16
 * dLogits go to the workspace (sc_lmhead_backward_workspace_size(chunk_rows,
 * vocab, d) bytes, 256-byte aligned, caller-owned; it also holds W^T and the
 * chunk's transposed dLogits and hidden states), then the two products run
 * on the same bf16 matrix-core loop as the forward, fp32 accumulation (the
 * dHidden product has one 256-row tile per 256 rows of the chunk and d / 256
 * vocabulary-side tiles, so chunks of >= 8,192 rows fill the GPU):
 *   d_hidden   [n_rows, dh_stride >= d], bf16 or fp32 (dh_dtype), written
 *   d_weight   fp32 [vocab, dw_stride >= d]; written, or added to when
 *              accumulate != 0 (e.g. over several calls of one step)
 * The same argument rules as sc_logprobs_lmhead apply to hidden and weight.
 * Sizes whose workspace would exceed 2^62 bytes return SC_ERR_UNSUPPORTED
 * (from the size query and from sc_lmhead_backward alike).
 */
int sc_lmhead_dlogits(const void* hidden, int64_t n_rows, int32_t d,
                      int64_t hidden_stride, const void* weight, int64_t vocab,
                      int64_t weight_stride, const int32_t* head_ids,
                      const float* head_probs, int32_t k, const int32_t* sampled,
                      const int32_t* resp_idx, const float* advantages,
                      int32_t n_responses, float temperature, const int64_t* n_valid,
                      const float* row_stats, const int32_t* row_idx,
                      const float* head_logp, int centering, void* dlogits,
                      int64_t dlogits_stride, void* stream);

int64_t sc_lmhead_backward_workspace_size(int64_t chunk_rows, int64_t vocab, int32_t d);

int sc_lmhead_backward(const void* hidden, int64_t n_rows, int32_t d,
                       int64_t hidden_stride, const void* weight, int64_t vocab,
                       int64_t weight_stride, const int32_t* head_ids,
                       const float* head_probs, int32_t k, const int32_t* sampled,
                       const int32_t* resp_idx, const float* advantages,
                       int32_t n_responses, float temperature, const int64_t* n_valid,
                       const float* row_stats, const int32_t* row_idx,
                       const float* head_logp, int centering, void* d_hidden,
                       int dh_dtype, int64_t dh_stride, float* d_weight,
                       int64_t dw_stride, int accumulate, int64_t chunk_rows,
                       void* workspace, int64_t workspace_bytes, void* stream);

/*
 * sc_record -- the rollout engine's record of each generated position.
 *
 * Score Centering page, section "Score Centering": for every generated
 * position the rollout records the top K behaviour probabilities of its
 * sampling call (original normalisation kept, so they may sum below one) and,
 * separately, the log-probability of the token it sampled.  This produces
 * that record from the rollout logits: head_ids are the k largest logits
 * (ties go to the lower id), listed largest first; head_probs their
 * probabilities softmax(z / T) in fp32; sampled_logp = log softmax(z / T) at
 * the sampled id.  The selection is exact (a decision on the input values),
 * and head_probs uses the same fp32 arithmetic as sc_logprobs.
 *
 *   logits        device bf16/fp32 [n_rows, row_stride >= vocab]
 *   temperature   finite, > 0
 *   k             1 <= k <= min(vocab, 1024)
 *   sampled       device int32 [n_rows] or NULL (then sampled_logp must be
 *                 NULL too)
 *   head_ids      device int32 [n_rows, k]  (written)
 *   head_probs    device float [n_rows, k]  (written)
 *   sampled_logp  device float [n_rows] or NULL (written)
 *   dev_status    as for sc_logprobs: a NaN or +inf logit, an all -inf row,
 *                 a sampled id outside [0, vocab) or at a -inf logit flags
 *                 the row (ids -1, floats NaN)
 * Rows whose top-k boundary sits inside a large group of equal logits take
 * extra passes over the row (at most six) but give the same exact result.
 */
int sc_record(const void* logits, int logits_dtype, int64_t n_rows, int64_t vocab,
              int64_t row_stride, float temperature, int32_t k,
              const int32_t* sampled, int32_t* head_ids, float* head_probs,
              float* sampled_logp, uint32_t* dev_status, void* stream);

/* Library version, major * 10000 + minor * 100 + patch. */
int sc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SC_H */
