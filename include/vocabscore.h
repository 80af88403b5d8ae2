/*
 * vocabscore.h - C ABI of libvocabscore.so: vocabulary-scale LM-head scoring
 * on one MI355X (gfx950).
 *
 * What the library computes (natural logs, entropy in nats):
 *   x[t, v]  input logit of token row t and vocabulary id v: either given
 *            (bf16 or fp32 logits) or the projection sum_h bf16(hidden[t,h]) *
 *            W[v,h] of the hidden state onto the LM-head weight, with fp32
 *            accumulation (xorl issue #71, section 1: "chunked projection";
 *            SkyRL PR #2004, review's selected-projection code: the hidden
 *            state is cast to the weight dtype before the dot product).
 *   z = x / tau_t        temperature divides the finished dot product
 *                        (same code: "... .sum(dim=-1) / temperature").
 *   LSE, logprob = z_y - LSE, entropy = -sum p ln p over a support: the full
 *   vocabulary, a recorded sampler support, or the top-k/top-p/min-p support.
 *
 * Conventions for every entry point:
 *   - Every array argument is a DEVICE pointer (hipMalloc'ed or a torch CUDA
 *     tensor), row-major, owned by the caller.  The scoring entry points
 *     allocate nothing and keep no per-call state outside the caller's
 *     buffers; concurrent calls on different streams with different buffers
 *     are safe.  The library's only process-wide state is a per-device cache
 *     of the compute-unit count (atomic; every writer stores the same value)
 *     and the diagnostic timer below (one caller at a time).
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  All work
 *     is enqueued on it; returning VS_OK means "enqueued", not "finished".
 *   - `workspace` is caller-owned device scratch of at least
 *     vs_workspace_size(...) bytes, 256-byte aligned.  Its contents on entry
 *     do not matter; it must not be used by anything else until the call's
 *     work on `stream` has finished.
 *   - Argument errors are detected on the host, before anything is enqueued,
 *     and reported as a VS_E_* code (vs_status_string gives the text).  Data
 *     problems (bad ids, NaN logits, invalid temperatures or filter
 *     parameters) are reported per row in `row_status` by the device; the
 *     host never synchronises.
 *   - Pointers marked "nullable" may be NULL: that output is not written (and,
 *     where stated, not computed).
 *   - Range: the full-vocabulary, recorded-support and L1 kernels work in fp32
 *     base-2 units u = x * log2(e) / tau.  A row whose largest logit has
 *     |x| * log2(e) / tau above the fp32 range (about 3.4e38) is BAD_INPUT,
 *     and a log-probability below about -2.3e38 comes out as -inf.  With fp32
 *     logits (or the projection's fp32 sums) each term's exponent carries the
 *     fp32 rounding of u, about |u| * 2^-24: the results keep 1e-3 accuracy
 *     for |x / tau| up to about 2^12.  For bf16 logits the scale log2(e)/tau
 *     is rounded to 16 significant bits (a 2^-17 relative change of 1/tau),
 *     which makes every product x * scale exact, so that accuracy holds at
 *     any magnitude.  The sampling transforms compute their masses in fp64 and
 *     take every finite bf16 logit; their fp32 outputs are the fp64 results
 *     rounded (a logprob beyond the fp32 range is -inf).
 */
#ifndef VOCABSCORE_H
#define VOCABSCORE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ------------------------------------------------------ */
enum {
  VS_OK = 0,
  VS_E_NULL = 1,        /* a required pointer is NULL                          */
  VS_E_SHAPE = 2,       /* T, H or V out of range, or a leading dim too small  */
  VS_E_DTYPE = 3,       /* unsupported dtype or dtype combination              */
  VS_E_ALIGN = 4,       /* pointer or leading dim breaks an alignment rule     */
  VS_E_PARAM = 5,       /* a scalar parameter is out of range                  */
  VS_E_WORKSPACE = 6,   /* workspace NULL, misaligned or smaller than needed   */
  VS_E_UNSUPPORTED = 7, /* valid request this version does not implement       */
  VS_E_DEVICE = 8,      /* a HIP launch failed                                 */
  VS_E_SCRATCH = 9      /* the call needs more scratch than the allocation-free
                           entry point holds (vs_noalloc_scratch_bytes)         */
};

/* ---- dtypes and source kinds ------------------------------------------- */
enum { VS_F32 = 0, VS_BF16 = 1 };
enum { VS_SRC_LOGITS = 0, VS_SRC_HIDDEN_WEIGHT = 1 };
enum {
  VS_OP_SCORE_FULL = 0,
  VS_OP_SCORE_SUPPORT = 1,
  VS_OP_SCORE_TRANSFORMS = 2,
  VS_OP_L1_DISTANCE = 3,
  VS_OP_SAMPLE_TRANSFORMS = 4,
  VS_OP_L1_LOSS = 5,
  VS_OP_SCORE_FULL_BACKWARD = 6,
  VS_OP_SCORE_SUPPORT_BACKWARD = 7
};

/* ---- per-row status bits (uint8 per row) -------------------------------- */
#define VS_ROW_EMPTY_SUPPORT 0x01u          /* recorded support has no id >= 0         */
#define VS_ROW_TARGET_OUTSIDE_SUPPORT 0x02u /* logprob is -inf                          */
#define VS_ROW_BAD_INPUT 0x04u              /* float outputs of the row are NaN         */
#define VS_ROW_FULL_VOCAB_FALLBACK 0x08u    /* synthetic-EOS full-vocabulary logprob    */
#define VS_ROW_SUPPORT_TRUNCATED 0x10u      /* dense support ids cut at the capacity    */

/*
 * The logits of T token rows over a vocabulary of V ids, in one of two forms.
 *
 * kind == VS_SRC_LOGITS:
 *   logits       [T, ld_logits] of logits_dtype (VS_BF16 or VS_F32), ld_logits >= V;
 *                base aligned to the element size.
 * kind == VS_SRC_HIDDEN_WEIGHT (logits are never materialised):
 *   hidden       [T, ld_hidden] of hidden_dtype (VS_BF16 or VS_F32; fp32 is
 *                rounded to bf16, nearest-even, before the projection);
 *   weight       [V, ld_weight] VS_BF16, row v = vocabulary id v (the LM head);
 *   H            hidden size, a multiple of 8; ld_hidden, ld_weight >= H and
 *                multiples of 8; hidden and weight 16-byte aligned.
 * temperature    [T] fp32 per-row tau (nullable: then temperature_scalar is
 *                used for every row).  tau <= 0 or non-finite => BAD_INPUT row.
 * Limits: 1 <= T < 2^31, 1 <= V < 2^31, H < 2^24 (vs_score_support_ids with
 * a hidden/weight source: H <= 16384, the hidden row it stages in LDS; larger
 * H returns VS_E_UNSUPPORTED).
 */
typedef struct vs_source {
  int32_t kind;
  const void* logits;
  int32_t logits_dtype;
  int64_t ld_logits;
  const void* hidden;
  int32_t hidden_dtype;
  int64_t ld_hidden;
  const void* weight;
  int32_t weight_dtype;
  int64_t ld_weight;
  int64_t T, H, V;
  const float* temperature;
  float temperature_scalar;
} vs_source;

/*
 * Bytes of workspace the call `op` needs for this source (width = support
 * width for VS_OP_SCORE_SUPPORT and VS_OP_SCORE_SUPPORT_BACKWARD, the
 * vocab_chunk for VS_OP_SCORE_FULL_BACKWARD, else 0).  For VS_OP_L1_DISTANCE only src->T
 * and src->V are read.  Returns 0 on a NULL src.
 */
size_t vs_workspace_size(int32_t op, const vs_source* src, int64_t width);

/*
 * Full-vocabulary scoring: for every row t,
 *   lse[t]     = ln sum_v exp(z[t,v])
 *   logprob[t] = z[t, y_t] - lse[t]
 *   entropy[t] = -sum_v p ln p,  p = softmax(z[t,:])
 * Source: xorl issue #71 section 1 (projection -> log-sum-exp -> selected
 * logprob) and SkyRL PR #2004 (the full-vocabulary entropy path).  With a
 * hidden/weight source the vocabulary is swept in tiles and each tile's
 * (max, sum-exp, sum p*z) is folded in registers; the per-tile partials are
 * merged in a fixed order (tiles ascending inside each vocab_chunk-wide
 * chunk, chunks combined by a fixed tree), so results are bitwise
 * reproducible.  vocab_chunk (> 0) is rounded down to a whole number of
 * tiles (at least one); it changes only rounding.  A logits source is read
 * once by one workgroup per row, whose per-thread states are merged by a
 * fixed tree; vocab_chunk does not apply to it and it needs no workspace.
 *   target_ids  [T] int64, y_t in [0, V) else BAD_INPUT.
 *   lse, entropy, row_status nullable; logprob required.
 * Row status: BAD_INPUT if tau is invalid, y_t is out of range, or the row's
 * LSE is not finite (a NaN or +inf logit, or all logits -inf).
 */
int vs_score_full(const vs_source* src, const int64_t* target_ids, int64_t vocab_chunk, float* lse,
                  float* logprob, float* entropy, uint8_t* row_status, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * The vector-Jacobian product of full-vocabulary scoring through the fused
 * projection (xorl issue #71 section 1: the op ends in "selected logprob +
 * VJP"; SkyRL PR #2004: gradients through logprob and entropy).  Given the
 * forward's lse and entropy and the upstream gradients a_t = grad_logprob[t],
 * b_t = grad_entropy[t] of sum_t (a_t logprob_t + b_t entropy_t):
 *   dX[t, v]          = (a_t ([v = y_t] - p_v) - b_t p_v (ln p_v + H_t)) / tau_t
 *   grad_hidden[t, h] = sum_v dX[t, v] W[v, h]               [T, ld_grad_hidden] fp32
 *   grad_weight[v, h] = sum_t dX[t, v] bf16(hidden)[t, h]    [V, ld_grad_weight] fp32
 * (an fp32 hidden state's bf16 cast passes its gradient through: grad_hidden
 * is also the gradient of the fp32 values).  dX is recomputed tile by tile
 * by the forward's MFMA sweep, rounded to bf16 (nearest even) and kept only
 * for one vocab_chunk-wide chunk of the vocabulary at a time; both products
 * run on the same MFMA loop, in a fixed order (chunks ascending), so results
 * are bitwise reproducible.  Source: VS_SRC_HIDDEN_WEIGHT (else
 * VS_E_UNSUPPORTED).  grad_logprob / grad_entropy nullable (0); entropy is
 * required with grad_entropy.  grad_hidden and grad_weight nullable (at
 * least one).  A row the forward marked BAD_INPUT (its lse not finite, an
 * invalid tau or target) contributes no gradient.  Workspace:
 * vs_workspace_size(VS_OP_SCORE_FULL_BACKWARD, src, vocab_chunk), about
 * 2 (2T + H) vocab_chunk + 2 H T bytes (bf16 dX, its transpose and the
 * chunk's transposed weight rows); vocab_chunk is rounded up to a multiple
 * of 256 and capped at V rounded up and at 2^23; vocab_chunk >= V makes one
 * chunk, the fastest form (one d_hidden product over the whole vocabulary).
 */
int vs_score_full_backward(const vs_source* src, const int64_t* target_ids, const float* lse, const float* entropy,
                           const float* grad_logprob, const float* grad_entropy, int64_t vocab_chunk,
                           float* grad_hidden, int64_t ld_grad_hidden, float* grad_weight, int64_t ld_grad_weight,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * The vector-Jacobian product of recorded-support scoring through the fused
 * projection (SkyRL PR #2004, Implementation: gradients through the replayed
 * support's logprob and entropy; the description: a singleton support has
 * exactly zero entropy and zero entropy gradient).  With the scores of
 * vs_score_support_ids and a_t = grad_logprob[t], b_t = grad_entropy[t] of
 * sum_t (a_t logprob_t + b_t entropy_t), for each id v = support_ids[t, j]
 * of the support S_t (p the softmax of z over S_t, H_S its entropy):
 *   dX[t, j]          = (a_t ([v = y_t] - p_v) - b_t p_v (ln p_v + H_S)) / tau_t
 *   grad_hidden[t, h] = sum_j dX[t, j] W[v_j, h]          (j ascending)
 *   grad_weight[v, h] = sum over (t, j) with v_j = v of dX[t, j] bf16(hidden)[t, h]
 *                       (pairs in ascending (t, j) order; 0 for ids in no support)
 * dX stays fp32; both sums are fp32 in a fixed order, so results are bitwise
 * reproducible.  Rows without gradient (their rows of grad_hidden are 0): the
 * BAD_INPUT rows of vs_score_support_ids (invalid tau, an id >= V, a repeated
 * id, a target outside [0, V), a support LSE that is not finite) and rows
 * with an empty support (their scores are constants; the full-vocabulary
 * logprob of a synthetic-EOS row has its gradient from
 * vs_score_full_backward).  A target outside the support drops the logprob
 * term (that logprob is the constant -inf).  Source: VS_SRC_HIDDEN_WEIGHT
 * with H <= 16384 (else VS_E_UNSUPPORTED).  support_ids, width, ld_ids as for
 * vs_score_support_ids.  grad_logprob / grad_entropy nullable (0);
 * grad_hidden [T, ld_grad_hidden] and grad_weight [V, ld_grad_weight] fp32,
 * nullable (at least one; every row of a given output is written).
 * Workspace: vs_workspace_size(VS_OP_SCORE_SUPPORT_BACKWARD, src, width).
 */
int vs_score_support_backward(const vs_source* src, const int64_t* support_ids, int64_t width, int64_t ld_ids,
                              const int64_t* target_ids, const float* grad_logprob, const float* grad_entropy,
                              float* grad_hidden, int64_t ld_grad_hidden, float* grad_weight, int64_t ld_grad_weight,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Recorded-support scoring (SkyRL PR #2004, sections Problem and
 * Implementation, and the review's selected-projection code): the support of
 * row t is S_t = {support_ids[t, j] : j < width, support_ids[t, j] >= 0}
 * (dense, padded with any negative id, no CSR).  Over S_t:
 *   logprob[t] = z[t, y_t] - ln sum_{v in S_t} exp(z[t, v])   (-inf and
 *                TARGET_OUTSIDE_SUPPORT if y_t is not in S_t)
 *   entropy[t] = -sum_{v in S_t} p ln p of the renormalised distribution.
 * A singleton support gives exactly 0 and 0.  With a hidden/weight source
 * only the selected weight rows are read (the hidden row once per token row).
 * Empty rows: EMPTY_SUPPORT, entropy 0; logprob is the full-vocabulary one
 * (FULL_VOCAB_FALLBACK) when full_vocab_fallback[t] != 0 (synthetic EOS), else 0.
 *   support_ids          [T, ld_ids] int64, ld_ids >= width, 0 <= width <= 1024.
 *   full_vocab_fallback  [T] uint8, nullable (no fallback).
 *   vocab_chunk          merge chunk of the fallback's full-vocabulary scoring.
 *   entropy, row_status  nullable; logprob required.
 * BAD_INPUT: tau invalid, an id >= V, a repeated id, or (on a scored row) a
 * target outside [0, V) or a support whose LSE is not finite.
 * VS_E_UNSUPPORTED: a hidden/weight source with H > 16384.
 */
int vs_score_support_ids(const vs_source* src, const int64_t* support_ids, int64_t width,
                         int64_t ld_ids, const int64_t* target_ids,
                         const uint8_t* full_vocab_fallback, int64_t vocab_chunk, float* logprob,
                         float* entropy, uint8_t* row_status, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Scores over the sampling-transform support (xorl issue #71 section 3: the
 * program temperature -> stable token-id top-k -> inclusive top-p -> min-p
 * against the original row max).  Rank order pi = ids by (z desc, id asc).
 *   top_k[t]  <= 0 or >= V: no top-k; else keep the first k ranks.
 *   top_p[t]  >= 1: no top-p; else, on the top-k renormalised masses, keep
 *             rank j iff the mass of ranks before j is < top_p (the crossing
 *             rank is kept).  NaN or <= 0 => BAD_INPUT.
 *   min_p[t]  <= 0: off; else keep rank j iff exp(z_pi(j) - z_pi(0)) >= min_p.
 *             NaN or > 1 => BAD_INPUT.
 * The support S_t = pi[0:L], L = min(L_k, L_p, L_m) >= 1.  Outputs per row:
 *   logprob, entropy      support-conditioned, as vs_score_support_ids
 *   support_len[t]        L
 *   threshold_logit[t]    x at rank L-1 (the input logit, not divided by tau)
 *   threshold_ties[t]     #{j < L : x_pi(j) == x_pi(L-1)}
 *   support_ids_out       [T, support_ids_cap] int64: pi[0:min(L, cap)], -1
 *                         padded; SUPPORT_TRUNCATED if L > cap (nullable)
 *   full_lse[t]           full-vocabulary LSE of z (nullable)
 * Sources: VS_BF16 logits (VS_F32 logits give VS_E_UNSUPPORTED), or a
 * hidden/weight source (xorl issue #71, "Proposed direction" item 3: support
 * masking over the chunked projection), whose logits are
 *   x[t, v] = bf16_rne(sum_h bf16(hidden[t, h]) W[v, h])   (fp32 sums)
 * - the fused sweep's fp32 logits rounded to bf16, nearest even - computed by
 * the MFMA sweep for blocks of up to 2048 token rows into the workspace and
 * scored block by block; the caller never sees them.  That source takes
 * V <= 2^23 (VS_E_UNSUPPORTED above: the block's row stride, V rounded up to
 * 8, stays at most 2^23 elements).
 * The transform parameters are never ignored.  support_ids_cap > 4096 with a
 * non-NULL support_ids_out gives VS_E_UNSUPPORTED.  A target outside S_t gives
 * logprob -inf and TARGET_OUTSIDE_SUPPORT.  BAD_INPUT rows: NaN floats,
 * support_len 0, ids -1.  entropy, row_status, support_len, threshold_logit,
 * threshold_ties, full_lse nullable; logprob required.  Workspace
 * (vs_workspace_size(VS_OP_SCORE_TRANSFORMS, src, 0)): T bytes for V <= 81920;
 * above that also a per-row record of 51,456 bytes (the count pass hands the
 * finishing pass each row's non-empty key counts, up to 256 segments of 64
 * keys, and dense-id candidates through it; a row whose keys fill more
 * segments is redone by a kernel that re-reads it, with the same results).  A hidden/weight source needs these for one block
 * of min(T, 2048) rows, plus that block's logits (rows x V rounded up to 8,
 * bf16) and, for an fp32 hidden state, its bf16 copy (T x H x 2 bytes).
 */
int vs_score_transforms(const vs_source* src, const int32_t* top_k, const float* top_p,
                        const float* min_p, const int64_t* target_ids, float* logprob,
                        float* entropy, uint8_t* row_status, int32_t* support_len,
                        float* threshold_logit, int32_t* threshold_ties, int64_t* support_ids_out,
                        int64_t support_ids_cap, float* full_lse, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * The seeded Gumbel draw that ends the transform program (xorl issue #71,
 * section 3: temperature -> stable token-id top-k -> inclusive top-p -> min-p
 * -> seeded Gumbel; the pages name the last stage without defining its
 * generator).  For every row t: the support S_t of vs_score_transforms, then
 *   sampled_ids[t] = argmax over v in S_t of (x_v - x_max)/tau - ln(-ln u_v)
 * (the lower id on equal scores; computed in fp64), with
 *   u_v = (r_v + 1/2) 2^-32, r_v = word (v mod 4) of Philox4x32-10 (Salmon et
 *   al., "Parallel random numbers: as easy as 1, 2, 3", SC 2011) of the counter
 *   (v div 4, t, offset mod 2^32, offset div 2^32) under the key
 *   (seed mod 2^32, seed div 2^32).
 * A (seed, offset) pair gives a fixed draw on every run; distinct offsets
 * give independent draws.  Parameters and sources as for
 * vs_score_transforms (bf16 logits, or a hidden/weight source through its
 * bf16-rounded logits; t is always the row's index in the whole batch).
 * Outputs:
 *   sampled_ids [T] int64 (-1 on a BAD_INPUT row)
 *   row_status, support_len, threshold_logit, threshold_ties  (nullable) the
 *                row's BAD_INPUT bit and support descriptor.
 * The support-conditioned logprob and entropy of the drawn tokens come from
 * vs_score_transforms with target_ids = sampled_ids.  Workspace:
 * vs_workspace_size(VS_OP_SAMPLE_TRANSFORMS, src, 0).
 */
int vs_sample_transforms(const vs_source* src, const int32_t* top_k, const float* top_p, const float* min_p,
                         uint64_t seed, uint64_t offset, int64_t* sampled_ids, uint8_t* row_status,
                         int32_t* support_len, float* threshold_logit, int32_t* threshold_ties, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Draft/target softmax L1 distance (DeepSpec PR #87, section Purpose):
 *   l1[t]          = sum_v |softmax(target[t,:])_v - softmax(draft[t,:])_v|, in [0, 2]
 *   accept_rate[t] = clamp(1 - 0.5 * l1[t], 0, 1)
 * No temperature.  Identical rows give exactly 0 and 1.  A row whose target
 * or draft LSE is not finite gives NaN for both.
 *   target_logits [T, ld_target], draft_logits [T, ld_draft], both of `dtype`
 *   (VS_BF16 or VS_F32), ld >= V.  accept_rate nullable; l1 required.
 *   No workspace: workspace may be null and workspace_bytes 0.
 */
int vs_l1_distance(const void* target_logits, const void* draft_logits, int32_t dtype, int64_t T,
                   int64_t V, int64_t ld_target, int64_t ld_draft, float* l1, float* accept_rate,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * vs_score_full without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, outputs and row status as vs_score_full,
 * minus workspace and workspace_bytes; the same kernels and results.  The
 * scratch the hidden/weight source needs sits in one device array of
 * vs_noalloc_scratch_bytes() bytes (64 MiB) per GPU, held from the library's
 * load until the process ends: enough for the per-tile partials of 4096 rows
 * over a vocabulary of 151,936 (38.9 MB; fp32 hidden states add T * H * 2
 * bytes).  vs_workspace_size(VS_OP_SCORE_FULL, ...) above that limit returns
 * VS_E_SCRATCH before anything is enqueued.  The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine).  All calls on one GPU
 * share its array: calls that overlap on one GPU (on two streams, or from two
 * threads) race and must be ordered by the caller.  Its contents carry over
 * between calls; nothing in it needs to start at zero.
 */
int vs_score_full_noalloc(const vs_source* src, const int64_t* target_ids, int64_t vocab_chunk, float* lse,
                          float* logprob, float* entropy, uint8_t* row_status, void* stream);

/* Bytes of the allocation-free entry point's scratch array on each GPU. */
size_t vs_noalloc_scratch_bytes(void);

/*
 * The weighted L1 distillation loss on the shared distance, and its gradient
 * with respect to the draft logits (DeepSpec PR #87, Purpose: the per-token
 * distance is computed once and reused for accept_rate and for the weighted
 * L1 loss; Test Plan: its numerator, denominator and draft-logit gradients):
 *   l1[t], accept_rate[t]   as vs_l1_distance
 *   loss[0] = num = sum_t w_t l1[t] over rows with w_t != 0
 *   loss[1] = den = sum_t w_t,   loss[2] = num / den          (device, fp32)
 *   grad_draft[t, v] = grad_scale * (w_t / den) * q_v (s_v - sum_u s_u q_u),
 *     p = softmax(target[t]), q = softmax(draft[t]), s = sign(q - p) (0 where
 *     equal): the gradient of grad_scale * loss[2].  The target is a fixed
 *     reference (no gradient).
 * A row of weight 0 adds nothing to num and gets a zero gradient row, even if
 * its distance is NaN (a loss mask); a row whose target or draft LSE is not
 * finite and whose weight is not 0 makes num, the loss and its gradient row
 * NaN.  Weights are read as given (finite and >= 0 is the caller's part).
 *   target_logits, draft_logits, dtype, T, V, ld_*   as vs_l1_distance
 *   weights     [T] fp32, nullable (every weight 1)
 *   grad_draft  [T, ld_grad] of grad_dtype (VS_F32 or VS_BF16, the latter
 *               rounded to nearest even), nullable: no gradient computed
 *   accept_rate nullable; l1 and loss required.
 * Workspace: vs_workspace_size(VS_OP_L1_LOSS, src with T, 0) bytes.
 */
int vs_l1_loss(const void* target_logits, const void* draft_logits, int32_t dtype, int64_t T, int64_t V,
               int64_t ld_target, int64_t ld_draft, const float* weights, float grad_scale, float* l1,
               float* accept_rate, float* loss, void* grad_draft, int32_t grad_dtype, int64_t ld_grad,
               void* workspace, size_t workspace_bytes, void* stream);

/* ---- Diagnostics (not part of the scoring contract) -------------------- */

/* vs_sweep_timer(1): every later scoring call records two HIP events on its
 * own stream, immediately before and immediately after its main sweep
 * kernel(s) -- the MFMA sweep of the fused input, the logits sweep, the
 * support kernel, the transforms kernels or the L1 kernel; not the merge,
 * not the fallback rows' sweep.  vs_sweep_timer(0) stops recording.
 * Process-wide state for the device current at enable time: one caller at a
 * time.  Returns VS_OK, or VS_E_DEVICE when the events cannot be created. */
int vs_sweep_timer(int32_t enable);

/* Waits for the most recent bracket and writes its length in milliseconds
 * to *ms (host pointer).  VS_E_NULL for a NULL ms, VS_E_PARAM when no bracket
 * has been recorded since the timer was enabled, VS_E_DEVICE on a HIP error. */
int vs_sweep_timer_ms(float* ms);

/* Static text for a return code. */
const char* vs_status_string(int32_t code);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t vs_version(void);

#ifdef __cplusplus
}
#endif
#endif /* VOCABSCORE_H */
