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
 *     tensor), row-major, owned by the caller.  The library allocates nothing
 *     and keeps no mutable global state; concurrent calls on different
 *     streams with different buffers are safe.
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
  VS_E_DEVICE = 8       /* a HIP launch failed                                 */
};

/* ---- dtypes and source kinds ------------------------------------------- */
enum { VS_F32 = 0, VS_BF16 = 1 };
enum { VS_SRC_LOGITS = 0, VS_SRC_HIDDEN_WEIGHT = 1 };
enum { VS_OP_SCORE_FULL = 0, VS_OP_SCORE_SUPPORT = 1, VS_OP_SCORE_TRANSFORMS = 2, VS_OP_L1_DISTANCE = 3 };

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
 * Limits: 1 <= T < 2^31, 1 <= V < 2^31, H < 2^24.
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
 * width for VS_OP_SCORE_SUPPORT, else 0).  For VS_OP_L1_DISTANCE only src->T
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
 * Source must be VS_SRC_LOGITS with VS_BF16 logits (else VS_E_UNSUPPORTED);
 * the transform parameters are never ignored.  support_ids_cap > 4096 with a
 * non-NULL support_ids_out gives VS_E_UNSUPPORTED.  A target outside S_t gives
 * logprob -inf and TARGET_OUTSIDE_SUPPORT.  BAD_INPUT rows: NaN floats,
 * support_len 0, ids -1.  entropy, row_status, support_len, threshold_logit,
 * threshold_ties, full_lse nullable; logprob required.  Workspace: T bytes for
 * V <= 81920; above that also a per-row record of 149,760 bytes (the count
 * pass hands the finishing pass each row's non-empty key counts and dense-id
 * candidates through it).
 */
int vs_score_transforms(const vs_source* src, const int32_t* top_k, const float* top_p,
                        const float* min_p, const int64_t* target_ids, float* logprob,
                        float* entropy, uint8_t* row_status, int32_t* support_len,
                        float* threshold_logit, int32_t* threshold_ties, int64_t* support_ids_out,
                        int64_t support_ids_cap, float* full_lse, void* workspace,
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
