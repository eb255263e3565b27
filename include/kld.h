/*
 * libkld -- full-vocabulary KL scoring of a candidate model against a bf16
 * reference, on one AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources are cited by page title and section):
 *
 *  - Per position, KL(p || q) over every vocabulary id, p = softmax of the
 *    reference logits, q = softmax of the candidate logits, natural log,
 *    f32 softmax.  ("Qwen3.8-27B fidelity suite v5": opening paragraphs,
 *    the metric KL(BF16 || candidate); "Qwen3.8-27B Quantization Challenge":
 *    "How the references were made" -- the full 248,320-id distribution in
 *    f32 -- and "The score".)
 *  - Top-1 agreement (exact argmax match, ties to the lower id), the NLL of
 *    the true next token on both sides, the log-sum-exp of both rows.
 *    ("Qwopus3.8-27B-Coder-Flash: quality-eval reference": "Method".)
 *  - Logits either given, or produced in-kernel from final hidden states
 *    through one shared bf16 head W[V, d] that is never written out as
 *    logits.  (fidelity suite v5: opening paragraphs; "What is in here".)
 *  - Top-64 export: ids int32 and fp16 log-probs, most likely first, and the
 *    top-64 + one-tail-bucket approximate KLD.  (quality-eval reference:
 *    "Files", "Method".)
 *  - Mean / median / p99 / p99.9 KLD, top-1 rate and perplexities.
 *    ("The score"; "Qwen3.8-27B IQ8R": "Quality".)
 *  - Golden records (the 512 most likely ids with f32 log-probs, the NLL of
 *    the true next token, the entropy and the tail mass) and the 513-cell
 *    coarsened KL of a candidate against them.  ("Qwen3.8-27B Quantization
 *    Challenge": "Golden distributions", "The score".)
 *
 * Conventions shared by every entry point:
 *
 *  - Every tensor argument is DEVICE memory owned by the caller; the library
 *    never allocates or frees memory.  Scratch space comes from the caller's
 *    workspace (`ws`, `ws_bytes`), sized by kld_workspace_size().
 *  - Alignment: every pointer must be aligned to its element size (4 bytes
 *    for f32 / int32 arrays, 2 for bf16 / fp16 bit patterns, 8 for f64 /
 *    int64), otherwise KLD_EUNSUPPORTED; the head and hidden states of the
 *    fused entry points need 16 bytes.  A workspace must be 16-byte aligned,
 *    otherwise KLD_EWORKSPACE.  Allocations from the HIP allocator (or
 *    torch) meet all of these.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream).  Outputs are valid once that stream has completed the work.
 *  - Fail-closed: every argument (pointers, sizes, alignment, workspace size)
 *    is checked before anything is launched; on an error nothing is launched
 *    and nothing is written.  n == 0 is a valid no-op.  A failed launch
 *    returns KLD_EHIP.
 *  - No global mutable state (except the static scratch of
 *    kld_from_logits_noalloc): calls are thread-safe.  Results are bitwise
 *    deterministic (fixed-order merges, no floating-point atomics).
 *  - Non-finite inputs: a -inf logit is a zero-probability id; a finite
 *    reference logit against a -inf candidate logit makes KL +inf; a row with
 *    a NaN or +inf logit, or whose reference or candidate row is all -inf,
 *    gets KL = NaN.  A target id outside [0, V) gives NLL = NaN.
 */
#ifndef LIBKLD_KLD_H
#define LIBKLD_KLD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KLD_ABI_VERSION 1
#define KLD_TOPK 64           /* the export width the quality-eval reference uses */
#define KLD_GOLDEN_TOPK 512   /* ids listed per golden record (the challenge's references) */
#define KLD_MAX_QUANTILES 16
#define KLD_MAX_THRESHOLDS 16
#define KLD_MAX_REPLICATES 16384
#define KLD_NOALLOC_SCRATCH_BYTES (16u << 20)   /* static scratch of kld_from_logits_noalloc */

typedef enum kld_status {
  KLD_OK = 0,
  KLD_EINVAL = 1,       /* a required pointer is NULL or a count is negative */
  KLD_ESHAPE = 2,       /* inconsistent sizes (ld < v, v < 64 with top-k, k != 64, ...) */
  KLD_EDTYPE = 3,       /* unknown dtype code */
  KLD_EWORKSPACE = 4,   /* workspace missing, smaller than kld_workspace_size() or not 16-byte aligned */
  KLD_EUNSUPPORTED = 5, /* valid request the library does not serve (alignment, d % 8) */
  KLD_EHIP = 6,         /* the HIP runtime reported an error at launch */
  KLD_ETOOBIG = 7       /* kld_from_logits_noalloc: needs more than its static scratch */
} kld_status;

typedef enum kld_dtype {
  KLD_F32 = 0,          /* IEEE binary32 logits */
  KLD_BF16 = 1          /* bfloat16 logits, passed as uint16 bit patterns */
} kld_dtype;

/* Operation codes for kld_workspace_size(). */
enum {
  KLD_OP_FROM_LOGITS = 0,
  KLD_OP_FUSED_HEAD = 1,
  KLD_OP_TOPK_EXPORT = 2,
  KLD_OP_SUMMARY = 3,
  KLD_OP_COARSE_KL = 4,
  KLD_OP_PAIRED = 5,
  KLD_OP_COARSE_FUSED = 6
};
#define KLD_FLAG_TOPK 1       /* the call will also export top-64 lists */

/* Per-position outputs, each [n] device arrays.  `kl` is required; any other
 * member may be NULL to skip it.  nll_* need a target array. */
typedef struct kld_rows {
  float *kl;            /* KL(ref || cand) in nats, >= +0 (never -0) or NaN/+inf */
  float *nll_ref;       /* lse_ref - ref[target] */
  float *nll_cand;      /* lse_cand - cand[target] */
  float *lse_ref;       /* log-sum-exp of the reference row */
  float *lse_cand;
  int32_t *argmax_ref;  /* lowest id among the row's maxima */
  int32_t *argmax_cand;
} kld_rows;

/* Optional top-64 export, [n, 64] device arrays, most likely first (value
 * descending, then id ascending); lp is log-prob rounded to fp16 (nearest
 * even), given as uint16 bit patterns.  Members may be NULL per side. */
typedef struct kld_topk {
  int32_t *ids_ref;
  uint16_t *lp_ref;
  int32_t *ids_cand;
  uint16_t *lp_cand;
} kld_topk;

/* Optional launch options (any pointer may be NULL).  main_start/main_stop
 * are hipEvent_t handles recorded on `stream` immediately before and after the
 * call's dominant kernel (the streaming pass or the fused MFMA kernel), so a
 * caller can time that kernel alone. */
typedef struct kld_launch_opts {
  void *main_start;
  void *main_stop;
} kld_launch_opts;

/* Bytes of workspace an operation needs.  op is a KLD_OP_* code; flags may
 * hold KLD_FLAG_TOPK.  d is used by KLD_OP_FUSED_HEAD only; for
 * KLD_OP_SUMMARY, n is the number of positions; for KLD_OP_PAIRED, n is the
 * number of clusters and v the number of replicates.  Returns 0 for an
 * unknown op or negative sizes. */
size_t kld_workspace_size(int op, int64_t n, int64_t v, int64_t d, int flags);

/*
 * kld_from_logits -- score n positions given both logit tensors.
 *
 * ref, cand : [n, v] row-major logits (dtype f32 or bf16 bits), leading
 *             dimensions ld_ref, ld_cand >= v (in elements).  Element
 *             alignment suffices; 16-byte-aligned rows take the vector path.
 * target    : [n] int32 true next-token ids, or NULL (then nll_* must be NULL).
 * out       : per-position outputs (see kld_rows).
 * topk      : NULL, or top-64 export of both sides (needs v >= 64).
 * opts      : NULL, or launch options (timing events).
 * Definition: KL over all v ids per row ("Qwen3.8-27B fidelity suite v5",
 * opening paragraphs; "Qwen3.8-27B Quantization Challenge", "The score").
 */
kld_status kld_from_logits(const void *ref, const void *cand, int dtype, int64_t n, int64_t v,
                           int64_t ld_ref, int64_t ld_cand, const int32_t *target,
                           const kld_rows *out, const kld_topk *topk, void *ws, size_t ws_bytes,
                           void *stream, const kld_launch_opts *opts);

/*
 * kld_from_logits_noalloc -- kld_from_logits for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, outputs and results as
 * kld_from_logits, without the workspace: the library's own static device
 * buffer of KLD_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU serves instead, so the
 * call allocates nothing (no hipMalloc, no allocating library routine).
 *
 * Limit: a request whose kld_workspace_size(KLD_OP_FROM_LOGITS, n, v, 0,
 * flags) exceeds KLD_NOALLOC_SCRATCH_BYTES is rejected with KLD_ETOOBIG
 * before anything is launched (at v = 248,320: about 15,000 rows with top-64,
 * about 600,000 without).
 * The buffer belongs to the calling thread's current device, which must be
 * the device of `stream`.  Every call on one GPU shares that GPU's buffer:
 * calls that overlap on one GPU (concurrent streams or threads) race and
 * must be serialised by the caller.  The buffer is held until the process
 * ends.  The first call on a device looks up the buffer's address once.
 */
kld_status kld_from_logits_noalloc(const void *ref, const void *cand, int dtype, int64_t n,
                                   int64_t v, int64_t ld_ref, int64_t ld_cand,
                                   const int32_t *target, const kld_rows *out,
                                   const kld_topk *topk, void *stream,
                                   const kld_launch_opts *opts);

/*
 * kld_fused_head -- score n positions from final hidden states through one
 * shared bf16 head, without writing logits to memory ("Qwen3.8-27B fidelity
 * suite v5": opening paragraphs, one shared BF16 head for both sides;
 * "What is in here": hidden states [2047, 5120] bf16).
 *
 * W             : [v, d] bf16 head, row-major, contiguous.
 * h_ref, h_cand : [n, d] bf16 hidden states, row-major, contiguous.
 * Logits z = W h are accumulated in f32 from exact bf16 products and are not
 * rounded to bf16; the softmax is taken in f32.  d must be a multiple of 8
 * and at most 2^20 (KLD_ESHAPE otherwise).
 * target, out, topk, opts as for kld_from_logits.
 */
kld_status kld_fused_head(const uint16_t *W, int64_t v, int64_t d, const uint16_t *h_ref,
                          const uint16_t *h_cand, int64_t n, const int32_t *target,
                          const kld_rows *out, const kld_topk *topk, void *ws, size_t ws_bytes,
                          void *stream, const kld_launch_opts *opts);

/*
 * topk_export -- top-k ids and fp16 log-probs of one logit tensor, and the
 * log-prob of the true next token ("Qwopus3.8-27B-Coder-Flash: quality-eval
 * reference", "Files": <set>.ids int32, <set>.lp float16, <set>.target f32).
 *
 * logits    : [n, v] (dtype f32 or bf16 bits), leading dimension ld >= v.
 * k         : must be 64.  v >= 64.
 * ids, lp   : [n, 64] outputs (int32, fp16 bits).
 * target, target_lp : NULL, or [n] ids and [n] f32 log-prob outputs.
 */
kld_status topk_export(const void *logits, int dtype, int64_t n, int64_t v, int64_t ld, int k,
                       int32_t *ids, uint16_t *lp, const int32_t *target, float *target_lp,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * kld_topk_tail -- the top-64 + one-tail-bucket approximate KLD of the
 * quality-eval reference ("Method"), per position, from two exported lists.
 *
 * ids_p, lp_p : reference list [n, k] (int32 ids, fp16 log-prob bits).
 * ids_q, lp_q : candidate list [n, k].
 * k = 64; v > k is the vocabulary size.  kl_tail: [n] f32 output.
 * Cells: the reference's k ids plus one tail cell.  A reference id absent
 * from the candidate list gets r / (v - k), r = max(0, 1 - candidate list
 * mass); the candidate tail cell is max(0, 1 - sum of its cell estimates);
 * the reference tail is max(0, 1 - reference list mass).  0 ln(0/x) = 0,
 * p ln(p/0) = +inf.  Needs no workspace.
 */
kld_status kld_topk_tail(const int32_t *ids_p, const uint16_t *lp_p, const int32_t *ids_q,
                         const uint16_t *lp_q, int64_t n, int k, int64_t v, float *kl_tail,
                         void *stream);

/*
 * kld_summary -- aggregate per-position scores, every position weighted
 * equally ("Qwen3.8-27B Quantization Challenge", "The score": mean KL ranks,
 * with median, p99, p99.9, top-1 and the perplexity ratio).
 *
 * kl          : [n] per-position KL (required, values >= +0 or NaN/+inf).
 * argmax_ref/argmax_cand : [n] or both NULL.   nll_ref/nll_cand : [n] or both NULL.
 * quantiles   : HOST array of nq values in [0, 1], nq <= 16.
 * out         : DEVICE double[8 + nq]:
 *   [0] mean KL  [1] top-1 rate  [2] mean NLL ref  [3] mean NLL cand
 *   [4] ppl ref = exp(mean NLL ref)  [5] ppl cand  [6] ppl cand / ppl ref
 *   [7] count of non-finite KL values
 *   [8 + i] quantile i of KL: linear interpolation between exact order
 *           statistics (h = q (n - 1)); NaN values sort above +inf.
 * Entries whose inputs are NULL are written as NaN.
 */
kld_status kld_summary(const float *kl, const int32_t *argmax_ref, const int32_t *argmax_cand,
                       const float *nll_ref, const float *nll_cand, int64_t n,
                       const double *quantiles, int nq, double *out, void *ws, size_t ws_bytes,
                       void *stream);

/*
 * kld_golden_export -- the golden record of each reference row ("Qwen3.8-27B
 * Quantization Challenge", "Golden distributions": the 512 most likely
 * tokens exactly, most likely first, as {int32 id, float32 log p}, plus the
 * reference's NLL of the true next token, its entropy in nats and the tail
 * mass of the rest).
 *
 * logits : [n, v] reference logits (dtype f32 or bf16 bits), leading
 *          dimension ld >= v, v >= 512.
 * target : [n] true next-token ids, or NULL (then rec[i][0] = NaN).
 * k      : must be KLD_GOLDEN_TOPK (512).
 * ids    : [n, 512] int32 output: ids by probability, descending, ties to the
 *          lower id.
 * lp     : [n, 512] f32 output: log p = logit - lse of the listed ids.
 * rec    : [n, 3] f32 output: NLL of target (lse - logit[target]), entropy
 *          -sum_j p_j ln p_j over every id, and the tail mass: the sum of p
 *          over the ids outside the 512, summed directly (not 1 - the listed
 *          mass, which would drown a tiny tail in rounding).
 * Needs no workspace.  Rows holding NaN logits give unspecified records.
 */
kld_status kld_golden_export(const void *logits, int dtype, int64_t n, int64_t v, int64_t ld,
                             const int32_t *target, int k, int32_t *ids, float *lp, float *rec,
                             void *stream);

/*
 * kld_coarse_kl -- the 513-cell score of candidate rows against golden
 * records ("Qwen3.8-27B Quantization Challenge", "The score"): the
 * candidate's distribution q is coarsened onto the record's cells -- its 512
 * listed ids and one tail cell holding the rest of q's mass -- and
 * KL(p || q) = sum over the cells of p_i (ln p_i - ln q_i), with p_i =
 * exp(lp_i) and p_tail = rec[i][2] as stored.
 *
 * cand   : [n, v] candidate logits (dtype f32 or bf16 bits), ld >= v >= 512.
 * ids, lp, rec : the records as kld_golden_export writes them; ids distinct.
 * k      : must be KLD_GOLDEN_TOPK.
 * kl     : [n] f32 output.  A cell with p = 0 adds 0; p > 0 against q = 0
 *          gives +inf; a listed id outside [0, v) or a candidate row with a
 *          NaN or +inf logit gives NaN.
 * ws     : workspace of kld_workspace_size(KLD_OP_COARSE_KL, n, v, 0, 0) bytes.
 */
kld_status kld_coarse_kl(const void *cand, int dtype, int64_t n, int64_t v, int64_t ld,
                         const int32_t *ids, const float *lp, const float *rec, int k, float *kl,
                         void *ws, size_t ws_bytes, void *stream);

/*
 * kld_coarse_fused -- the 513-cell score of a candidate given as hidden
 * states against golden records ("Qwen3.8-27B Quantization Challenge", "The
 * score" and "Scoring an entry yourself": the candidate's log-softmax at every
 * position coarsened onto the record's 512 ids plus the tail; "Qwen3.8-27B
 * fidelity suite v5", opening paragraphs: candidate logits come from its
 * final hidden states through the one shared BF16 head).  The logits
 * z = W h_cand are reduced on the fly and never written to memory.
 *
 * W      : [v, d] bf16 head, row-major; v >= 512, d a multiple of 8.
 * h_cand : [n, d] bf16 candidate hidden states, row-major.
 * ids, lp, rec : golden records [n, 512] int32, [n, 512] f32, [n, 3] f32
 *          (kld_golden_export); a repeated id in a record counts in each of
 *          its cells, like kld_coarse_kl.
 * k      : must be KLD_GOLDEN_TOPK.
 * kl     : [n] f32 output: KL(p || q) over the 513 cells, q from the f32
 *          softmax of the f32-accumulated logits, the tail cell summed
 *          directly over the unlisted ids.  An id outside [0, v) gives NaN.
 * ws     : kld_workspace_size(KLD_OP_COARSE_FUSED, n, v, d, 0) bytes.
 * opts   : optional events around the head kernel, as for kld_fused_head.
 * W and h_cand need 16-byte alignment.
 */
kld_status kld_coarse_fused(const uint16_t *W, int64_t v, int64_t d, const uint16_t *h_cand,
                            int64_t n, const int32_t *ids, const float *lp, const float *rec, int k,
                            float *kl, void *ws, size_t ws_bytes, void *stream,
                            const kld_launch_opts *opts);

/*
 * kld_window_summary -- scored-window statistics of a per-position score
 * ("Qwen3.8-27B Quantization Challenge", "Golden distributions": the first
 * score_from positions of a document are not scored; "The score": the mean
 * over all positions and over a subset such as the long traces; "Qwen3.8-27B
 * fidelity suite v5": exact exceedance counts and the score_from 0 / 256 /
 * 1024 window control).
 *
 * kl         : [n] per-position scores (device).
 * offsets    : [nseg + 1] int64 (device): segment i (a window or document)
 *              covers positions offsets[i] .. offsets[i+1] - 1, nondecreasing
 *              within [0, n].
 * score_from : the first score_from positions of every segment are skipped.
 * thresholds : HOST array of nthr <= KLD_MAX_THRESHOLDS values.
 * seg_sum    : [nseg] f64 output, the sum of each segment's scored values
 *              (its mean is seg_sum / seg_count; the mean over a subset of
 *              segments is the sum of their sums over the sum of their counts).
 * seg_count  : [nseg] int64 output, scored positions per segment.
 * seg_exceed : [nseg, nthr] int64 output (row-major; may be NULL when
 *              nthr == 0): per segment, the scored positions whose score
 *              exceeds thresholds[t] (strictly).
 * totals     : [2 + nthr] f64 output: [0] mean over every scored position
 *              (each weighted equally), [1] their count, [2 + t] how many
 *              exceed thresholds[t] over every segment.
 * Needs no workspace.  A segment whose offsets break the rules gets seg_sum
 * NaN and count 0, and totals[0] is NaN.  Sums are taken in a fixed order
 * and nothing uses atomics: results are bitwise reproducible.
 */
kld_status kld_window_summary(const float *kl, int64_t n, const int64_t *offsets, int64_t nseg,
                              int64_t score_from, const float *thresholds, int nthr,
                              double *seg_sum, int64_t *seg_count, int64_t *seg_exceed,
                              double *totals, void *stream);

/*
 * kld_paired_bootstrap -- paired per-context comparison of two candidates
 * with a source-cluster bootstrap interval ("Qwen3.8-27B fidelity suite v5",
 * "Replay: score your own checkpoint against the published BF16 reference":
 * the difference of two reports' means paired per context, a 95 % interval
 * from a bootstrap over source clusters, the contexts each side wins and
 * the ties; "What these inputs measured": intervals over clusters).
 *
 * sum_a, sum_b : [nctx] f64 (device): per-context sums of the two
 *                candidates' per-position scores (seg_sum of
 *                kld_window_summary on each candidate's scores).
 * count        : [nctx] int64 (device): scored positions per context.
 * cluster      : [nctx] int32 (device): source cluster of each context,
 *                in [0, nclust), nclust <= 2^28.
 * draws        : [nrep, nclust] int32 (device), row-major: replicate r uses
 *                the clusters draws[r][0..nclust-1], drawn by the caller
 *                uniformly with replacement.
 * quantiles    : HOST array of nq <= KLD_MAX_QUANTILES levels in [0, 1]
 *                (0.025 and 0.975 give a 95 % interval).
 * replicates   : [nrep] f64 output (device), nrep <= KLD_MAX_REPLICATES:
 *                sum over the drawn clusters of (sum_a - sum_b) over the
 *                sum of their counts.
 * out          : [4 + nq] f64 output (device): [0] the difference
 *                sum_c (sum_a - sum_b) / sum_c count, [1] contexts where
 *                a's mean is lower, [2] where b's is lower, [3] ties
 *                (contexts with count 0 are in none), [4 + i] the type-7
 *                percentile of the replicates at quantiles[i].
 * ws           : kld_workspace_size(KLD_OP_PAIRED, nclust, nrep, 0, 0) bytes
 *                (an input-check flag, per-cluster sums and two copies of the
 *                replicates).
 * A cluster label outside [0, nclust) or a negative count makes out[0],
 * every replicate and every percentile NaN (the cluster sums are not valid);
 * a draw outside [0, nclust) makes that replicate NaN; any NaN replicate (or
 * none) makes every percentile NaN.  Sums run in a fixed order: results are
 * bitwise reproducible.
 */
kld_status kld_paired_bootstrap(const double *sum_a, const double *sum_b, const int64_t *count,
                                int64_t nctx, const int32_t *cluster, int64_t nclust,
                                const int32_t *draws, int64_t nrep, const double *quantiles,
                                int nq, double *replicates, double *out, void *ws,
                                size_t ws_bytes, void *stream);

/* Human-readable name of a status code (static string). */
const char *kld_status_str(int status);

/* KLD_ABI_VERSION of the built library. */
int kld_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBKLD_KLD_H */
