"""Plain f64 CPU oracle for full-vocabulary KL scoring.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
module: only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library (no kernels, headers, helpers or constants) and it imports
nothing from the ``full_vocab_kl_amd`` package.

Every function is the plain definition of one quantity, written in numpy
float64 with no blocking, fusion or reordering beyond what the definition
states.  Sources are cited by page title and section:

* [QC]  "Qwen3.8-27B Quantization Challenge" (dataset card):
        sections "How the references were made", "Golden distributions",
        "The score", "Scoring an entry yourself".
* [FS]  "Qwen3.8-27B fidelity suite v5 -- evaluation inputs, the BF16
        reference, and every per-shard report": opening paragraphs (the
        metric definition through one shared BF16 LM head) and "What is in
        here" (hidden-state shapes).
* [QE]  "Qwopus3.8-27B-Coder-Flash: quality-eval reference": sections
        "Files" (top-64 export layout) and "Method" (top-64 + tail bucket
        KLD, top-1, perplexity).
* [IQ]  "Qwen3.8-27B IQ8R (GPTQ int8, Hadamard-rotated)": section
        "Quality" (mean / 99 % / 99.9 % KLD, top-1).

Readings where the pages are silent (each also listed in the design notes):

* R1  ties in argmax and top-k are broken toward the lower vocabulary id.
* R2  percentiles use linear interpolation between order statistics
      (Hyndman-Fan type 7).
* R3  in the top-64 + tail rule the candidate's tail cell is the complement
      1 - sum over the reference ids of the candidate's per-id estimates.
* R4  the reference tail mass p_T comes from the exported fp16 top-64
      log-probs (the export stores no tail mass).
* R5  fused-path logits are not rounded to bf16: products of the bf16
      operands are summed exactly (f64 here) and the softmax is taken on
      those sums.
* R6  a finite reference logit against a -inf candidate logit makes KL
      +inf; a reference logit of -inf contributes nothing; a row whose
      reference or candidate logits are all -inf, or that holds a NaN or
      +inf, has KL = NaN.
* R7  NLL of a target id outside [0, V) is NaN.
* R8  argmax ignores NaN entries; a row of only NaN reports id 0.
* R14 the golden record's tail mass is the mass of the ids outside the
      top-K, summed over those ids of the full row (equal to 1 - sum of the
      listed probabilities in exact arithmetic, but free of its
      cancellation when the tail is tiny).
* R15 the 513-cell score takes p from the stored record (the f32 log-probs
      of the listed ids and the stored tail mass) and q from the candidate's
      full row: q of a listed id is its softmax probability, q's tail cell
      the candidate mass of every unlisted id.
* R16 score_from skips the first score_from positions of every segment
      (window or document); a segment shorter than that scores nothing; an
      exceedance is a score strictly above the threshold.
* R17 the paired difference of two candidates is position-weighted, mean(a)
      - mean(b) over the scored positions of the contexts both were scored
      on (with equal scored positions per context, as in the pages' shard,
      this is also the mean of the per-context differences); a context is
      won by the candidate with the strictly lower per-context mean.
* R18 the source-cluster bootstrap resamples clusters: each replicate draws
      as many cluster ids as there are clusters, uniformly with replacement,
      and recomputes R17's statistic over the drawn clusters' contexts (a
      cluster drawn twice counts twice); the interval is the percentile
      interval of the replicates by R2 (2.5 % and 97.5 % for a 95 %
      interval).  The draws are an input: the pages give neither the
      generator nor the replicate count (10,000 is used here).

Parity is pinned for every function here by the ``-m "not gpu"`` tests
(tests/test_oracle_pins.py); no function is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

TOPK = 64

# --------------------------------------------------------------------------
# exact decoding of the storage formats
# --------------------------------------------------------------------------


def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns exactly: a bf16 value is the upper half of
    an IEEE binary32, so shifting its 16 bits left by 16 gives that binary32,
    which widens to binary64 without rounding."""
    u16 = np.asarray(u16, dtype=np.uint16)
    return (u16.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def fp16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    """Decode IEEE binary16 bit patterns exactly (binary16 widens exactly)."""
    return np.asarray(u16, dtype=np.uint16).view(np.float16).astype(np.float64)


def f64_to_fp16_bits(x: np.ndarray) -> np.ndarray:
    """Round binary64 to binary16, round-to-nearest-even, and return the bits.

    numpy converts double to half directly (one rounding, ties to even),
    which the pins check on hand-built halfway cases."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


# --------------------------------------------------------------------------
# per-row definitions
# --------------------------------------------------------------------------


def _row_is_bad(x: np.ndarray) -> bool:
    return bool(np.isnan(x).any() or np.isposinf(x).any() or not np.isfinite(x).any())


def logsumexp(x: np.ndarray) -> float:
    """O1: lse(x) = m + ln sum_j exp(x_j - m), m = max_j x_j.

    [QC] "How the references were made": each position's distribution over
    the full vocabulary, in natural-log units; the log-softmax of a row is
    x - lse(x) ([QC] "Scoring an entry yourself")."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any() or np.isposinf(x).any():
        return float("nan")
    m = x.max()
    if m == -np.inf:
        return -math.inf
    return float(m + np.log(np.sum(np.exp(x - m))))


def kl_row(a: np.ndarray, b: np.ndarray) -> float:
    """O2: KL(p || q) = sum_j p_j (ln p_j - ln q_j), p = softmax(a) (reference),
    q = softmax(b) (candidate), summed over every vocabulary id.

    [FS] opening paragraph: the metric is KL(BF16 || candidate); [QC] "The
    score": the sum over cells of p_i (log p_i - log q_i), here with every
    vocabulary id as its own cell; [QE] "Method": KL(BF16 || quant) per
    position.  Edge cases follow reading R6."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if _row_is_bad(a) or _row_is_bad(b):
        return float("nan")
    lse_a = logsumexp(a)
    lse_b = logsumexp(b)
    support = a > -np.inf                      # p_j > 0 exactly where a_j is finite
    if np.any(support & (b == -np.inf)):       # p_j > 0 and q_j = 0
        return math.inf
    la = a[support] - lse_a
    lb = b[support] - lse_b
    p = np.exp(la)
    return float(np.sum(p * (la - lb)))


def argmax_row(x: np.ndarray) -> int:
    """O3: the smallest id j with x_j equal to the row maximum (reading R1).

    [QE] "Method": top-1 agreement is an exact argmax match; [QC] "The
    score": the leaderboard's top-1 agreement (argmax match)."""
    x = np.asarray(x, dtype=np.float64)
    ok = ~np.isnan(x)                          # reading R8: NaN ids never win
    if not ok.any():
        return 0
    m = x[ok].max()
    return int(np.flatnonzero(x == m)[0])


def nll_row(x: np.ndarray, target: int) -> float:
    """O4: NLL of the true next token = lse(x) - x_target (reading R7 for ids
    outside the vocabulary).

    [QE] "Method": perplexity is exp(mean NLL) of the true next token;
    [QE] "Files": the stored target log-prob of the true next token;
    [QC] "Golden distributions": the reference's NLL of the true next token."""
    x = np.asarray(x, dtype=np.float64)
    if target < 0 or target >= x.shape[0]:
        return float("nan")
    return float(logsumexp(x) - x[target])


def topk_row(x: np.ndarray, k: int = TOPK):
    """O6: the k most likely ids, most likely first, ties to the lower id
    (reading R1), with log-probs x_j - lse(x) rounded to fp16 (nearest-even).

    [QE] "Files": top-64 ids int32 and log-probs float16, sorted; [QC]
    "Golden distributions": the most likely tokens, most likely first.
    Returns (ids int32 [k], lp fp16 bits uint16 [k], lp f64 [k] unrounded)."""
    x = np.asarray(x, dtype=np.float64)
    ids = np.arange(x.shape[0])
    order = np.lexsort((ids, -x))              # primary key -x, then id ascending
    top = order[:k]
    lp = x[top] - logsumexp(x)
    return top.astype(np.int32), f64_to_fp16_bits(lp), lp


def tail_kld_probs(ids_p, p, ids_q, q, v: int) -> float:
    """O7: top-K + one-tail-bucket KLD of the quality-eval reference, on
    probabilities.

    [QE] "Method": the divergence is taken over 65 cells -- the reference's
    64 listed ids and one cell for all other ids.  When a reference id is
    absent from the candidate's list, its candidate probability is an equal
    share of the mass the candidate's list leaves over, divided among the
    ids that list does not name.  With K = len(ids_q) (the candidate list
    length):

      1. p_i for i in P; p_T = max(0, 1 - sum_P p_i)                  (R4)
      2. r = max(0, 1 - sum_{j in Q} q_j); u = r / (V - K)
      3. qhat_i = q_i if i in Q else u
      4. qhat_T = max(0, 1 - sum_{i in P} qhat_i)                     (R3)
      5. KL = sum_{i in P} p_i ln(p_i/qhat_i) + p_T ln(p_T/qhat_T),
         with 0 ln(0/x) = 0 and p ln(p/0) = +inf for p > 0.
    """
    ids_p = np.asarray(ids_p, dtype=np.int64)
    ids_q = np.asarray(ids_q, dtype=np.int64)
    p = np.asarray(p, dtype=np.float64)
    qv = np.asarray(q, dtype=np.float64)
    k = ids_q.shape[0]
    p_tail = max(0.0, 1.0 - float(np.sum(p)))
    r = max(0.0, 1.0 - float(np.sum(qv)))
    u = r / (v - k) if v > k else 0.0
    q_of = {int(j): float(qj) for j, qj in zip(ids_q, qv)}
    qhat = np.array([q_of.get(int(i), u) for i in ids_p], dtype=np.float64)
    q_tail = max(0.0, 1.0 - float(np.sum(qhat)))
    total = 0.0
    for pi, qi in zip(np.append(p, p_tail), np.append(qhat, q_tail)):
        if pi == 0.0:
            continue
        if qi == 0.0:
            return math.inf
        total += pi * math.log(pi / qi)
    return total


def tail_kld_row(ids_p, lp_p_bits, ids_q, lp_q_bits, v: int) -> float:
    """O7 on the export format: fp16 log-prob bits are decoded exactly and
    exponentiated in f64 ([QE] "Files": top-64 ids int32 and log-probs
    float16), then :func:`tail_kld_probs`."""
    p = np.exp(fp16_bits_to_f64(lp_p_bits))
    q = np.exp(fp16_bits_to_f64(lp_q_bits))
    return tail_kld_probs(ids_p, p, ids_q, q, v)


# --------------------------------------------------------------------------
# fused head: logits from hidden states through one shared head
# --------------------------------------------------------------------------


def head_logits(w_bits: np.ndarray, h_bits: np.ndarray, v_chunk: int = 8192) -> np.ndarray:
    """O8: z[i, j] = sum_k W[j, k] h[i, k] in f64 from bf16-decoded operands.

    [FS] opening paragraph: both sides' logits are produced by applying one
    and the same bf16 output head to each side's final hidden states; "What
    is in here": hidden states are [positions, 5120] bf16.  Reading R5: the sums are
    not rounded to bf16.  Each product of two bf16 values is exact in f64;
    the matmul routine sums them in f64.  Returns f64 [n, V]; the head is
    decoded ``v_chunk`` rows at a time only to bound memory."""
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    h = bf16_bits_to_f64(h_bits)
    n, v = h.shape[0], w_bits.shape[0]
    out = np.empty((n, v), dtype=np.float64)
    for j0 in range(0, v, v_chunk):
        wj = bf16_bits_to_f64(w_bits[j0:j0 + v_chunk])
        out[:, j0:j0 + v_chunk] = h @ wj.T
    return out


# --------------------------------------------------------------------------
# whole-row scoring and aggregation
# --------------------------------------------------------------------------


def score_rows(a: np.ndarray, b: np.ndarray, target=None, k: int | None = None) -> dict:
    """Per-position scores for logit rows a (reference) and b (candidate),
    each [n, V] (any float dtype; promoted to f64).

    Returns kl, lse_ref, lse_cand, argmax_ref, argmax_cand, nll_ref,
    nll_cand (NaN where no target is given), and with k: top-k ids / fp16
    lp bits per side."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    n = a.shape[0]
    out = {
        "kl": np.empty(n), "lse_ref": np.empty(n), "lse_cand": np.empty(n),
        "argmax_ref": np.empty(n, np.int64), "argmax_cand": np.empty(n, np.int64),
        "nll_ref": np.full(n, np.nan), "nll_cand": np.full(n, np.nan),
    }
    if k is not None:
        for s in ("ref", "cand"):
            out[f"ids_{s}"] = np.empty((n, k), np.int32)
            out[f"lp_{s}"] = np.empty((n, k), np.uint16)
    for i in range(n):
        out["kl"][i] = kl_row(a[i], b[i])
        out["lse_ref"][i] = logsumexp(a[i])
        out["lse_cand"][i] = logsumexp(b[i])
        out["argmax_ref"][i] = argmax_row(a[i])
        out["argmax_cand"][i] = argmax_row(b[i])
        if target is not None:
            out["nll_ref"][i] = nll_row(a[i], int(target[i]))
            out["nll_cand"][i] = nll_row(b[i], int(target[i]))
        if k is not None:
            for s, x in (("ref", a[i]), ("cand", b[i])):
                ids, lp, _ = topk_row(x, k)
                out[f"ids_{s}"][i] = ids
                out[f"lp_{s}"][i] = lp
    return out


GOLDEN_TOPK = 512


def golden_row(x: np.ndarray, target=None, k: int = GOLDEN_TOPK):
    """The golden record of one reference position ([QC] "Golden
    distributions": the k most likely tokens exactly, most likely first, as
    {int32 id, f32 log p}, plus the NLL of the true next token, the entropy
    in nats and the tail mass of the rest).

    Ids follow O6 (ties to the lower id, reading R1); lp = x_j - lse(x) in f64,
    rounded once to f32; entropy = -sum_j p_j ln p_j over every id with
    p_j > 0; tail = sum of p_j over the ids outside the top k (reading R14);
    nll per O4 (NaN without a target).  Returns (ids int32 [k], lp f32 [k],
    rec f32 [3] = (nll, entropy, tail))."""
    x = np.asarray(x, dtype=np.float64)
    v = x.shape[0]
    lse = logsumexp(x)
    order = np.lexsort((np.arange(v), -x))
    top, rest = order[:k], order[k:]
    lp = (x[top] - lse).astype(np.float32)
    pos = x > -np.inf
    logp = x[pos] - lse
    entropy = float(-np.sum(np.exp(logp) * logp))
    tail = float(np.sum(np.exp(x[rest] - lse)))
    nll = nll_row(x, int(target)) if target is not None else float("nan")
    rec = np.array([nll, entropy, tail], dtype=np.float32)
    return top.astype(np.int32), lp, rec


def coarse_kl_row(ids, lp, tail, b: np.ndarray) -> float:
    """The score of one position against a golden record ([QC] "The score"):
    the candidate's distribution q is coarsened onto the record's cells --
    its listed ids and one tail cell with the rest of q's mass -- and
    KL(p || q) = sum over the cells of p_i (ln p_i - ln q_i).

    p_i = exp(lp_i) for the listed ids and p_T = tail (the stored record,
    reading R15); q_i = softmax(b)_i and q_T = the sum of softmax(b) over the
    unlisted ids.  A cell with p = 0 adds 0; p > 0 against q = 0 gives +inf."""
    b = np.asarray(b, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    lse_b = logsumexp(b)
    lq = b - lse_b
    listed = np.zeros(b.shape[0], dtype=bool)
    listed[ids] = True
    q_t = float(np.sum(np.exp(lq[~listed])))
    lp = np.asarray(lp, dtype=np.float64)
    p = np.exp(lp)
    total = 0.0
    for pi, lpi, lqi in zip(p, lp, lq[ids]):
        if pi == 0.0:
            continue
        if lqi == -np.inf:
            return math.inf
        total += pi * (lpi - lqi)
    p_t = float(tail)
    if p_t > 0.0:
        if q_t == 0.0:
            return math.inf
        total += p_t * (math.log(p_t) - math.log(q_t))
    return float(total)


def golden_rows(x: np.ndarray, target=None, k: int = GOLDEN_TOPK) -> dict:
    """golden_row over the rows of x [n, V]: ids [n, k], lp [n, k], rec [n, 3]."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    out = {"ids": np.empty((n, k), np.int32), "lp": np.empty((n, k), np.float32),
           "rec": np.empty((n, 3), np.float32)}
    for i in range(n):
        t = None if target is None else int(target[i])
        out["ids"][i], out["lp"][i], out["rec"][i] = golden_row(x[i], t, k)
    return out


def coarse_kl_rows(ids, lp, rec, b: np.ndarray) -> np.ndarray:
    """coarse_kl_row over the rows of b [n, V] against records (ids, lp, rec)."""
    b = np.asarray(b, dtype=np.float64)
    return np.array([coarse_kl_row(ids[i], lp[i], float(rec[i][2]), b[i])
                     for i in range(b.shape[0])])


def window_summary(kl, offsets, score_from: int, thresholds=()) -> dict:
    """Scored-window statistics over segments (windows or documents) of a
    per-position score array.

    Segment i covers positions offsets[i] .. offsets[i+1] - 1; its first
    score_from positions are not scored (reading R16; [QC] "Golden distributions": a
    document of T tokens has T - 1 - score_from scored rows, row j predicting
    token score_from + j + 1; [FS] "What these inputs measured": the
    scored-window control with score_from 0 / 256 / 1024).  Per segment: the
    sum and count of the scored values (its mean is sum / count); overall:
    the mean over every scored position, weighted equally ([QC] "The score":
    the mean over all positions, and the mean over a subset of them such as
    the 256K-token traces), and for each threshold the exact count of scored
    positions whose score exceeds it ([FS] "What is in here": percentiles and
    exact exceedance counts)."""
    kl = np.asarray(kl, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    nseg = offsets.shape[0] - 1
    seg_sum = np.zeros(nseg)
    seg_count = np.zeros(nseg, np.int64)
    seg_exceed = np.zeros((nseg, len(thresholds)), np.int64)
    for i in range(nseg):
        x = kl[offsets[i] + score_from: offsets[i + 1]] if offsets[i] + score_from < offsets[i + 1] \
            else kl[0:0]
        seg_sum[i] = float(np.sum(x))
        seg_count[i] = x.shape[0]
        for t, thr in enumerate(thresholds):
            seg_exceed[i, t] = int(np.sum(x > thr))
    total = int(seg_count.sum())
    return {"seg_sum": seg_sum, "seg_count": seg_count, "seg_exceed": seg_exceed,
            "mean": float(seg_sum.sum() / total) if total else float("nan"), "count": total,
            "exceed": seg_exceed.sum(axis=0)}



def paired_bootstrap(sum_a, sum_b, count, cluster, draws, quantiles=(0.025, 0.975)) -> dict:
    """Paired per-context comparison of two candidates with a source-cluster
    bootstrap interval ([FS] "Replay: score your own checkpoint against the
    published BF16 reference": two reports compared per context give the
    difference of their means, a 95 % bootstrap interval over source
    clusters and how many contexts each side wins, with ties; "What these
    inputs measured": bootstrap intervals over clusters).

    Context c has sum_a[c] and sum_b[c], the sums of the two candidates'
    per-position scores over its count[c] scored positions, and belongs to
    source cluster cluster[c] in [0, K).  Reading R17: the difference is
    sum_c (sum_a[c] - sum_b[c]) / sum_c count[c]; context c is won by a when
    sum_a[c] / count[c] < sum_b[c] / count[c], by b when the reverse holds,
    and tied when the two means are equal.  Reading R18: replicate r takes
    the clusters draws[r, 0..K-1] (ids drawn with replacement) and computes
    the same difference over the contexts of those clusters, each cluster
    as often as it was drawn; the interval is percentile(replicates, q)
    by R2 for each q.  Returns diff, a_wins, b_wins, ties, replicates and
    the list of quantiles."""
    sum_a = np.asarray(sum_a, dtype=np.float64)
    sum_b = np.asarray(sum_b, dtype=np.float64)
    count = np.asarray(count, dtype=np.int64)
    cluster = np.asarray(cluster, dtype=np.int64)
    draws = np.asarray(draws, dtype=np.int64)
    nctx = sum_a.shape[0]
    n_clusters = draws.shape[1] if draws.ndim == 2 else 0
    total = int(count.sum())
    diff = float(np.sum(sum_a - sum_b) / total) if total else float("nan")
    mean_a = sum_a / np.where(count > 0, count, 1)
    mean_b = sum_b / np.where(count > 0, count, 1)
    scored = count > 0
    a_wins = int(np.sum(scored & (mean_a < mean_b)))
    b_wins = int(np.sum(scored & (mean_b < mean_a)))
    ties = int(np.sum(scored & (mean_a == mean_b)))
    # each cluster's summed difference and scored positions
    clus_diff = np.zeros(n_clusters)
    clus_count = np.zeros(n_clusters, np.int64)
    for c in range(nctx):
        clus_diff[cluster[c]] += sum_a[c] - sum_b[c]
        clus_count[cluster[c]] += count[c]
    reps = np.empty(draws.shape[0])
    for r in range(draws.shape[0]):
        num = 0.0
        den = 0
        for k in draws[r]:
            num += clus_diff[k]
            den += clus_count[k]
        reps[r] = num / den if den else float("nan")
    if reps.shape[0] and not np.isnan(reps).any():
        qs = [percentile(reps, q) for q in quantiles]
    else:
        qs = [float("nan")] * len(quantiles)
    return {"diff": diff, "a_wins": a_wins, "b_wins": b_wins, "ties": ties,
            "replicates": reps, "quantiles": qs}

def percentile(x: np.ndarray, q: float) -> float:
    """O5 percentile by reading R2 (linear interpolation, type 7): sort
    ascending, h = q (N - 1), value = x_(floor h) + (h - floor h) *
    (x_(floor h + 1) - x_(floor h)).

    [QC] "The score": the leaderboard shows the median, p99 and p99.9 KL;
    [IQ] "Quality": KLD 99 % and 99.9 %; [QE] "v1.0 at a glance": median
    and p99."""
    xs = np.sort(np.asarray(x, dtype=np.float64))
    n = xs.shape[0]
    h = q * (n - 1)
    lo = int(math.floor(h))
    hi = min(lo + 1, n - 1)
    return float(xs[lo] + (h - lo) * (xs[hi] - xs[lo]))


def summarize(kl, argmax_ref=None, argmax_cand=None, nll_ref=None, nll_cand=None,
              quantiles=(0.5, 0.99, 0.999)) -> dict:
    """Aggregate per-position scores, every position weighted equally.

    [QC] "The score": mean KL over all positions ranks entries, with median,
    p99, p99.9, top-1 agreement and the perplexity ratio; [QE] "Method":
    perplexity = exp(mean NLL) of the true next token."""
    kl = np.asarray(kl, dtype=np.float64)
    n = kl.shape[0]
    res = {"n": n, "mean_kl": float(np.sum(kl) / n)}
    if argmax_ref is not None and argmax_cand is not None:
        res["top1"] = float(np.sum(np.asarray(argmax_ref) == np.asarray(argmax_cand)) / n)
    if nll_ref is not None and nll_cand is not None:
        mr = float(np.sum(np.asarray(nll_ref, np.float64)) / n)
        mc = float(np.sum(np.asarray(nll_cand, np.float64)) / n)
        res.update(mean_nll_ref=mr, mean_nll_cand=mc, ppl_ref=math.exp(mr),
                   ppl_cand=math.exp(mc), ppl_ratio=math.exp(mc) / math.exp(mr))
    res["quantiles"] = {float(q): percentile(kl, q) for q in quantiles}
    return res
