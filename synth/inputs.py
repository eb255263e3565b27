"""Seeded, row-addressable synthetic inputs.

Every logits row r of stream k for workload c is drawn from
``numpy.random.default_rng(SeedSequence([BASE_SEED, c, k, r]))`` so any
subset of rows can be regenerated on its own.  The head weight is drawn in
blocks of ``HEAD_BLOCK`` vocabulary rows and hidden states in blocks of
``HIDDEN_BLOCK`` positions (block b uses index b), so a row is regenerated
from its block.  All fused-head workloads share the head of the one-window
workload.  Rounding to bf16 is round-to-nearest-even from float32.

The shapes follow the pages' workloads: a 248,320-id vocabulary, hidden
width 5120, windows of 2048 tokens with 2047 scored positions, a 2.54 GB
bf16 head.  The value recipes (logit scale, boosted id, noise widths) are
this project's synthetic stand-ins for the models and corpora, which are
not available.
"""
from __future__ import annotations

import functools
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BASE_SEED = 20261203
VOCAB = 248_320
HIDDEN = 5120
WINDOW_POSITIONS = 2047

STREAM_BASE, STREAM_NOISE, STREAM_BOOST, STREAM_TARGET, STREAM_HEAD, STREAM_SUBSET = range(6)
STREAM_SCORES = 6
HEAD_BLOCK = 2048
HIDDEN_BLOCK = 256

# workload ids used as the second seed word
LOGITS_F32, FUSED_WINDOW, LOGITS_BF16_TOPK, FUSED_BATCH, LONG_TRACE = range(5)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def rng(workload: int, stream: int, index: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([BASE_SEED, workload, stream, index]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.reshape(-1).view(np.uint32)
    hi = u.view(np.uint16)[1::2]                  # upper halves (little-endian)
    bias = (hi & np.uint16(1)).astype(np.uint32) + np.uint32(0x7FFF)
    r = u + bias                                  # finite inputs: no wrap-around
    return r.view(np.uint16)[1::2].reshape(x.shape).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _pmap(fn, items):
    items = list(items)
    if len(items) <= 1:
        return [fn(i) for i in items]
    with ThreadPoolExecutor(_threads()) as ex:
        return list(ex.map(fn, items))


# --------------------------------------------------------------------------
# logits rows
# --------------------------------------------------------------------------

def logit_row_pair(workload: int, r: int, v: int, scale: float = 3.0, boost: float = 12.0,
                   noise: float = 0.03):
    """Reference row a = scale * N(0,1) with +boost on one uniformly drawn id;
    candidate row b = a + N(0, noise^2); both float32."""
    a = rng(workload, STREAM_BASE, r).standard_normal(v, dtype=np.float32)
    a *= np.float32(scale)
    j = int(rng(workload, STREAM_BOOST, r).integers(0, v))
    a[j] += np.float32(boost)
    b = a + np.float32(noise) * rng(workload, STREAM_NOISE, r).standard_normal(v, dtype=np.float32)
    return a, b.astype(np.float32)


def logit_rows(workload: int, rows, v: int, dtype: str = "f32", **kw):
    """Rows ``rows`` of the logits workload.  dtype 'f32' returns float32
    arrays; 'bf16' returns uint16 bit arrays (a and b rounded separately)."""
    rows = list(rows)
    a = np.empty((len(rows), v), np.float32 if dtype == "f32" else np.uint16)
    b = np.empty_like(a)

    def one(i):
        ra, rb = logit_row_pair(workload, rows[i], v, **kw)
        if dtype == "f32":
            a[i], b[i] = ra, rb
        else:
            a[i], b[i] = f32_to_bf16_bits(ra), f32_to_bf16_bits(rb)
    _pmap(one, range(len(rows)))
    return a, b


def targets(workload: int, rows, v: int) -> np.ndarray:
    """True next-token ids, uniform over [0, v), one seeded draw per row."""
    return np.array([int(rng(workload, STREAM_TARGET, r).integers(0, v)) for r in rows], np.int32)


# --------------------------------------------------------------------------
# fused head inputs
# --------------------------------------------------------------------------

@functools.lru_cache(maxsize=8)
def head_weight(workload: int, v: int, d: int, std: float = 0.02) -> np.ndarray:
    """Shared head W [v, d] as bf16 bits, W ~ N(0, std^2).  The array is
    cached because the full head takes tens of seconds to draw: callers must
    not modify it."""
    w = np.empty((v, d), np.uint16)

    def one(blk):
        j0 = blk * HEAD_BLOCK
        j1 = min(v, j0 + HEAD_BLOCK)
        z = rng(workload, STREAM_HEAD, blk).standard_normal((j1 - j0, d), dtype=np.float32)
        z *= np.float32(std)
        w[j0:j1] = f32_to_bf16_bits(z)
    _pmap(one, range((v + HEAD_BLOCK - 1) // HEAD_BLOCK))
    return w


def _hidden_block(workload: int, blk: int, d: int, noise):
    """Positions blk*HIDDEN_BLOCK .. +HIDDEN_BLOCK-1: h = N(0,1) rows scaled to
    unit RMS (float32); reference = bf16(h), candidate = bf16(h + N(0, s^2))
    with s = noise(row) (or the constant noise)."""
    r0 = blk * HIDDEN_BLOCK
    z = rng(workload, STREAM_BASE, blk).standard_normal((HIDDEN_BLOCK, d), dtype=np.float32)
    rms = np.sqrt(np.mean(np.square(z, dtype=np.float64), axis=1, keepdims=True)).astype(np.float32)
    h = (z / rms).astype(np.float32)
    e = rng(workload, STREAM_NOISE, blk).standard_normal((HIDDEN_BLOCK, d), dtype=np.float32)
    if callable(noise):
        s = np.array([noise(r0 + i) for i in range(HIDDEN_BLOCK)], np.float32)[:, None]
    else:
        s = np.float32(noise)
    hc = (h + s * e).astype(np.float32)
    return f32_to_bf16_bits(h), f32_to_bf16_bits(hc)


def hidden_rows(workload: int, rows, d: int, noise) -> tuple:
    """Hidden-state rows (bf16 bits) for the given positions; ``noise`` is a
    float or a callable position -> std."""
    rows = np.asarray(list(rows), np.int64)
    hr = np.empty((len(rows), d), np.uint16)
    hc = np.empty_like(hr)
    blocks = np.unique(rows // HIDDEN_BLOCK) if len(rows) else np.zeros(0, np.int64)

    def one(blk):
        br, bc = _hidden_block(workload, int(blk), d, noise)
        sel = np.nonzero(rows // HIDDEN_BLOCK == blk)[0]
        hr[sel] = br[rows[sel] - blk * HIDDEN_BLOCK]
        hc[sel] = bc[rows[sel] - blk * HIDDEN_BLOCK]
    _pmap(one, blocks)
    return hr, hc


def long_trace_noise(row: int, chunk_rows: int = 8192, n_chunks: int = 32) -> float:
    """Candidate noise for the long-trace workload: linear sweep over chunks,
    0.005 for the first chunk up to 0.05 for the last."""
    c = min(row // chunk_rows, n_chunks - 1)
    return 0.005 + c * (0.045 / (n_chunks - 1))


def subset(workload: int, n: int, m: int) -> np.ndarray:
    """A seeded sorted subset of m distinct row indices out of n."""
    g = rng(workload, STREAM_SUBSET, 0)
    return np.sort(g.choice(n, size=min(m, n), replace=False)).astype(np.int64)


def kl_scores(workload: int, n: int, median: float = 0.02, sigma: float = 1.6) -> np.ndarray:
    """n seeded per-position scores (float32), lognormal with the given
    median: mostly small values with a heavy upper tail, the shape of a
    per-position KL stream; about one value in a thousand is exactly zero."""
    g = rng(workload, STREAM_SCORES, 0)
    x = (median * np.exp(sigma * g.standard_normal(n))).astype(np.float32)
    x[g.random(n) < 1e-3] = 0.0
    return x


def doc_offsets(workload: int, lengths) -> np.ndarray:
    """Segment offsets [len(lengths) + 1] (int64) for segments of the given
    lengths laid end to end, in a seeded shuffled order."""
    g = rng(workload, STREAM_SCORES, 1)
    lens = np.asarray(lengths, np.int64)[g.permutation(len(lengths))]
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def kl_score_pair(workload: int, n: int, spread: float = 0.1) -> tuple:
    """Two candidates' per-position scores over the same n positions: the
    first as kl_scores, the second the first times exp(spread * N(0, 1))
    (two close candidates, paired by position)."""
    a = kl_scores(workload, n)
    g = rng(workload, STREAM_SCORES, 2)
    b = (a * np.exp(spread * g.standard_normal(n))).astype(np.float32)
    return a, b


def cluster_labels(workload: int, nctx: int, nclust: int) -> np.ndarray:
    """Source-cluster label (int32) of each of nctx contexts: every one of the
    nclust clusters holds at least one context, the rest are uniform."""
    g = rng(workload, STREAM_SCORES, 3)
    lab = np.concatenate([np.arange(nclust), g.integers(0, nclust, max(nctx - nclust, 0))])
    return g.permutation(lab)[:nctx].astype(np.int32)


def bootstrap_draws(workload: int, nrep: int, nclust: int) -> np.ndarray:
    """Bootstrap draws [nrep, nclust] (int32): each row nclust cluster ids
    drawn uniformly with replacement."""
    g = rng(workload, STREAM_SCORES, 4)
    return g.integers(0, nclust, (nrep, nclust)).astype(np.int32)


def sparse_records(workload: int, n: int, v: int, k: int = 512) -> tuple:
    """n seeded stand-in records for scoring against stored sparse
    references: k distinct ids per row (uniform over [0, v)), f32 log-probs
    of a random distribution over them that leaves a tail mass in [0.05, 0.6)
    for the rest, and [n, 3] f32 (NaN, NaN, tail).  Used where every row of a
    large launch needs a record but only sampled rows are checked."""
    g = rng(workload, STREAM_SCORES, 5)
    ids = np.empty((n, k), np.int32)
    lp = np.empty((n, k), np.float32)
    rec = np.full((n, 3), np.nan, np.float32)
    for i in range(n):
        ids[i] = g.choice(v, size=k, replace=False)
        w = g.exponential(1.0, k) ** 3
        tail = g.uniform(0.05, 0.6)
        lp[i] = np.log(w / w.sum() * (1.0 - tail))
        rec[i, 2] = tail
    return ids, lp, rec
