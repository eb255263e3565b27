"""GPU parity of the golden records (kld_golden_export: 512 listed ids with
f32 log-probs, NLL, entropy, tail mass) and of the 513-cell coarsened score
(kld_coarse_kl) against the f64 oracle.  The score is checked on records the
oracle wrote, so no GPU output feeds the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
import full_vocab_kl_amd as kld
from gpu_util import gpu, need_gpu, to_dev

pytestmark = gpu
K = oracle.GOLDEN_TOPK


def _lp_tol(want):
    # lp = z - lse: the f32 rounding of the result (a few ulp of |lp|) plus
    # the error of the f32-summed log-sum-exp (below 1e-6 here)
    return 4 * np.spacing(np.abs(want).astype(np.float32)).astype(np.float64) + 1e-6


def _check_records(got, want, where):
    assert np.array_equal(got["ids"], want["ids"]), f"{where}: ids"
    g, w = got["lp"].astype(np.float64), want["lp"].astype(np.float64)
    fin = np.isfinite(w)
    assert np.array_equal(np.isfinite(g), fin), f"{where}: lp finiteness"
    bad = np.abs(g[fin] - w[fin]) > _lp_tol(w[fin])
    assert not bad.any(), f"{where}: lp off at {np.argwhere(bad)[:4]}"
    gr, wr = got["rec"].astype(np.float64), want["rec"].astype(np.float64)
    # NLL and entropy: 1e-5 relative to max(1, value); NaN where no target
    for c, name in ((0, "nll"), (1, "entropy")):
        assert np.array_equal(np.isnan(gr[:, c]), np.isnan(wr[:, c])), f"{where}: {name} NaN"
        assert np.array_equal(np.isposinf(gr[:, c]), np.isposinf(wr[:, c])), f"{where}: {name} inf"
        ok = np.isfinite(wr[:, c])
        err = np.abs(gr[ok, c] - wr[ok, c])
        assert np.all(err <= 1e-5 * np.maximum(1.0, np.abs(wr[ok, c]))), f"{where}: {name} {err.max()}"
    # tail mass: summed directly on both sides, 1e-4 relative
    err = np.abs(gr[:, 2] - wr[:, 2])
    assert np.all(err <= 1e-4 * wr[:, 2] + 1e-12), f"{where}: tail {err.max()} at {wr[:, 2][np.argmax(err)]}"


def _run_export(a, bf16, target=None, pad=0):
    n, v = a.shape
    if pad:
        pa = np.zeros((n, v + pad), a.dtype); pa[:, :v] = a
        da = to_dev(pa, bf16)[:, :v]
    else:
        da = to_dev(a, bf16)
    out = kld.kld_golden_export(da, None if target is None else to_dev(target))
    torch.cuda.synchronize()
    return {k: x.cpu().numpy() for k, x in out.items()}


def _decode(a, bf16):
    return oracle.bf16_bits_to_f64(a) if bf16 else np.asarray(a, np.float64)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("n,v,pad", [(3, 512, 0), (4, 1000, 0), (2, 33000, 8), (3, 70001, 0),
                                     (5, 4099, 1)])
def test_golden_export_shapes(n, v, pad, bf16):
    need_gpu()
    print(f"golden n={n} v={v} pad={pad} bf16={bf16}", flush=True)
    a, _ = synth.logit_rows(synth.LOGITS_F32, range(n), v)
    if bf16:
        a = synth.f32_to_bf16_bits(a)
    t = synth.targets(synth.LOGITS_F32, range(n), v)
    got = _run_export(a, bf16, t, pad)
    want = oracle.golden_rows(_decode(a, bf16), t)
    _check_records(got, want, f"n={n} v={v}")


def test_golden_export_adversarial():
    need_gpu()
    v = 9000
    g = np.random.default_rng(3)
    rows = [np.arange(v, dtype=np.float32) * 1e-3,             # every element a new maximum
            -np.arange(v, dtype=np.float32) * 1e-3,
            np.full(v, 1.5, np.float32),                       # all equal: ids 0..511
            np.round(g.normal(0, 1, v), 1).astype(np.float32),  # heavy ties
            np.where(np.arange(v) % 7 == 0, -np.inf, g.normal(0, 2, v)).astype(np.float32)]
    a = np.stack(rows)
    t = np.array([5, v - 1, 0, -3, 7], np.int32)               # -3: no such id -> NaN NLL
    got = _run_export(a, False, t)
    want = oracle.golden_rows(a.astype(np.float64), t)
    _check_records(got, want, "adversarial")
    assert list(got["ids"][2]) == list(range(K))
    assert np.isnan(got["rec"][3, 0])


def test_golden_export_repeatable():
    """Repeated exports of the same rows are bitwise identical: 192 f32 rows
    of the 512-row logits workload at V = 248,320 and the all-equal row
    (every id a candidate, so the buffer is cut several times), each exported
    four times.  (The candidate buffer fills in whatever order the threads
    append, so the mass of the keys a cut drops must be summed in a way that
    order cannot change.)"""
    need_gpu()
    n, v = 192, synth.VOCAB
    a, _ = synth.logit_rows(synth.LOGITS_F32, range(n), v)
    a = np.concatenate([a, np.full((1, v), 1.5, np.float32)])
    t = synth.targets(synth.LOGITS_F32, range(n + 1), v)
    da, dt = to_dev(a, False), to_dev(t)
    first = None
    for rep in range(4):
        print(f"golden repeat {rep}", flush=True)
        out = kld.kld_golden_export(da, dt)
        torch.cuda.synchronize()
        got = {k: x.cpu().numpy() for k, x in out.items()}
        if first is None:
            first = got
            continue
        for k in first:
            same = first[k].view(np.uint8).reshape(n + 1, -1) == got[k].view(np.uint8).reshape(n + 1, -1)
            rows = np.flatnonzero(~same.all(axis=1))
            assert rows.size == 0, f"repeat {rep}: {k} differs in rows {rows[:8]}"


def test_golden_export_full_vocab_sampled():
    """Eight f32 rows of the 512-row logits workload at V = 248,320; three
    seeded rows against the oracle."""
    need_gpu()
    n, v = 8, synth.VOCAB
    a, _ = synth.logit_rows(synth.LOGITS_F32, range(n), v)
    t = synth.targets(synth.LOGITS_F32, range(n), v)
    got = _run_export(a, False, t)
    rows = synth.subset(synth.LOGITS_F32, n, 3)
    want = oracle.golden_rows(a[rows].astype(np.float64), t[rows])
    _check_records({k: x[rows] for k, x in got.items()}, want, "V=248320")
    assert np.all(got["rec"][:, 2] > 0) and np.all(got["rec"][:, 2] < 1)


def _score_close(got, want, where):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want)), f"{where}: NaN pattern"
    assert np.array_equal(np.isposinf(got), np.isposinf(want)), f"{where}: +inf pattern"
    fin = np.isfinite(want)
    err = np.abs(got[fin] - want[fin])
    tol = 1e-6 + 1e-3 * np.abs(want[fin])
    assert np.all(err <= tol), f"{where}: score off by {err.max()} (want {want[fin][np.argmax(err)]})"


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("n,v", [(4, 512), (3, 5000), (2, 70001)])
def test_coarse_kl_shapes(n, v, bf16):
    need_gpu()
    print(f"coarse n={n} v={v} bf16={bf16}", flush=True)
    a, b = synth.logit_rows(synth.LOGITS_F32, range(n), v)
    if bf16:
        a, b = synth.f32_to_bf16_bits(a), synth.f32_to_bf16_bits(b)
    rec = oracle.golden_rows(_decode(a, bf16))
    db = to_dev(b, bf16)
    got = kld.kld_coarse_kl(db, to_dev(rec["ids"]), to_dev(rec["lp"]), to_dev(rec["rec"]))
    torch.cuda.synchronize()
    want = oracle.coarse_kl_rows(rec["ids"], rec["lp"], rec["rec"], _decode(b, bf16))
    _score_close(got.cpu().numpy(), want, f"n={n} v={v}")


def test_coarse_kl_full_vocab_and_bound():
    """Eight rows at V = 248,320: three seeded rows against the oracle, and
    every row's score at most the full-vocabulary KL (coarsening)."""
    need_gpu()
    n, v = 8, synth.VOCAB
    a, b = synth.logit_rows(synth.LOGITS_F32, range(n), v)
    rows = synth.subset(synth.LOGITS_F32, n, 3)
    rec = oracle.golden_rows(a[rows].astype(np.float64))
    got = kld.kld_coarse_kl(to_dev(b[rows]), to_dev(rec["ids"]), to_dev(rec["lp"]), to_dev(rec["rec"]))
    full = kld.kld_from_logits(to_dev(a[rows]), to_dev(b[rows]))
    torch.cuda.synchronize()
    want = oracle.coarse_kl_rows(rec["ids"], rec["lp"], rec["rec"], b[rows].astype(np.float64))
    _score_close(got.cpu().numpy(), want, "V=248320")
    assert np.all(got.cpu().numpy() <= full["kl"].cpu().numpy() * (1 + 1e-3) + 1e-6)


def test_coarse_kl_edges():
    need_gpu()
    v = 2048
    g = np.random.default_rng(11)
    a = g.normal(0, 2, (4, v)).astype(np.float32)
    rec = oracle.golden_rows(a.astype(np.float64))
    b = a.copy()
    b[1, rec["ids"][1][5]] = -np.inf          # a listed id the candidate rules out -> +inf
    b[2, 17] = np.nan                          # NaN candidate logit -> NaN
    ids = rec["ids"].copy()
    ids[3, 0] = v + 3                          # a listed id outside the vocabulary -> NaN
    got = kld.kld_coarse_kl(to_dev(b), to_dev(ids), to_dev(rec["lp"]), to_dev(rec["rec"]))
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    want0 = oracle.coarse_kl_row(rec["ids"][0], rec["lp"][0], float(rec["rec"][0][2]), b[0].astype(np.float64))
    assert abs(got[0] - want0) <= 1e-6      # the candidate is the reference: only rounding of lp
    assert got[1] == np.inf and np.isnan(got[2]) and np.isnan(got[3])


def test_golden_workload_launch_sampled():
    """The golden workload as timed: records of all 512 f32 reference rows at
    V = 248,320 in one call, then the 513-cell score of all 512 candidate
    rows in one call.  Six seeded rows are checked: their records against the
    oracle's, and their scores computed from the oracle's records (written
    over the GPU's on those rows) against the oracle's scores."""
    need_gpu()
    n, v = 512, synth.VOCAB
    a, b = synth.logit_rows(synth.LOGITS_F32, range(n), v)
    t = synth.targets(synth.LOGITS_F32, range(n), v)
    got = _run_export(a, False, t)
    rows = synth.subset(synth.LOGITS_F32, n, 6)
    want = oracle.golden_rows(a[rows].astype(np.float64), t[rows])
    _check_records({k: x[rows] for k, x in got.items()}, want, "512 rows")
    ids, lp, rec = got["ids"].copy(), got["lp"].copy(), got["rec"].copy()
    ids[rows], lp[rows], rec[rows] = want["ids"], want["lp"], want["rec"]
    score = kld.kld_coarse_kl(to_dev(b), to_dev(ids), to_dev(lp), to_dev(rec))
    torch.cuda.synchronize()
    score = score.cpu().numpy()
    ws = oracle.coarse_kl_rows(want["ids"], want["lp"], want["rec"], b[rows].astype(np.float64))
    _score_close(score[rows], ws, "512 rows")
    assert np.all(np.isfinite(score)) and np.all(score > 0)
