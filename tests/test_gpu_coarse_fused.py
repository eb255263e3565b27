"""GPU parity of kld_coarse_fused -- a candidate given as hidden states,
through the shared bf16 head, scored against golden records -- with the
oracle: head logits in f64 from the bf16 operands, the reference's golden
records and the candidate's 513-cell score.  The records fed to the GPU are
the oracle's (or seeded stand-ins on rows the test does not check), so no GPU
output feeds the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
import full_vocab_kl_amd as kld
from gpu_util import gpu, need_gpu, to_dev

pytestmark = gpu


def _score_close(got, want, where):
    # per-position bar of the scores: 1e-6 + 1e-3 * KL
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want)), f"{where}: NaN pattern"
    fin = np.isfinite(want)
    err = np.abs(got[fin] - want[fin])
    tol = 1e-6 + 1e-3 * np.abs(want[fin])
    assert np.all(err <= tol), f"{where}: score off by {err.max()} (want {want[fin][np.argmax(err)]})"


def _run(w, hc, ids, lp, rec):
    got = kld.kld_coarse_fused(to_dev(w, True), to_dev(hc, True), to_dev(ids), to_dev(lp),
                               to_dev(rec))
    torch.cuda.synchronize()
    return got.cpu().numpy()


def _case(n, v, d, noise, wl=synth.FUSED_WINDOW):
    w = synth.head_weight(wl, v, d)
    hr, hc = synth.hidden_rows(wl, range(n), d, noise)
    za, zb = oracle.head_logits(w, hr), oracle.head_logits(w, hc)
    rec = oracle.golden_rows(za)
    return w, hc, rec, zb


@pytest.mark.parametrize("n,v,d", [(3, 512, 64), (300, 1000, 128), (37, 5003, 200), (257, 2048, 8),
                                   (1, 4097, 520)])
def test_coarse_fused_shapes(n, v, d):
    """Several vocabulary tiles with a ragged last one, one and two
    256-position tiles with ragged tails, d not a multiple of the 64-wide
    stage."""
    need_gpu()
    print(f"coarse_fused n={n} v={v} d={d}", flush=True)
    w, hc, rec, zb = _case(n, v, d, 0.02)
    got = _run(w, hc, rec["ids"], rec["lp"], rec["rec"])
    want = oracle.coarse_kl_rows(rec["ids"], rec["lp"], rec["rec"], zb)
    _score_close(got, want, f"n={n} v={v} d={d}")


def test_coarse_fused_matches_logits_path():
    """The same candidate scored through the head and from its f32 logits
    (kld_coarse_kl on the oracle's logits rounded to f32) agree."""
    need_gpu()
    n, v, d = 64, 3000, 256
    w, hc, rec, zb = _case(n, v, d, 0.05)
    got = _run(w, hc, rec["ids"], rec["lp"], rec["rec"])
    via_logits = kld.kld_coarse_kl(to_dev(zb.astype(np.float32)), to_dev(rec["ids"]),
                                   to_dev(rec["lp"]), to_dev(rec["rec"]))
    torch.cuda.synchronize()
    _score_close(got, via_logits.cpu().numpy().astype(np.float64), "head vs logits")


def test_coarse_fused_candidate_is_reference():
    """Candidate hidden states equal to the reference's: the score is the
    rounding of the stored f32 log-probs only (near zero)."""
    need_gpu()
    n, v, d = 40, 2048, 64
    w = synth.head_weight(synth.FUSED_WINDOW, v, d)
    hr, _ = synth.hidden_rows(synth.FUSED_WINDOW, range(n), d, 0.0)
    rec = oracle.golden_rows(oracle.head_logits(w, hr))
    got = _run(w, hr, rec["ids"], rec["lp"], rec["rec"])
    assert np.all(np.abs(got) <= 1e-6), got.max()


def test_coarse_fused_repeated_and_bad_ids():
    need_gpu()
    n, v, d = 6, 2000, 64
    w, hc, rec, zb = _case(n, v, d, 0.02)
    ids = rec["ids"].copy()
    ids[1, 7] = ids[1, 3]          # a repeated id counts in both of its cells (as in the oracle)
    ids[2, 100] = ids[2, 0]
    ids[3, 0] = v + 5               # outside the vocabulary -> NaN
    ids[4, 9] = -1                  # negative -> NaN
    got = _run(w, hc, ids, rec["lp"], rec["rec"])
    want = oracle.coarse_kl_rows(np.where(ids < 0, 0, np.minimum(ids, v - 1)), rec["lp"], rec["rec"], zb)
    want[3] = want[4] = np.nan
    _score_close(got, want, "repeated / bad ids")


def test_coarse_fused_full_window_sampled():
    """One 2047-position window at d = 5120, V = 248,320 (the launch the bench
    times): 32 seeded positions carry the oracle's records and are checked;
    the other positions carry seeded stand-in records."""
    need_gpu()
    n, v, d = synth.WINDOW_POSITIONS, synth.VOCAB, synth.HIDDEN
    w = synth.head_weight(synth.FUSED_WINDOW, v, d)
    hr, hc = synth.hidden_rows(synth.FUSED_WINDOW, range(n), d, 0.01)
    ids, lp, rec = synth.sparse_records(synth.FUSED_WINDOW, n, v)
    rows = synth.subset(synth.FUSED_WINDOW, n, 32)
    za = oracle.head_logits(w, hr[rows])
    zb = oracle.head_logits(w, hc[rows])
    g = oracle.golden_rows(za)
    ids[rows], lp[rows], rec[rows] = g["ids"], g["lp"], g["rec"]
    got = _run(w, hc, ids, lp, rec)
    want = oracle.coarse_kl_rows(g["ids"], g["lp"], g["rec"], zb)
    _score_close(got[rows], want, "full window")
    assert abs(got[rows].mean() - want.mean()) <= 1e-4 * want.mean()
    assert np.all(np.isfinite(got)) and np.all(got >= -1e-6)
