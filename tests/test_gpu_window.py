"""GPU parity of the scored-window statistics (kld_window_summary) against
the oracle: per-segment sums and counts past score_from, the mean over every
scored position and exact exceedance counts, on seeded per-position scores
laid out as fixed windows, as documents of mixed length and as one long
trace.  Counts are compared exactly; sums of f32 values in f64 differ from the
oracle's only by summation order (relative 1e-12 here)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import full_vocab_kl_amd as kld
from gpu_util import gpu, need_gpu, to_dev

pytestmark = gpu
THR = (0.0, 0.01, 0.1, 0.5, 1.0, 2.0, 5.0)   # f32-representable, compared in f32 on both sides


def _run(x, offsets, score_from, thr=THR):
    need_gpu()
    got = kld.kld_window_summary(to_dev(x), to_dev(offsets), score_from, thr)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in got.items()}


def _check(x, offsets, score_from, thr=THR, where=""):
    got = _run(x, offsets, score_from, thr)
    want = oracle.window_summary(x, offsets, score_from, thr)
    assert np.array_equal(got["seg_count"], want["seg_count"]), f"{where}: counts"
    assert np.array_equal(got["seg_exceed"], want["seg_exceed"]), f"{where}: segment exceedances"
    err = np.abs(got["seg_sum"] - want["seg_sum"])
    assert np.all(err <= 1e-12 * np.maximum(np.abs(want["seg_sum"]), 1e-300)), f"{where}: sums"
    t = got["totals"]
    assert int(t[1]) == want["count"], f"{where}: total count"
    if want["count"]:
        assert abs(t[0] - want["mean"]) <= 1e-12 * abs(want["mean"]), f"{where}: mean"
    else:
        assert np.isnan(t[0]), f"{where}: empty mean"
    assert np.array_equal(t[2:].astype(np.int64), want["exceed"]), f"{where}: exceedances"
    return got, want


@pytest.mark.parametrize("score_from", [0, 256, 1024])
def test_fixed_windows(score_from):
    # 64 windows of 2047 scored positions, the window control of the pages
    n = 64 * 2047
    x = synth.kl_scores(301, n)
    offsets = np.arange(0, n + 1, 2047, dtype=np.int64)
    _check(x, offsets, score_from, where=f"windows sf={score_from}")


def test_mixed_documents_and_subset_mean():
    # documents from empty to 70,000 positions, several shorter than score_from
    lengths = [0, 1, 255, 256, 257, 1000, 2047, 4096, 70_000, 12_345, 3, 999, 50_000]
    offsets = synth.doc_offsets(302, lengths)
    x = synth.kl_scores(302, int(offsets[-1]))
    got, want = _check(x, offsets, 256, where="documents")
    # the mean over a subset of documents (the long ones) from the per-segment sums
    sel = want["seg_count"] > 10_000
    sub_g = got["seg_sum"][sel].sum() / got["seg_count"][sel].sum()
    sub_w = want["seg_sum"][sel].sum() / want["seg_count"][sel].sum()
    assert abs(sub_g - sub_w) <= 1e-12 * sub_w


def test_long_trace():
    # one 262,144-position trace (a 256K-token document), score_from 1024
    n = 262_144
    x = synth.kl_scores(303, n)
    _check(x, np.array([0, n], np.int64), 1024, where="long trace")


def test_gaps_and_reproducible():
    # segments need not tile the array: positions outside every segment are ignored
    n = 100_000
    x = synth.kl_scores(304, n)
    offsets = np.array([10, 5000, 5000, 40_000, 99_999], np.int64)
    a, _ = _check(x, offsets, 100, where="gaps")
    b = _run(x, offsets, 100)
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), f"{k} not reproducible"


def test_degenerate():
    x = synth.kl_scores(305, 1000)
    # no thresholds; every segment shorter than score_from -> empty mean
    _check(x, np.array([0, 100, 1000], np.int64), 2000, thr=(), where="all unscored")
    # no segments at all
    got = _run(x, np.array([0], np.int64), 0)
    assert got["seg_sum"].shape == (0,) and np.isnan(got["totals"][0]) and got["totals"][1] == 0
    assert np.all(got["totals"][2:] == 0)
    # empty score array
    got = _run(np.zeros(0, np.float32), np.array([0, 0], np.int64), 0)
    assert got["seg_count"][0] == 0 and np.isnan(got["totals"][0])
    # sixteen thresholds, the most the entry point takes
    thr = tuple(float(np.float32(v)) for v in np.geomspace(1e-4, 10.0, 16))
    _check(synth.kl_scores(306, 50_000), np.array([0, 20_000, 50_000], np.int64), 0, thr=thr,
           where="16 thresholds")


def test_bad_offsets_give_nan():
    x = synth.kl_scores(307, 1000)
    got = _run(x, np.array([0, 500, 400, 1000], np.int64), 0)   # decreasing pair
    assert np.isnan(got["seg_sum"][1]) and got["seg_count"][1] == 0
    assert got["seg_count"][0] == 500 and got["seg_count"][2] == 600
    assert np.isnan(got["totals"][0])
    got = _run(x, np.array([0, 1001], np.int64), 0)             # past the end
    assert np.isnan(got["seg_sum"][0]) and np.isnan(got["totals"][0])


def test_ten_shard_launch():
    """The aggregation workload as timed: 10,480,640 positions in 5,120
    contexts of 2,047, seven thresholds, every segment against the oracle."""
    n = 5120 * 2047
    x, _ = synth.kl_score_pair(synth.LOGITS_F32, n)
    offsets = np.arange(0, n + 1, 2047, dtype=np.int64)
    _check(x, offsets, 0, where="ten-shard layout")


def test_many_short_documents():
    """Enough short documents (at least 1,024, averaging at most 16 Ki
    positions) for the one-wave-per-segment launch: ragged lengths from 0 to
    9,000 positions, some shorter than score_from, sixteen thresholds."""
    lengths = [int(v) for v in np.random.default_rng(308).integers(0, 9000, 1500)]
    lengths[:4] = [0, 1, 256, 2048]
    offsets = synth.doc_offsets(308, lengths)
    x = synth.kl_scores(308, int(offsets[-1]))
    thr = tuple(float(np.float32(v)) for v in np.geomspace(1e-4, 10.0, 16))
    a, _ = _check(x, offsets, 256, thr=thr, where="short documents")
    b = _run(x, offsets, 256, thr)
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), f"{k} not reproducible"


def test_many_short_documents_bad_pair():
    """A decreasing offset pair in the one-wave launch: that segment's sum is
    NaN and its count 0, the mean is NaN, every other segment is unaffected."""
    x = synth.kl_scores(309, 1200 * 500)
    offsets = np.arange(0, 1200 * 500 + 1, 500, dtype=np.int64)
    offsets[7] = offsets[6] - 1                                  # segment 6 decreasing
    got = _run(x, offsets, 0)
    assert np.isnan(got["seg_sum"][6]) and got["seg_count"][6] == 0
    assert np.isnan(got["totals"][0])
    want = oracle.window_summary(x, offsets, 0, THR)            # segment 6 empty there
    ok = np.arange(1200) != 6
    assert np.array_equal(got["seg_count"][ok], want["seg_count"][ok])
    assert np.array_equal(got["seg_exceed"][ok], want["seg_exceed"][ok])
    err = np.abs(got["seg_sum"][ok] - want["seg_sum"][ok])
    assert np.all(err <= 1e-12 * want["seg_sum"][ok])
    assert got["seg_count"][7] == 1001


@pytest.mark.parametrize("nthr", [0, 1, 4, 5, 9, 16])
@pytest.mark.parametrize("layout", ["wave", "block"])
def test_threshold_counts(nthr, layout):
    """Every padded threshold-count class (none, up to 4, 8 and 16) in both
    launches: 1,100 segments of 300 positions (one wave each) and 10 segments
    of 3,000 (one block each), score_from 7, unsorted thresholds with a
    duplicate."""
    pool = [0.5, 0.01, 2.0, 0.1, 0.5, 5.0, 1.0, 0.0, 0.05, 3.0, 0.2, 8.0, 0.3, 0.02, 0.7, 1.5]
    thr = tuple(float(np.float32(v)) for v in pool[:nthr])
    nseg, per = (1100, 300) if layout == "wave" else (10, 3000)
    x = synth.kl_scores(310 + nthr, nseg * per)
    offsets = np.arange(0, nseg * per + 1, per, dtype=np.int64)
    _check(x, offsets, 7, thr=thr, where=f"{layout} nthr={nthr}")
