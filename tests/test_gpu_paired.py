"""GPU parity of the paired per-context comparison with a source-cluster
bootstrap (kld_paired_bootstrap) against the oracle: on integer-valued sums
every quantity is exact in f64, so the comparison is bitwise; on scores
summed per context by kld_window_summary (realistic values) sums differ from
the oracle's only by summation order (1e-12 of the largest per-context mean
difference here), and wins and ties agree except where two means are within
rounding of a tie."""
import numpy as np
import pytest
import torch

import oracle
import synth
import full_vocab_kl_amd as kld
from gpu_util import gpu, need_gpu, to_dev

pytestmark = gpu
Q = (0.025, 0.5, 0.975)


def _gpu(sum_a, sum_b, count, cluster, draws, q=Q):
    need_gpu()
    r = kld.kld_paired_bootstrap(to_dev(np.asarray(sum_a, np.float64)),
                                 to_dev(np.asarray(sum_b, np.float64)),
                                 to_dev(np.asarray(count, np.int64)),
                                 to_dev(np.asarray(cluster, np.int32)),
                                 to_dev(np.asarray(draws, np.int32)), q)
    torch.cuda.synchronize()
    return r["out"].cpu().numpy(), r["replicates"].cpu().numpy()


def _integer_inputs(w, nctx, nclust, nrep):
    g = synth.rng(w, synth.STREAM_SCORES, 10)
    count = g.integers(1, 3000, nctx)
    sum_a = g.integers(0, 10 ** 6, nctx).astype(np.float64)
    sum_b = sum_a + g.integers(-5000, 5000, nctx)
    return (sum_a, sum_b, count, synth.cluster_labels(w, nctx, nclust),
            synth.bootstrap_draws(w, nrep, nclust))


@pytest.mark.parametrize("nctx,nclust,nrep", [(512, 330, 10_000), (7, 3, 27), (5120, 842, 16384),
                                              (1000, 1, 100), (300, 300, 1)])
def test_exact_on_integer_sums(nctx, nclust, nrep):
    sa, sb, cnt, lab, dr = _integer_inputs(401, nctx, nclust, nrep)
    out, reps = _gpu(sa, sb, cnt, lab, dr)
    want = oracle.paired_bootstrap(sa, sb, cnt, lab, dr, Q)
    assert np.array_equal(reps, want["replicates"])
    assert out[0] == want["diff"]
    assert (out[1], out[2], out[3]) == (want["a_wins"], want["b_wins"], want["ties"])
    assert np.array_equal(out[4:], np.array(want["quantiles"]))


def test_chain_from_window_sums():
    # ten-shard-like layout at a tenth of the size: 512 contexts of 2047
    # scored positions in 330 clusters, scored from position 256
    need_gpu()
    nctx, nclust, nrep = 512, 330, 10_000
    a, b = synth.kl_score_pair(402, nctx * 2048)
    offsets = np.arange(0, nctx * 2048 + 1, 2048, dtype=np.int64)
    wa = kld.kld_window_summary(to_dev(a), to_dev(offsets), 256)
    wb = kld.kld_window_summary(to_dev(b), to_dev(offsets), 256)
    lab = synth.cluster_labels(402, nctx, nclust)
    dr = synth.bootstrap_draws(402, nrep, nclust)
    r = kld.kld_paired_bootstrap(wa["seg_sum"], wb["seg_sum"], wa["seg_count"], to_dev(lab),
                                 to_dev(dr), Q)
    torch.cuda.synchronize()
    out, reps = r["out"].cpu().numpy(), r["replicates"].cpu().numpy()
    # the oracle from the raw scores
    oa = oracle.window_summary(a, offsets, 256)
    ob = oracle.window_summary(b, offsets, 256)
    want = oracle.paired_bootstrap(oa["seg_sum"], ob["seg_sum"], oa["seg_count"], lab, dr, Q)
    m = np.max(np.abs(oa["seg_sum"] - ob["seg_sum"]) / oa["seg_count"])
    tol = 1e-12 * m
    assert abs(out[0] - want["diff"]) <= tol
    assert np.max(np.abs(reps - want["replicates"])) <= tol
    assert np.max(np.abs(out[4:] - np.array(want["quantiles"]))) <= tol
    # wins and ties: equal to the oracle's wherever the two means are not
    # within rounding of a tie
    close = np.abs(oa["seg_sum"] - ob["seg_sum"]) <= 1e-12 * np.abs(oa["seg_sum"])
    assert abs(out[1] - want["a_wins"]) <= close.sum()
    assert want["quantiles"][0] < want["diff"] < want["quantiles"][2]


def test_edges():
    # identical candidates: zero difference, every context tied, zero interval
    s = np.arange(10, dtype=np.float64)
    cnt = np.full(10, 4)
    lab = np.arange(10) % 3
    dr = synth.bootstrap_draws(403, 50, 3)
    out, reps = _gpu(s, s, cnt, lab, dr)
    assert out[0] == 0.0 and out[3] == 10 and out[1] == 0 and out[2] == 0
    assert np.all(reps == 0.0) and np.all(out[4:] == 0.0)
    # contexts without scored positions count in neither wins nor ties
    cnt0 = cnt.copy()
    cnt0[:4] = 0
    s1, s0 = s + 1, s.copy()
    s1[:4] = s0[:4] = 0.0
    out, _ = _gpu(s1, s0, cnt0, lab, dr)
    want = oracle.paired_bootstrap(s1, s0, cnt0, lab, dr, Q)
    assert (out[1], out[2], out[3]) == (want["a_wins"], want["b_wins"], want["ties"]) == (0, 6, 0)
    # no replicates: NaN percentiles, the difference still reported
    out, reps = _gpu(s + 1, s, cnt, lab, np.zeros((0, 3), np.int32))
    assert reps.shape == (0,) and np.all(np.isnan(out[4:])) and out[0] == 10 / 40
    # a cluster drawn only where it holds no positions: NaN replicate, NaN percentiles
    out, reps = _gpu(s1, s0, cnt0, np.array([1] * 4 + [0] * 6, np.int32),
                     np.array([[1, 1], [0, 1]], np.int32))
    assert np.isnan(reps[0]) and reps[1] == 6 / 24 and np.all(np.isnan(out[4:]))


def test_bad_labels_and_draws_give_nan():
    s = np.arange(6, dtype=np.float64)
    cnt = np.full(6, 2)
    # a label outside [0, nclust): the cluster sums are invalid, so the
    # difference, every replicate and every percentile are NaN
    out, reps = _gpu(s, s + 1, cnt, [0, 1, 2, 0, 1, 5], np.array([[0, 1, 2], [2, 2, 2]], np.int32))
    assert np.isnan(out[0]) and np.all(np.isnan(reps)) and np.all(np.isnan(out[4:]))
    # a negative count: the same
    out, reps = _gpu(s, s + 1, [2, 2, -1, 2, 2, 2], [0, 1, 2, 0, 1, 2],
                     np.array([[0, 1, 2], [1, 1, 0]], np.int32))
    assert np.isnan(out[0]) and np.all(np.isnan(reps)) and np.all(np.isnan(out[4:]))
    # valid inputs after invalid ones: finite again (every call rewrites the check)
    out, reps = _gpu(s, s + 1, cnt, [0, 1, 2, 0, 1, 2], np.array([[0, 1, 2]], np.int32))
    assert out[0] == -0.5 and reps[0] == -0.5 and np.all(np.isfinite(out[4:]))
    out, reps = _gpu(s, s + 1, cnt, [0, 1, 2, 0, 1, 2], np.array([[0, 1, 3], [0, 1, 2]], np.int32))
    assert np.isnan(reps[0]) and reps[1] == -0.5 and np.all(np.isnan(out[4:]))


def test_ten_shard_launch():
    """The bootstrap as timed: 5,120 contexts' window sums of two candidates
    (10,480,640 positions), 842 clusters, 10,000 replicates."""
    need_gpu()
    nctx, nclust, nrep, per = 5120, 842, 10_000, 2047
    a, b = synth.kl_score_pair(synth.LOGITS_F32, nctx * per)
    offsets = np.arange(0, nctx * per + 1, per, dtype=np.int64)
    wa = kld.kld_window_summary(to_dev(a), to_dev(offsets), 0)
    wb = kld.kld_window_summary(to_dev(b), to_dev(offsets), 0)
    lab = synth.cluster_labels(synth.LOGITS_F32, nctx, nclust)
    dr = synth.bootstrap_draws(synth.LOGITS_F32, nrep, nclust)
    r = kld.kld_paired_bootstrap(wa["seg_sum"], wb["seg_sum"], wa["seg_count"], to_dev(lab),
                                 to_dev(dr), Q)
    torch.cuda.synchronize()
    out, reps = r["out"].cpu().numpy(), r["replicates"].cpu().numpy()
    # the oracle from the raw scores: its own window sums, then the bootstrap
    oa = oracle.window_summary(a, offsets, 0)
    ob = oracle.window_summary(b, offsets, 0)
    want = oracle.paired_bootstrap(oa["seg_sum"], ob["seg_sum"], oa["seg_count"], lab, dr, Q)
    m = np.max(np.abs(oa["seg_sum"] - ob["seg_sum"]) / oa["seg_count"])
    assert abs(out[0] - want["diff"]) <= 1e-12 * m
    assert np.max(np.abs(reps - want["replicates"])) <= 1e-12 * m
    assert np.max(np.abs(out[4:] - np.array(want["quantiles"]))) <= 1e-12 * m
    # wins and ties: equal wherever the two means are not within rounding of a tie
    close = np.abs(oa["seg_sum"] - ob["seg_sum"]) <= 1e-12 * np.abs(oa["seg_sum"])
    assert abs(out[1] - want["a_wins"]) <= close.sum() and abs(out[2] - want["b_wins"]) <= close.sum()
