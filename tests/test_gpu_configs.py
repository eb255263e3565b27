"""GPU parity on the full-size workloads beyond the single window: the
16-window fused batch (32,752 positions in one call), the 262,144-position
long trace (32 chunks of 8192 rows with top-64 export, candidate noise rising
from 0.005 to 0.05), and every 4096-row batch of the 32,752-row bf16 top-64
stream.  Seeded positions are checked against the f64 oracle one by one and
their mean KL to 1e-4 relative; every position is checked for the
properties that hold at any size; the device summary's quantiles must equal
a host sort of the device's own per-position values."""
import numpy as np
import pytest
import torch

import oracle
import synth
import full_vocab_kl_amd as kld
from gpu_util import (gpu, need_gpu, to_dev, assert_kl_close, assert_mean_rel, assert_nll_close,
                      oracle_rows, top_gaps, host_quantiles)
from test_gpu_fused_topk import check_topk, check_tail
from test_gpu_topk import assert_lp_close

pytestmark = gpu

GAP = 1e-3         # fused-path argmax exemption (oracle top-2 gap below this)
STRICT_GAP = 1e-4  # argmaxes with a wider gap must match (f32 accumulation error ~1e-6)
V, D, NW = synth.VOCAB, synth.HIDDEN, synth.WINDOW_POSITIONS
QUANTILES = (0.5, 0.99, 0.999)
STREAM_ROWS, BATCH = 16 * NW, 4096


def _fused_oracle(w, hr, hc, t, k=None):
    """Oracle scores of sampled positions: both sides' logits through the head
    in one f64 product, then the per-row definitions; plus the top-2 gaps."""
    m = hr.shape[0]
    z = oracle.head_logits(w, np.concatenate([hr, hc]))
    za, zb = z[:m], z[m:]
    res = oracle_rows(za, zb, t, k=k)
    res["gap_ref"] = top_gaps(za, (1,))[1]
    res["gap_cand"] = top_gaps(zb, (1,))[1]
    return res, {"ref": za, "cand": zb}


def _compare(got, want, where):
    assert_kl_close(got["kl"], want["kl"], where)
    assert_mean_rel(got["kl"], want["kl"], where=where)
    for s in ("ref", "cand"):
        ok = want[f"gap_{s}"] >= STRICT_GAP
        assert np.array_equal(got[f"argmax_{s}"][ok], want[f"argmax_{s}"][ok]), f"{where}: argmax {s}"
        if "nll_ref" in got:
            assert_nll_close(got[f"nll_{s}"], want[f"nll_{s}"], where)
    return {s: int(np.sum(want[f"gap_{s}"] < GAP)) for s in ("ref", "cand")}


def _properties(kl, where):
    assert np.all(np.isfinite(kl)) and np.all(kl >= 0) and not np.any(np.signbit(kl)), where


def _check_summary(summ, kl, top1, nll_r, nll_c, where):
    """The device summary against the per-position values it summarises: the
    mean, top-1 rate and mean NLLs are their sums (f64, any order: 1e-12), and
    each quantile equals the type-7 interpolation of a host sort of the same
    f32 values, computed with the same f64 operations (exact)."""
    n = len(kl)
    k = np.asarray(kl, np.float64)
    assert summ[0] == pytest.approx(k.mean(), rel=1e-12), where
    assert summ[1] == pytest.approx(top1, abs=0.5 / n), where
    if nll_r is not None:
        assert summ[2] == pytest.approx(np.mean(np.asarray(nll_r, np.float64)), rel=1e-12), where
        assert summ[3] == pytest.approx(np.mean(np.asarray(nll_c, np.float64)), rel=1e-12), where
        assert summ[6] == pytest.approx(np.exp(summ[3]) / np.exp(summ[2]), rel=1e-12), where
    assert summ[7] == 0, where
    for i, hq in enumerate(host_quantiles(kl, QUANTILES)):
        assert summ[8 + i] == hq, f"{where}: quantile {QUANTILES[i]}: {summ[8 + i]!r} vs {hq!r}"


def test_fused_batch_sampled():
    """16 windows x 2047 = 32,752 positions (candidate noise 0.02) through one
    kld_fused_head call, then kld_summary; 16 seeded positions per window
    (256) against the oracle."""
    need_gpu()
    n = 16 * NW
    w = synth.head_weight(synth.FUSED_WINDOW, V, D)   # the fused workloads share one head
    hr, hc = synth.hidden_rows(synth.FUSED_BATCH, range(n), D, 0.02)
    t = synth.targets(synth.FUSED_BATCH, range(n), V)
    print(f"fused batch n={n}", flush=True)
    out = kld.kld_fused_head(to_dev(w, True), to_dev(hr, True), to_dev(hc, True), to_dev(t))
    summ = kld.kld_summary(out["kl"], out["argmax_ref"], out["argmax_cand"], out["nll_ref"],
                           out["nll_cand"], QUANTILES)
    torch.cuda.synchronize()
    got = {k: x.cpu().numpy() for k, x in out.items()}
    summ = summ.cpu().numpy()
    _properties(got["kl"], "batch")
    top1 = float(np.mean(got["argmax_ref"] == got["argmax_cand"]))
    _check_summary(summ, got["kl"], top1, got["nll_ref"], got["nll_cand"], "batch")
    rows = np.concatenate([wi * NW + synth.subset(synth.FUSED_BATCH * 1000 + wi, NW, 16)
                           for wi in range(16)])
    want, _ = _fused_oracle(w, hr[rows], hc[rows], t[rows])
    ex = _compare({k: x[rows] for k, x in got.items()}, want, "batch")
    print(f"argmax gap-exempt: {ex} of {len(rows)}", flush=True)


def test_long_trace_sampled():
    """262,144 positions in 32 chunks of 8192 rows: full KLD + top-1 + NLL and
    top-64 export per chunk, then kld_summary over all positions; 8 seeded
    positions per chunk (256) against the oracle (values and their mean,
    argmax, top-64 lists and log-probs, the tail KLD from the exports)."""
    need_gpu()
    chunk, nchunk, per = 8192, 32, 8
    w = synth.head_weight(synth.FUSED_WINDOW, V, D)
    W = to_dev(w, True)
    kl_dev = torch.empty(chunk * nchunk, dtype=torch.float32, device="cuda")
    am = {s: torch.empty(chunk * nchunk, dtype=torch.int32, device="cuda") for s in ("ref", "cand")}
    nll = {s: torch.empty(chunk * nchunk, dtype=torch.float32, device="cuda") for s in ("ref", "cand")}
    sub, hrs, hcs, ts = [], [], [], []
    for c in range(nchunk):
        r = range(c * chunk, (c + 1) * chunk)
        hr, hc = synth.hidden_rows(synth.LONG_TRACE, r, D, synth.long_trace_noise)
        t = synth.targets(synth.LONG_TRACE, r, V)
        print(f"long trace chunk {c} noise {synth.long_trace_noise(c * chunk):.4f}", flush=True)
        out = kld.kld_fused_head(W, to_dev(hr, True), to_dev(hc, True), to_dev(t), topk=True)
        sl = slice(c * chunk, (c + 1) * chunk)
        kl_dev[sl] = out["kl"]
        for s in ("ref", "cand"):
            am[s][sl] = out[f"argmax_{s}"]
            nll[s][sl] = out[f"nll_{s}"]
        torch.cuda.synchronize()
        rows = synth.subset(synth.LONG_TRACE * 1000 + c, chunk, per)
        sub.append({k: x[torch.from_numpy(rows).cuda()].cpu().numpy() for k, x in out.items()})
        hrs.append(hr[rows]); hcs.append(hc[rows]); ts.append(t[rows])
    summ = kld.kld_summary(kl_dev, am["ref"], am["cand"], nll["ref"], nll["cand"], QUANTILES)
    tail = kld.kld_topk_tail(*(torch.from_numpy(np.ascontiguousarray(
        np.concatenate([x[k] for x in sub]))).cuda() for k in ("ids_ref", "lp_ref", "ids_cand",
                                                               "lp_cand")), V)
    torch.cuda.synchronize()
    kl_all = kl_dev.cpu().numpy()
    _properties(kl_all, "long trace")
    top1 = float(np.mean(am["ref"].cpu().numpy() == am["cand"].cpu().numpy()))
    _check_summary(summ.cpu().numpy(), kl_all, top1, nll["ref"].cpu().numpy(),
                   nll["cand"].cpu().numpy(), "long trace")
    got = {k: np.concatenate([x[k] for x in sub]) for k in sub[0]}
    want, z = _fused_oracle(w, np.concatenate(hrs), np.concatenate(hcs), np.concatenate(ts), k=64)
    ex = _compare(got, want, "long trace")
    c = check_topk(got, z, want, "long trace")
    same = check_tail(tail.cpu().numpy(), got, want, V, "long trace")
    print(f"argmax gap-exempt: {ex}; top-64 sets: {c}; tail compared on {same} of "
          f"{len(got['kl'])} rows", flush=True)
    # noise rises along the trace: the last chunk scores far above the first
    assert kl_all[-chunk:].mean() > 10 * kl_all[:chunk].mean()


@pytest.mark.parametrize("batch", range((STREAM_ROWS + BATCH - 1) // BATCH))
def test_topk_bf16_stream_batch(batch):
    """Batch `batch` of the bf16 top-64 workload (16 windows = 32,752 rows in
    4096-row batches; the last holds 4080 rows): full KLD with both sides'
    top-64 in one pass, then the tail KLD from the exported lists; 32 seeded
    rows against the oracle (KL and their mean, ids bit-exact, fp16
    log-probs, tail KLD on identical lists)."""
    need_gpu()
    r0 = batch * BATCH
    n = min(BATCH, STREAM_ROWS - r0)
    a, b = synth.logit_rows(synth.LOGITS_BF16_TOPK, range(r0, r0 + n), V, dtype="bf16")
    print(f"bf16 top-64 batch {batch}: rows {r0}..{r0 + n - 1}", flush=True)
    out = kld.kld_from_logits(to_dev(a, True), to_dev(b, True), None, topk=True)
    tail = kld.kld_topk_tail(out["ids_ref"], out["lp_ref"], out["ids_cand"], out["lp_cand"], V)
    torch.cuda.synchronize()
    got = {k: x.cpu().numpy() for k, x in out.items()}
    tail = tail.cpu().numpy()
    _properties(got["kl"], f"bf16 batch {batch}")
    assert np.all(np.isfinite(tail)) and np.all(tail >= 0)
    sel = synth.subset(synth.LOGITS_BF16_TOPK * 1000 + batch, n, 32)
    want = oracle_rows(oracle.bf16_bits_to_f64(a[sel]), oracle.bf16_bits_to_f64(b[sel]), None, k=64)
    sub = {k: x[sel] for k, x in got.items()}
    assert_kl_close(sub["kl"], want["kl"], f"bf16 batch {batch}")
    assert_mean_rel(sub["kl"], want["kl"], where=f"bf16 batch {batch}")
    for s in ("ref", "cand"):
        assert np.array_equal(sub[f"argmax_{s}"], want[f"argmax_{s}"]), s
        assert np.array_equal(sub[f"ids_{s}"], want[f"ids_{s}"]), f"batch {batch} ids {s}"
        assert_lp_close(sub[f"lp_{s}"].view(np.uint16), want[f"lp_{s}"], f"batch {batch} {s}")
    same = check_tail(tail[sel], sub, want, V, f"bf16 batch {batch}")
    print(f"tail compared on {same} of {len(sel)} rows; mean full KL {got['kl'].mean():.4e}, "
          f"mean tail KL {tail.mean():.4e}", flush=True)
