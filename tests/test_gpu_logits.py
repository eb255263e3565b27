"""GPU parity of kld_from_logits against the f64 oracle (through the C ABI)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
import full_vocab_kl_amd as kld
from gpu_util import (gpu, need_gpu, to_dev, assert_kl_close, assert_mean_rel, assert_nll_close,
                      oracle_rows, host_quantiles)

pytestmark = gpu


def _run(a, b, t, bf16, ld_pad=0):
    """a, b: f32 arrays (or bf16 bit arrays when bf16); returns GPU results as numpy."""
    n, v = a.shape
    if ld_pad:
        pa = np.zeros((n, v + ld_pad), a.dtype); pa[:, :v] = a
        pb = np.zeros((n, v + ld_pad), b.dtype); pb[:, :v] = b
        da, db = to_dev(pa, bf16)[:, :v], to_dev(pb, bf16)[:, :v]
    else:
        da, db = to_dev(a, bf16), to_dev(b, bf16)
    dt = to_dev(t) if t is not None else None
    out = kld.kld_from_logits(da, db, dt)
    torch.cuda.synchronize()
    return {k: x.cpu().numpy() for k, x in out.items()}


def _oracle(a, b, t, bf16):
    if bf16:
        a, b = oracle.bf16_bits_to_f64(a), oracle.bf16_bits_to_f64(b)
    return oracle.score_rows(a, b, t)


def _compare(got, want, where, strict_mean=False):
    """strict_mean: the workload-level bar, mean KL within 1e-4 relative.
    Otherwise (tiny synthetic shapes, where KL can sit near the f32
    quantisation floor of the dominant weight) the mean must stay within the
    mean of the per-position bounds."""
    assert_kl_close(got["kl"], want["kl"], where)
    fin = np.isfinite(want["kl"])
    if fin.any():
        if strict_mean:
            assert_mean_rel(got["kl"][fin], want["kl"][fin], where=where)
        else:
            g = np.asarray(got["kl"][fin], np.float64); w = want["kl"][fin]
            assert abs(g.mean() - w.mean()) <= np.mean(1e-6 + 1e-3 * w), where
    assert np.array_equal(got["argmax_ref"], want["argmax_ref"]), where
    assert np.array_equal(got["argmax_cand"], want["argmax_cand"]), where
    for s in ("ref", "cand"):
        w = want[f"lse_{s}"]
        ok = np.isfinite(w)
        assert np.all(np.abs(got[f"lse_{s}"][ok] - w[ok]) <= 1e-5 * np.maximum(1, np.abs(w[ok]))), where
        if "nll_ref" in got:
            assert_nll_close(got[f"nll_{s}"], want[f"nll_{s}"], where)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("n,v,pad", [(3, 2, 0), (5, 16, 0), (7, 65, 0), (4, 1000, 0), (3, 5003, 1),
                                     (6, 4096 * 3 + 8, 0), (2, 70001, 0), (9, 33000, 8)])
def test_logits_small_shapes(n, v, pad, bf16):
    need_gpu()
    a, b = synth.logit_rows(synth.LOGITS_F32, range(n), v)
    if bf16:
        a, b = synth.f32_to_bf16_bits(a), synth.f32_to_bf16_bits(b)
    t = synth.targets(synth.LOGITS_F32, range(n), v)
    print(f"case n={n} v={v} pad={pad} bf16={bf16}", flush=True)
    got = _run(a, b, t, bf16, pad)
    _compare(got, _oracle(a, b, t, bf16), f"n={n} v={v} bf16={bf16}")


def test_logits_identical_rows_give_exact_zero():
    need_gpu()
    a, _ = synth.logit_rows(synth.LOGITS_F32, range(4), 20000)
    got = _run(a, a.copy(), None, False)
    assert np.all(got["kl"] == 0.0) and not np.any(np.signbit(got["kl"]))


def test_logits_edge_values():
    need_gpu()
    inf, nan = math.inf, math.nan
    v = 300
    g = np.random.default_rng(1)
    base = g.normal(0, 3, (9, v)).astype(np.float32)
    a = base.copy(); b = base + g.normal(0, 0.1, (9, v)).astype(np.float32)
    a[0, 5] = -inf                        # reference -inf id: contributes nothing
    a[1, 7] = -inf; b[1, 7] = -inf        # both -inf
    b[2, 11] = -inf                       # finite p against q = 0: +inf
    a[3, :] = -inf                        # empty reference row: NaN
    a[4, 3] = nan                         # NaN: NaN
    b[5, 2] = inf                         # +inf: NaN
    a[6] += 1000.0; b[6] -= 1000.0        # large shifts
    a[7, :] = 2.5; b[7, :] = 2.5          # all ties: argmax 0, KL 0
    a[8, 10] = a[8, 20] = 50.0            # tie at the max: lowest id
    b[2, 100] = -inf; a[2, 100] = -200.0  # weight underflows f32 but q = 0 still gives +inf
    t = np.array([0, 7, 11, 3, 2, 1, 299, 0, 20], np.int32)
    got = _run(a, b, t, False)
    want = _oracle(a, b, t, False)
    assert_kl_close(got["kl"], want["kl"], "edges")
    assert got["kl"][2] == inf and math.isnan(got["kl"][3]) and math.isnan(got["kl"][4])
    assert math.isnan(got["kl"][5]) and got["kl"][7] == 0.0
    for r in (0, 1, 2, 6, 7, 8):
        assert got["argmax_ref"][r] == want["argmax_ref"][r]
        assert got["argmax_cand"][r] == want["argmax_cand"][r]
    assert got["argmax_ref"][8] == 10


@pytest.mark.parametrize("bf16", [False, True])
def test_logits_shifted_rows(bf16):
    """Rows shifted by large opposite constants (|c| up to 300, a different
    one per row and side): KL is invariant under such shifts, and the kernel's
    exponents against rounded offsets must keep the per-position bar and the
    mean bar there (a form that sums w (a - b) without offsets misses the
    per-position bar by 50x on these rows)."""
    need_gpu()
    g = np.random.default_rng(5)
    n, v = 48, 20_000
    a = (3 * g.standard_normal((n, v))).astype(np.float32)
    b = (a + 0.03 * g.standard_normal((n, v))).astype(np.float32)
    ca = g.uniform(-300, 300, (n, 1)).astype(np.float32)
    cb = g.uniform(-300, 300, (n, 1)).astype(np.float32)
    a, b = (a + ca).astype(np.float32), (b + cb).astype(np.float32)
    if bf16:
        a, b = synth.f32_to_bf16_bits(a), synth.f32_to_bf16_bits(b)
    got = _run(a, b, None, bf16)
    want = _oracle(a, b, None, bf16)
    _compare(got, want, f"shifted bf16={bf16}", strict_mean=True)


@pytest.mark.parametrize("topk", [False, True])
@pytest.mark.parametrize("bf16", [False, True])
def test_argmax_ties_across_lanes_rounds_and_splits(bf16, topk):
    """Equal maxima planted at ids that fall in different lanes, rounds,
    waves and vocabulary splits of full-vocabulary rows: the argmax is the
    lowest of them on each side (reading R1), both from the plain kernels
    (maxima per wave, the search when the wave's maximum rises) and from the
    top-k kernels (maxima per lane, the id located after the loop)."""
    need_gpu()
    n, v = 7, synth.VOCAB
    a, b = synth.logit_rows(synth.LOGITS_F32, range(n), v)
    a[6] = np.linspace(-4.0, 4.0, v, dtype=np.float32)   # the maximum rises all along the row
    m = float(np.ceil(max(a.max(), b.max()))) + 8.0       # an integer: exact in bf16 too
    plants = [[150000, 70000, 200000],                    # different splits
              [5, 6, 1029],                               # one vector, then another lane
              [v - 1, 124160],                            # the last id and a split boundary
              [4, 4100, 8196, 12292],                     # one lane, later rounds
              [99999, 100000, 1000, 63000],
              [0, v - 1],
              [248000, 100]]                              # on the rising row
    for r, ids in enumerate(plants):
        a[r, ids] = m
        b[r, sorted(ids)[1:]] = m                         # the candidate's lowest is the second
    if bf16:
        a, b = synth.f32_to_bf16_bits(a), synth.f32_to_bf16_bits(b)
    da, db = to_dev(a, bf16), to_dev(b, bf16)
    out = kld.kld_from_logits(da, db, None, topk=topk)
    torch.cuda.synchronize()
    got = {k: x.cpu().numpy() for k, x in out.items()}
    want = _oracle(a, b, None, bf16)
    for r, ids in enumerate(plants):
        lo = sorted(ids)
        assert got["argmax_ref"][r] == lo[0], (r, got["argmax_ref"][r], lo)
        assert got["argmax_cand"][r] == lo[1], (r, got["argmax_cand"][r], lo)
    assert np.array_equal(got["argmax_ref"], want["argmax_ref"])
    assert np.array_equal(got["argmax_cand"], want["argmax_cand"])
    assert_kl_close(got["kl"], want["kl"], f"ties bf16={bf16} topk={topk}")


def test_logits_target_out_of_range_gives_nan_nll():
    need_gpu()
    a, b = synth.logit_rows(synth.LOGITS_F32, range(3), 500)
    got = _run(a, b, np.array([-1, 500, 499], np.int32), False)
    assert math.isnan(got["nll_ref"][0]) and math.isnan(got["nll_cand"][1])
    assert np.isfinite(got["nll_ref"][2])


def test_logits_deterministic():
    need_gpu()
    a, b = synth.logit_rows(synth.LOGITS_F32, range(8), 100000)
    r1 = _run(a, b, None, False)
    r2 = _run(a, b, None, False)
    for k in r1:
        assert np.array_equal(r1[k].view(np.uint8), r2[k].view(np.uint8)), k


def test_logits_full_size_f32_all_rows():
    """The f32 workload at full size (512 x 248,320) in the launch the bench
    times; the oracle checks every row, and the device summary of the call
    equals the oracle's summary of the device values (quantiles exactly)."""
    need_gpu()
    n, v = 512, synth.VOCAB
    a, b = synth.logit_rows(synth.LOGITS_F32, range(n), v)
    t = synth.targets(synth.LOGITS_F32, range(n), v)
    got = _run(a, b, t, False)
    want = oracle_rows(a, b, t)
    _compare(got, want, "full f32", strict_mean=True)
    assert np.all(np.isfinite(got["kl"])) and np.all(got["kl"] >= 0)
    qs = (0.5, 0.99, 0.999)
    summ = kld.summary_dict(kld.kld_summary(*(to_dev(got[k]) for k in (
        "kl", "argmax_ref", "argmax_cand", "nll_ref", "nll_cand")), quantiles=qs), qs)
    ow = oracle.summarize(want["kl"], want["argmax_ref"], want["argmax_cand"], want["nll_ref"],
                          want["nll_cand"], quantiles=qs)
    assert summ["top1"] == ow["top1"]
    assert summ["mean_kl"] == pytest.approx(ow["mean_kl"], rel=1e-4)
    assert summ["ppl_ref"] == pytest.approx(ow["ppl_ref"], rel=1e-4)
    assert summ["ppl_cand"] == pytest.approx(ow["ppl_cand"], rel=1e-4)
    for q, hq in zip(qs, host_quantiles(got["kl"], qs)):
        assert summ["quantiles"][q] == hq, q
