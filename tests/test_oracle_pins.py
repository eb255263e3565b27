"""Pins for the f64 oracle against facts fixed by the pages and by mathematics
(closed forms, invariants, hand-worked examples, library routines, brute force
at tiny sizes).  CPU only."""
import itertools
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import scipy.stats
import torch

import oracle

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- decoding

def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x7F80, 0xFF80, 0x0001, 0x7F7F, 0x0000, 0x8000], np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    want = [1.0, -1.0, 3.140625, math.inf, -math.inf, 2.0 ** -133,
            (2 - 2 ** -7) * 2.0 ** 127, 0.0, -0.0]
    assert list(got) == want
    assert math.copysign(1.0, got[-1]) == -1.0


def test_fp16_decode_and_round_to_nearest_even():
    bits = np.array([0x3C00, 0xC000, 0x0001, 0x7BFF, 0xFC00], np.uint16)
    assert list(oracle.fp16_bits_to_f64(bits)) == [1.0, -2.0, 2.0 ** -24, 65504.0, -math.inf]
    # exact halfway cases round to the even neighbour
    x = np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 1 + 2 ** -11 + 2 ** -30, -(1 + 2 ** -11),
                  2.0 ** -25, 3 * 2.0 ** -25])
    got = oracle.fp16_bits_to_f64(oracle.f64_to_fp16_bits(x))
    assert list(got) == [1.0, 1 + 2 ** -9, 1 + 2 ** -10, -1.0, 0.0, 2.0 ** -23]


# ---------------------------------------------------------------- KL

def test_two_token_closed_form_golden():
    g = _gold("two_token.json")
    got = oracle.kl_row(np.array(g["a"]), np.array(g["b"]))
    assert abs(got - float(g["expected_kl"])) < 1e-15


@pytest.mark.parametrize("x,y", [(0.7, -0.3), (-4.0, 2.5), (10.0, 9.99), (0.0, 0.0), (-30.0, 30.0)])
def test_two_token_closed_form_sweep(x, y):
    sig = 1.0 / (1.0 + math.exp(-x))
    softplus = lambda z: max(z, 0.0) + math.log1p(math.exp(-abs(z)))  # noqa: E731
    want = sig * (x - y) + softplus(y) - softplus(x)
    got = oracle.kl_row(np.array([0.0, x]), np.array([0.0, y]))
    assert abs(got - want) <= 1e-13 * max(1.0, abs(want))


def _decimal_kl(a, b):
    getcontext().prec = 40
    ea = [Decimal(float(v)).exp() for v in a]
    eb = [Decimal(float(v)).exp() for v in b]
    za, zb = sum(ea), sum(eb)
    return sum((x / za) * ((x / za).ln() - (y / zb).ln()) for x, y in zip(ea, eb))


@pytest.mark.parametrize("v", [2, 3, 5, 16])
def test_kl_decimal_brute_force(v):
    g = np.random.default_rng(v)
    for _ in range(4):
        a = g.normal(0, 3, v)
        b = a + g.normal(0, 0.5, v)
        want = float(_decimal_kl(a, b))
        got = oracle.kl_row(a, b)
        assert abs(got - want) <= 1e-14 + 1e-12 * want


def test_kl_matches_scipy_entropy():
    g = np.random.default_rng(7)
    a = g.normal(0, 2, 1000)
    b = a + g.normal(0, 0.1, 1000)
    p = np.exp(a - a.max()); p /= p.sum()
    q = np.exp(b - b.max()); q /= q.sum()
    assert abs(oracle.kl_row(a, b) - scipy.stats.entropy(p, q)) < 1e-13


def test_kl_self_is_zero_and_nonnegative():
    g = np.random.default_rng(3)
    for v in (2, 65, 1000):
        a = g.normal(0, 3, v)
        assert oracle.kl_row(a, a) == 0.0
        for s in (0.01, 1.0, 5.0):
            assert oracle.kl_row(a, a + g.normal(0, s, v)) >= -1e-15


@pytest.mark.parametrize("c,cp", [(-1000.0, 7.0), (-3.5, 1000.0), (7.0, -3.5), (1000.0, -1000.0)])
def test_kl_shift_invariance(c, cp):
    g = np.random.default_rng(11)
    a = g.normal(0, 3, 500)
    b = a + g.normal(0, 0.2, 500)
    assert abs(oracle.kl_row(a + c, b + cp) - oracle.kl_row(a, b)) < 1e-12


def test_kl_small_perturbation_asymptote():
    # KL(p || q) -> Var_p(a - b) / 2 as the perturbation shrinks (second-order expansion)
    g = np.random.default_rng(5)
    a = g.normal(0, 2, 4000)
    d = g.normal(0, 1e-3, 4000)
    p = np.exp(a - a.max()); p /= p.sum()
    var = float(np.sum(p * d * d) - np.sum(p * d) ** 2)
    assert abs(oracle.kl_row(a, a + d) - var / 2) < 1e-3 * var


def test_kl_edge_cases():
    inf = math.inf
    # reference -inf entries contribute nothing
    a = np.array([0.0, 1.0, -inf]); b = np.array([0.3, 0.2, 5.0])
    want = float(_decimal_kl([0.0, 1.0], [0.3, 0.2]))  # b's third id only moves lse_b
    lse_b3 = math.log(math.exp(0.3) + math.exp(0.2) + math.exp(5.0))
    lse_b2 = math.log(math.exp(0.3) + math.exp(0.2))
    assert abs(oracle.kl_row(a, b) - (want + lse_b3 - lse_b2)) < 1e-13
    # both -inf at the same id: no contribution
    assert abs(oracle.kl_row(np.array([0.0, 1.0, -inf]), np.array([0.3, 0.2, -inf]))
               - float(_decimal_kl([0.0, 1.0], [0.3, 0.2]))) < 1e-14
    # finite reference against a -inf candidate: +inf
    assert oracle.kl_row(np.array([0.0, 1.0]), np.array([0.0, -inf])) == inf
    # degenerate rows
    assert math.isnan(oracle.kl_row(np.array([-inf, -inf]), np.array([0.0, 1.0])))
    assert math.isnan(oracle.kl_row(np.array([0.0, 1.0]), np.array([-inf, -inf])))
    assert math.isnan(oracle.kl_row(np.array([0.0, math.nan]), np.array([0.0, 1.0])))
    assert math.isnan(oracle.kl_row(np.array([0.0, inf]), np.array([0.0, 1.0])))


# ---------------------------------------------------------------- lse / NLL

def test_nll_matches_torch_cross_entropy():
    g = np.random.default_rng(2)
    x = g.normal(0, 3, (6, 700))
    t = g.integers(0, 700, 6)
    want = torch.nn.functional.cross_entropy(torch.from_numpy(x), torch.from_numpy(t),
                                             reduction="none").numpy()
    got = [oracle.nll_row(x[i], int(t[i])) for i in range(6)]
    assert np.max(np.abs(np.array(got) - want)) < 1e-12


def test_nll_one_hot_limit_and_range():
    x = np.zeros(50); x[7] = 80.0
    assert 0.0 <= oracle.nll_row(x, 7) < 1e-30
    assert math.isnan(oracle.nll_row(x, -1)) and math.isnan(oracle.nll_row(x, 50))


def test_logsumexp_decimal():
    getcontext().prec = 40
    x = np.array([-3.0, 0.5, 2.25, 7.0])
    want = float(sum(Decimal(v).exp() for v in x).ln())
    assert abs(oracle.logsumexp(x) - want) < 1e-14
    assert oracle.logsumexp(np.array([-math.inf, -math.inf])) == -math.inf


# ---------------------------------------------------------------- argmax / top-k

def test_argmax_lowest_id_on_ties():
    assert oracle.argmax_row(np.array([1.0, 3.0, 2.0, 3.0])) == 1
    assert oracle.argmax_row(np.array([-math.inf, -math.inf])) == 0
    assert oracle.argmax_row(np.array([5.0, 5.0, 5.0])) == 0
    assert oracle.argmax_row(np.array([1.0, math.nan, 7.0, 7.0])) == 2
    assert oracle.argmax_row(np.array([math.nan, math.nan])) == 0


def _brute_topk(x, k):
    return [j for _, j in sorted(((-float(v), j) for j, v in enumerate(x)))[:k]]


@pytest.mark.parametrize("v,k", [(16, 4), (16, 16), (1000, 64), (200, 64)])
def test_topk_brute_force(v, k):
    g = np.random.default_rng(v + k)
    x = np.round(g.normal(0, 2, v), 1)      # rounding makes many exact ties
    ids, lp_bits, lp = oracle.topk_row(x, k)
    assert list(ids) == _brute_topk(x, k)
    assert len(set(ids.tolist())) == k
    vals = x[ids]
    assert np.all(np.diff(vals) <= 0)
    lse = oracle.logsumexp(x)
    assert np.array_equal(lp, x[ids] - lse)
    assert np.array_equal(lp_bits, np.asarray(x[ids] - lse).astype(np.float16).view(np.uint16))


def test_topk_hand_built_ties():
    x = np.array([1.0, 2.0, 2.0, 0.5, 2.0, 1.0])
    ids, _, _ = oracle.topk_row(x, 4)
    assert list(ids) == [1, 2, 4, 0]


# ---------------------------------------------------------------- tail rule

def test_tail_example_a_golden():
    g = _gold("tail_example_a.json")
    got = oracle.tail_kld_probs(g["ids_p"], g["p"], g["ids_q"], g["q"], g["v"])
    assert abs(got - float(g["expected_tail_kl"])) < 1e-15
    full = oracle.kl_row(np.log(np.array(g["full_p"])), np.log(np.array(g["full_q"])))
    assert abs(full - float(g["expected_full_kl"])) < 1e-14
    assert got <= full


def test_tail_example_b_golden():
    g = _gold("tail_example_b.json")
    got = oracle.tail_kld_probs(g["ids_p"], g["p"], g["ids_q"], g["q"], g["v"])
    assert abs(got - float(g["expected_tail_kl"])) < 1e-15


def _coarsened_kl(p_full, q_full, cells):
    """Brute force: coarsen full p and q onto the listed ids plus one tail
    cell holding all other ids, then sum p log(p/q) over the cells."""
    pc = [p_full[i] for i in cells] + [1.0 - sum(p_full[i] for i in cells)]
    qc = [q_full[i] for i in cells] + [1.0 - sum(q_full[i] for i in cells)]
    return sum(a * math.log(a / b) for a, b in zip(pc, qc) if a > 0)


@pytest.mark.parametrize("seed", range(6))
def test_tail_rule_exact_when_candidate_uniform_off_its_list(seed):
    # when q is exactly uniform outside its own top-K the spread share equals
    # the true q of every unlisted id, so the rule must equal the brute-force
    # coarsening of the full distributions onto the reference's K ids + tail.
    g = np.random.default_rng(100 + seed)
    v, k = 40, 6
    p = g.dirichlet(np.ones(v) * 0.3)
    q_top_ids = g.choice(v, k, replace=False)
    q = np.zeros(v)
    q[q_top_ids] = g.uniform(0.05, 0.12, k)
    q[np.setdiff1d(np.arange(v), q_top_ids)] = (1 - q.sum()) / (v - k)
    p_ids = np.argsort(-p, kind="stable")[:k]
    q_ids = np.argsort(-q, kind="stable")[:k]
    got = oracle.tail_kld_probs(p_ids, p[p_ids], q_ids, q[q_ids], v)
    want = _coarsened_kl(p, q, list(p_ids))
    assert abs(got - want) < 1e-13
    assert got <= oracle.kl_row(np.log(p), np.log(q)) + 1e-13


def test_tail_rule_zero_when_lists_identical():
    ids = np.array([3, 1, 2]); pr = np.array([0.5, 0.2, 0.1])
    assert oracle.tail_kld_probs(ids, pr, ids, pr, 10) == 0.0


def test_tail_rule_fp16_wrapper_decodes_log_probs():
    lp = np.log(np.array([0.5, 0.25]))
    bits = lp.astype(np.float16).view(np.uint16)
    p = np.exp(bits.view(np.float16).astype(np.float64))
    a = oracle.tail_kld_row([0, 1], bits, [0, 1], bits, 8)
    b = oracle.tail_kld_probs([0, 1], p, [0, 1], p, 8)
    assert a == b == 0.0
    q_bits = np.log(np.array([0.4, 0.3])).astype(np.float16).view(np.uint16)
    q = np.exp(q_bits.view(np.float16).astype(np.float64))
    assert oracle.tail_kld_row([0, 1], bits, [0, 2], q_bits, 8) == \
        oracle.tail_kld_probs([0, 1], p, [0, 2], q, 8)


def test_tail_rule_zero_cell_gives_inf():
    # the candidate lists all 4 ids with full mass on them except the reference's id 3
    assert oracle.tail_kld_probs([3], [0.5], [0, 1, 2], [0.5, 0.3, 0.2], 4) == math.inf


# ---------------------------------------------------------------- head logits

def test_head_logits_exact_small_integers():
    g = np.random.default_rng(9)
    import synth
    w = g.integers(-8, 9, (37, 24)).astype(np.float32)
    h = g.integers(-8, 9, (3, 24)).astype(np.float32)
    wb, hb = synth.f32_to_bf16_bits(w), synth.f32_to_bf16_bits(h)
    got = oracle.head_logits(wb, hb, v_chunk=10)
    want = [[sum(int(w[j, k]) * int(h[i, k]) for k in range(24)) for j in range(37)] for i in range(3)]
    assert np.array_equal(got, np.array(want, dtype=np.float64))


def test_head_byte_count_matches_published_head_size():
    # the fidelity suite's shared head is 2.54 GB: V * d * 2 bytes for bf16
    assert 248_320 * 5120 * 2 == 2_542_796_800


# ---------------------------------------------------------------- aggregation

def test_percentile_matches_numpy_linear():
    g = np.random.default_rng(4)
    for n in (1, 2, 7, 1000, 2047):
        x = g.exponential(1e-3, n)
        for q in (0.0, 0.5, 0.99, 0.999, 1.0):
            assert oracle.percentile(x, q) == pytest.approx(np.percentile(x, 100 * q, method="linear"),
                                                            rel=1e-12, abs=1e-300)


def test_summarize_hand_values():
    s = oracle.summarize(np.array([0.0, 0.25, 0.5, 1.25]), argmax_ref=np.array([1, 2, 3, 4]),
                         argmax_cand=np.array([1, 0, 3, 9]), nll_ref=np.full(4, math.log(5.0)),
                         nll_cand=np.full(4, math.log(6.0)), quantiles=(0.5,))
    assert s["mean_kl"] == 0.5
    assert s["top1"] == 0.5
    assert s["ppl_ref"] == pytest.approx(5.0, rel=1e-15)
    assert s["ppl_ratio"] == pytest.approx(1.2, rel=1e-14)
    assert s["quantiles"][0.5] == 0.375


def test_score_rows_consistency():
    g = np.random.default_rng(12)
    a = g.normal(0, 3, (3, 300)); b = a + g.normal(0, 0.05, (3, 300)); t = np.array([0, 5, 299])
    s = oracle.score_rows(a, b, t, k=8)
    for i in range(3):
        assert s["kl"][i] == oracle.kl_row(a[i], b[i])
        assert s["nll_ref"][i] == oracle.nll_row(a[i], t[i])
        assert list(s["ids_cand"][i]) == _brute_topk(b[i], 8)


# ---------------------------------------------------- golden record + score

def _frac(s):
    from fractions import Fraction
    return float(Fraction(s))


def test_golden_record_hand_example():
    g = _gold("golden_record_example.json")
    p = np.array([_frac(s) for s in g["full_p"]])
    ids, lp, rec = oracle.golden_row(np.log(p), g["target"], k=g["k"])
    assert list(ids) == g["expected_ids"]
    assert np.array_equal(lp, np.log(p[:2]).astype(np.float32))
    assert rec[0] == np.float32(float(g["expected_nll"]))
    assert rec[1] == np.float32(float(g["expected_entropy"]))
    assert rec[2] == np.float32(float(g["expected_tail"]))
    # the score from the exact record (f64 log-probs and tail)
    q = np.array(g["full_q"])
    got = oracle.coarse_kl_row(ids, np.log(p[ids]), 0.25, np.log(q))
    assert abs(got - float(g["expected_score"])) < 1e-15
    # same cells as the top-K + tail rule of the quality-eval reference when q
    # is uniform off its own list (the tail-rule example uses this p, q)
    a = _gold("tail_example_a.json")
    assert abs(got - float(a["expected_tail_kl"])) < 1e-15


@pytest.mark.parametrize("seed", range(4))
def test_golden_entropy_matches_scipy_and_uniform(seed):
    g = np.random.default_rng(400 + seed)
    x = g.normal(0, 2, 3000)
    _, _, rec = oracle.golden_row(x, k=64)
    p = np.exp(x - oracle.logsumexp(x))
    assert abs(float(rec[1]) - scipy.stats.entropy(p)) <= 1e-6 * scipy.stats.entropy(p)
    _, _, rec_u = oracle.golden_row(np.full(1000, 3.25), k=16)
    assert abs(float(rec_u[1]) - math.log(1000)) < 1e-6


@pytest.mark.parametrize("seed", range(4))
def test_golden_ids_brute_force_and_mass(seed):
    g = np.random.default_rng(500 + seed)
    v, k = 2000, 512
    x = np.round(g.normal(0, 1.5, v), 1)      # heavy ties
    ids, lp, rec = oracle.golden_row(x, k=k)
    want = [j for _, j in sorted((-x[j], j) for j in range(v))][:k]
    assert list(ids) == want
    lse = oracle.logsumexp(x)
    assert np.allclose(lp, (x[want] - lse).astype(np.float32), rtol=0, atol=0)
    listed = float(np.sum(np.exp(x[want] - lse)))
    assert abs(listed + float(rec[2]) - 1.0) < 1e-6
    _, _, rec_more = oracle.golden_row(x, k=k + 100)
    assert rec_more[2] <= rec[2]


def _exact_record(x, k):
    lse = oracle.logsumexp(x)
    ids = np.lexsort((np.arange(x.shape[0]), -x))[:k]
    rest = np.setdiff1d(np.arange(x.shape[0]), ids)
    return ids, x[ids] - lse, float(np.sum(np.exp(x[rest] - lse)))


@pytest.mark.parametrize("seed", range(6))
def test_coarse_score_brute_force_and_lower_bound(seed):
    g = np.random.default_rng(600 + seed)
    v, k = 300, int(g.integers(1, 40))
    a = g.normal(0, 2, v)
    b = a + g.normal(0, 0.3, v)
    ids, lp, tail = _exact_record(a, k)
    got = oracle.coarse_kl_row(ids, lp, tail, b)
    p = np.exp(a - oracle.logsumexp(a))
    q = np.exp(b - oracle.logsumexp(b))
    assert abs(got - _coarsened_kl(p, q, list(ids))) < 1e-12
    assert got <= oracle.kl_row(a, b) + 1e-12       # coarsening lowers KL (log-sum inequality)


def test_coarse_score_all_ids_listed_is_full_kl():
    g = np.random.default_rng(7)
    v = 500
    a = g.normal(0, 2, v)
    b = a + g.normal(0, 0.5, v)
    ids, lp, tail = _exact_record(a, v)
    assert tail == 0.0
    assert abs(oracle.coarse_kl_row(ids, lp, tail, b) - oracle.kl_row(a, b)) < 1e-12


def test_coarse_score_edges():
    a = np.log(np.array([0.5, 0.3, 0.2]))
    ids, lp, tail = _exact_record(a, 2)
    assert abs(oracle.coarse_kl_row(ids, lp, tail, a)) < 1e-15       # q = p
    b = np.array([0.0, -np.inf, 0.0])                                 # a listed id with q = 0
    assert oracle.coarse_kl_row(ids, lp, tail, b) == math.inf
    b2 = np.array([0.0, 0.0, -np.inf])                                # q's tail cell empty
    assert oracle.coarse_kl_row(ids, lp, tail, b2) == math.inf


# ---------------------------------------------------- scored windows

def test_window_summary_hand_example():
    # two windows of 5 and 3 positions, score_from 2: scored values are
    # (0.3, 0.4, 0.5) and (0.8,): sums 1.2 and 0.8, mean 2.0 / 4 = 0.5,
    # exceedances of 0.35: 2 + 1 = 3, of 0.8: 0 (strictly greater)
    kl = [0.1, 0.2, 0.3, 0.4, 0.5, 0.6, 0.7, 0.8]
    w = oracle.window_summary(kl, [0, 5, 8], 2, thresholds=(0.35, 0.8))
    assert np.allclose(w["seg_sum"], [1.2, 0.8]) and list(w["seg_count"]) == [3, 1]
    assert abs(w["mean"] - 0.5) < 1e-15 and w["count"] == 4
    assert list(w["exceed"]) == [3, 0]


def test_window_summary_reduces_to_plain_mean_and_brute_force():
    g = np.random.default_rng(31)
    kl = g.exponential(1e-3, 5000)
    offs = np.concatenate([[0], np.sort(g.choice(np.arange(1, 5000), 12, replace=False)), [5000]])
    w0 = oracle.window_summary(kl, offs, 0, thresholds=(1e-3,))
    assert abs(w0["mean"] - oracle.summarize(kl)["mean_kl"]) < 1e-15
    assert w0["exceed"][0] == int(np.sum(kl > 1e-3))
    sf = 37
    w = oracle.window_summary(kl, offs, sf, thresholds=(1e-3, 5e-3))
    mask = np.zeros(5000, bool)
    for i in range(len(offs) - 1):
        mask[min(offs[i] + sf, offs[i + 1]):offs[i + 1]] = True
    assert w["count"] == int(mask.sum())
    assert abs(w["mean"] - kl[mask].mean()) < 1e-15
    assert list(w["exceed"]) == [int(np.sum(kl[mask] > 1e-3)), int(np.sum(kl[mask] > 5e-3))]
    # a segment shorter than score_from contributes nothing
    w_short = oracle.window_summary(kl, [0, 10, 5000], 20)
    assert w_short["seg_count"][0] == 0 and w_short["count"] == 4990 - 20


# ---------------------------------------------------- paired bootstrap

def test_paired_bootstrap_hand_example():
    ex = _gold("paired_bootstrap_example.json")
    r = oracle.paired_bootstrap(ex["sum_a"], ex["sum_b"], ex["count"], ex["cluster"], ex["draws"],
                                ex["quantiles"])
    assert abs(r["diff"] - float(ex["expected_diff"])) < 1e-16
    assert (r["a_wins"], r["b_wins"], r["ties"]) == (ex["expected_a_wins"], ex["expected_b_wins"],
                                                     ex["expected_ties"])
    assert np.allclose(r["replicates"], [float(x) for x in ex["expected_replicates"]], rtol=1e-15,
                       atol=0)
    assert np.allclose(r["quantiles"], [float(x) for x in ex["expected_quantiles"]], rtol=1e-15,
                       atol=0)


def _paired_inputs(seed, nctx, k, equal_counts=True):
    g = np.random.default_rng(seed)
    count = np.full(nctx, 2047) if equal_counts else g.integers(0, 3000, nctx)
    sum_a = g.integers(0, 10 ** 6, nctx).astype(np.float64)       # integer sums: exact in f64
    sum_b = sum_a + g.integers(-5000, 5000, nctx)
    cluster = np.concatenate([np.arange(k), g.integers(0, k, nctx - k)])
    g.shuffle(cluster)
    return sum_a, sum_b, count, cluster


def test_paired_bootstrap_brute_force_over_every_draw():
    # K = 3 clusters, all 27 draw sequences: each replicate recomputed by
    # expanding the drawn clusters into their contexts, in exact rationals
    from fractions import Fraction
    sum_a, sum_b, count, cluster = _paired_inputs(41, 7, 3, equal_counts=False)
    draws = np.array(list(itertools.product(range(3), repeat=3)))
    r = oracle.paired_bootstrap(sum_a, sum_b, count, cluster, draws, (0.5,))
    for d, got in zip(draws, r["replicates"]):
        ctx = [c for k in d for c in range(7) if cluster[c] == k]
        num = sum(Fraction(int(sum_a[c]) - int(sum_b[c])) for c in ctx)
        den = sum(int(count[c]) for c in ctx)
        assert got == float(num / den)
    assert r["quantiles"][0] == np.percentile(r["replicates"], 50.0)
    # the point estimate over all contexts, and the win counts by brute force
    assert r["diff"] == float(Fraction(int(np.sum(sum_a - sum_b)), int(np.sum(count))))
    ma, mb = sum_a / np.maximum(count, 1), sum_b / np.maximum(count, 1)
    wins = [0, 0, 0]
    for c in range(7):
        if count[c]:
            wins[0 if ma[c] < mb[c] else 1 if mb[c] < ma[c] else 2] += 1
    assert [r["a_wins"], r["b_wins"], r["ties"]] == wins


def test_paired_bootstrap_invariants():
    sum_a, sum_b, count, cluster = _paired_inputs(42, 512, 330)
    g = np.random.default_rng(43)
    draws = np.vstack([np.arange(330), g.integers(0, 330, (999, 330))])
    r = oracle.paired_bootstrap(sum_a, sum_b, count, cluster, draws, (0.025, 0.5, 0.975))
    # every cluster drawn once reproduces the point estimate (integer inputs: exact)
    assert r["replicates"][0] == r["diff"]
    # equal counts per context: the position-weighted difference is the
    # mean of the per-context differences
    assert abs(r["diff"] - np.mean(sum_a / 2047 - sum_b / 2047)) < 1e-12
    # percentile interval: numpy's type-7 percentiles of the replicates
    for q, v in zip((0.025, 0.5, 0.975), r["quantiles"]):
        assert v == np.percentile(r["replicates"], 100 * q)
    # swapping the candidates negates the difference, the replicates and the interval
    s = oracle.paired_bootstrap(sum_b, sum_a, count, cluster, draws, (0.025, 0.975))
    assert s["diff"] == -r["diff"] and np.array_equal(s["replicates"], -r["replicates"])
    assert (s["a_wins"], s["b_wins"], s["ties"]) == (r["b_wins"], r["a_wins"], r["ties"])
    assert abs(s["quantiles"][0] + r["quantiles"][2]) <= 1e-12 * abs(r["quantiles"][2])
    assert r["a_wins"] + r["b_wins"] + r["ties"] == 512
    # an interval of a real bootstrap brackets the point estimate here
    assert r["quantiles"][0] < r["diff"] < r["quantiles"][2]


def test_paired_bootstrap_edges():
    # no scored position: NaN difference and NaN replicates
    r = oracle.paired_bootstrap([0.0, 0.0], [0.0, 0.0], [0, 0], [0, 1], [[0, 1]], (0.5,))
    assert math.isnan(r["diff"]) and math.isnan(r["quantiles"][0])
    assert (r["a_wins"], r["b_wins"], r["ties"]) == (0, 0, 0)
    # identical candidates: zero difference, every context tied
    r = oracle.paired_bootstrap([1.0, 2.0], [1.0, 2.0], [3, 4], [0, 1], [[0, 1], [1, 1]], (0.5,))
    assert r["diff"] == 0.0 and r["ties"] == 2 and r["quantiles"][0] == 0.0
