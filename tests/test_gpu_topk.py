"""GPU parity of the top-64 export (kld_from_logits with top-k, topk_export)
and of kld_topk_tail against the f64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
import full_vocab_kl_amd as kld
from gpu_util import gpu, need_gpu, to_dev, assert_kl_close

pytestmark = gpu


def _f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


LSE_ABS = 4e-6   # bound on |lse_gpu - lse_f64| from the f32 exponential sums


def assert_lp_close(got_bits, want_bits, where):
    """fp16 log-probs within one fp16 ulp plus the lse error: lp = z - lse is
    rounded once on each side, and near lp = 0 the fp16 spacing is finer than
    the f32-sum error of lse."""
    g, w = _f16(got_bits), _f16(want_bits)
    ulp = np.spacing(np.abs(w).astype(np.float16)).astype(np.float64)
    bad = np.abs(g - w) > ulp + LSE_ABS
    assert not bad.any(), f"{where}: lp off at {np.argwhere(bad)[:5]}"


def _decode(a, bf16):
    return oracle.bf16_bits_to_f64(a) if bf16 else np.asarray(a, np.float64)


def _check_rows(a, b, bf16, where, pad=0):
    n, v = a.shape
    if pad:
        pa = np.zeros((n, v + pad), a.dtype); pa[:, :v] = a
        pb = np.zeros((n, v + pad), b.dtype); pb[:, :v] = b
        da, db = to_dev(pa, bf16)[:, :v], to_dev(pb, bf16)[:, :v]
    else:
        da, db = to_dev(a, bf16), to_dev(b, bf16)
    out = kld.kld_from_logits(da, db, None, topk=True)
    torch.cuda.synchronize()
    got = {k: x.cpu().numpy() for k, x in out.items()}
    want = oracle.score_rows(_decode(a, bf16), _decode(b, bf16), None, k=64)
    for s in ("ref", "cand"):
        assert np.array_equal(got[f"ids_{s}"], want[f"ids_{s}"]), f"{where}: ids {s}"
        assert_lp_close(got[f"lp_{s}"].view(np.uint16), want[f"lp_{s}"], f"{where} {s}")
        # the top-k kernels locate the argmax after their loop
        assert np.array_equal(got[f"argmax_{s}"], want[f"argmax_{s}"]), f"{where}: argmax {s}"
    assert_kl_close(got["kl"], want["kl"], where)
    return got


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("n,v,pad", [(3, 64, 0), (4, 65, 0), (5, 1000, 0), (2, 33000, 8),
                                     (3, 70001, 0), (9, 5003, 1)])
def test_topk_logits_shapes(n, v, pad, bf16):
    need_gpu()
    print(f"case n={n} v={v} pad={pad} bf16={bf16}", flush=True)
    a, b = synth.logit_rows(synth.LOGITS_BF16_TOPK, range(n), v)
    if bf16:
        a, b = synth.f32_to_bf16_bits(a), synth.f32_to_bf16_bits(b)
    _check_rows(a, b, bf16, f"n={n} v={v}", pad)


def test_topk_adversarial_orders_and_ties():
    need_gpu()
    v = 20000
    rows = [np.arange(v, dtype=np.float32) * 1e-3,            # ascending: every element a new max
            -np.arange(v, dtype=np.float32) * 1e-3,           # descending
            np.full(v, 1.5, np.float32),                      # all equal: ids 0..63
            np.round(np.random.default_rng(0).normal(0, 1, v), 1).astype(np.float32),  # heavy ties
            np.where(np.arange(v) % 997 == 0, 5.0, -1.0).astype(np.float32)]  # sparse equal peaks
    a = np.stack(rows)
    b = a[::-1].copy()
    got = _check_rows(a, b, False, "adversarial")
    assert list(got["ids_ref"][2]) == list(range(64))


@pytest.mark.parametrize("bf16", [False, True])
def test_topk_export_single_side_with_target(bf16):
    need_gpu()
    n, v = 6, 50000
    a, _ = synth.logit_rows(synth.LOGITS_BF16_TOPK, range(n), v)
    if bf16:
        a = synth.f32_to_bf16_bits(a)
    t = synth.targets(synth.LOGITS_BF16_TOPK, range(n), v)
    res = kld.topk_export(to_dev(a, bf16), to_dev(t))
    torch.cuda.synchronize()
    x = _decode(a, bf16)
    for i in range(n):
        ids, lp, _ = oracle.topk_row(x[i])
        assert np.array_equal(res["ids"][i].cpu().numpy(), ids)
        assert_lp_close(res["lp"][i].cpu().numpy().view(np.uint16), lp, f"row {i}")
        want_t = -oracle.nll_row(x[i], int(t[i]))
        assert abs(res["target_lp"][i].item() - want_t) <= 1e-5 * max(1.0, abs(want_t))


def test_topk_tail_matches_oracle_on_oracle_lists():
    """The tail kernel on top-64 lists the oracle exports from seeded bf16
    logits, against the oracle's tail KLD on the same lists."""
    need_gpu()
    n, v = 64, 248_320
    a, b = synth.logit_rows(synth.LOGITS_BF16_TOPK, range(n), v, dtype="bf16")
    want = oracle.score_rows(oracle.bf16_bits_to_f64(a), oracle.bf16_bits_to_f64(b), None, k=64)
    lists = [want[k] for k in ("ids_ref", "lp_ref", "ids_cand", "lp_cand")]
    dev = [torch.from_numpy(np.ascontiguousarray(x.view(np.int16) if x.dtype == np.uint16 else x)).cuda()
           for x in lists]
    tail = kld.kld_topk_tail(*dev, v)
    torch.cuda.synchronize()
    wt = np.array([oracle.tail_kld_row(*(x[i] for x in lists), v) for i in range(n)])
    assert_kl_close(tail.cpu().numpy(), wt, "tail")


def test_topk_tail_hand_example_and_edges():
    need_gpu()
    # K = 64 lists built so that the rule's cells are known: the reference
    # lists ids 0..63, the candidate ids 1..64 (id 0 unlisted -> share u)
    v = 1000
    g = np.random.default_rng(3)
    p = g.dirichlet(np.ones(64)) * 0.9
    q = g.dirichlet(np.ones(64)) * 0.8
    lp_p = np.log(p).astype(np.float16).view(np.uint16)[None]
    lp_q = np.log(q).astype(np.float16).view(np.uint16)[None]
    ids_p = np.arange(64, dtype=np.int32)[None]
    ids_q = np.arange(1, 65, dtype=np.int32)[None]
    got = kld.kld_topk_tail(to_dev(ids_p), to_dev(lp_p.view(np.float16)), to_dev(ids_q),
                            to_dev(lp_q.view(np.float16)), v)
    torch.cuda.synchronize()
    want = oracle.tail_kld_row(ids_p[0], lp_p[0], ids_q[0], lp_q[0], v)
    assert_kl_close(got.cpu().numpy(), np.array([want]), "hand")
    # identical lists: exactly 0 up to rounding of the shared tail cell
    same = kld.kld_topk_tail(to_dev(ids_p), to_dev(lp_p.view(np.float16)), to_dev(ids_p),
                             to_dev(lp_p.view(np.float16)), v)
    torch.cuda.synchronize()
    assert abs(same.item()) < 1e-12
