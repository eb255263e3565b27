"""GPU parity of kld_summary against the oracle's aggregation on identical
per-position values."""
import math

import numpy as np
import pytest
import torch

import oracle
import full_vocab_kl_amd as kld
from gpu_util import gpu, need_gpu, to_dev

pytestmark = gpu

QS = (0.0, 0.5, 0.9, 0.99, 0.999, 1.0)


def _run(kl, am_r=None, am_c=None, nr=None, nc=None, qs=QS):
    args = [to_dev(x) if x is not None else None for x in (kl, am_r, am_c, nr, nc)]
    out = kld.kld_summary(*args, quantiles=qs)
    torch.cuda.synchronize()
    return kld.summary_dict(out, qs)


@pytest.mark.parametrize("n", [1, 2, 7, 2047, 16_384, 16_385, 100_003, 262_144])
def test_summary_matches_oracle(n):
    need_gpu()
    g = np.random.default_rng(n)
    kl = g.exponential(4e-4, n).astype(np.float32)
    kl[g.random(n) < 0.05] = 0.0                      # many exact ties at zero
    am_r = g.integers(0, 50, n).astype(np.int32)
    am_c = np.where(g.random(n) < 0.9, am_r, g.integers(0, 50, n)).astype(np.int32)
    nr = g.gamma(2.0, 1.5, n).astype(np.float32)
    nc = (nr + g.normal(0, 0.01, n)).astype(np.float32)
    got = _run(kl, am_r, am_c, nr, nc)
    want = oracle.summarize(kl.astype(np.float64), am_r, am_c, nr, nc, quantiles=QS)
    assert got["mean_kl"] == pytest.approx(want["mean_kl"], rel=1e-12, abs=1e-300)
    assert got["top1"] == want["top1"]
    for k in ("mean_nll_ref", "mean_nll_cand", "ppl_ref", "ppl_cand", "ppl_ratio"):
        assert got[k] == pytest.approx(want[k], rel=1e-12), k
    assert got["n_nonfinite"] == 0
    for q in QS:
        assert got["quantiles"][q] == pytest.approx(want["quantiles"][q], rel=1e-15, abs=0), q


def test_summary_optional_inputs_and_nonfinite():
    need_gpu()
    kl = np.array([0.0, 1e-3, math.inf, 2e-3, math.nan, 5e-4], np.float32)
    got = _run(kl, qs=(0.5,))
    assert got["n_nonfinite"] == 2
    assert math.isnan(got["top1"]) and math.isnan(got["ppl_ref"])
    # ascending bit order: 0, 5e-4, 1e-3, 2e-3, inf, nan -> median between 1e-3 and 2e-3
    assert got["quantiles"][0.5] == pytest.approx(
        float(np.float32(1e-3)) + 0.5 * (float(np.float32(2e-3)) - float(np.float32(1e-3))), rel=1e-15)


def test_summary_deterministic():
    need_gpu()
    kl = np.random.default_rng(1).exponential(1e-3, 50_000).astype(np.float32)
    a = _run(kl)
    b = _run(kl)
    assert repr(a) == repr(b)   # NaN entries (no NLL given) compare equal as text
