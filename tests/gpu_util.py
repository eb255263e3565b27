"""Helpers for the GPU tests: device transfer and tolerance checks."""
import numpy as np
import pytest
import torch

gpu = pytest.mark.gpu


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def to_dev(x: np.ndarray, bf16: bool = False):
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def kl_tol(kl_ref):
    """Per-position KL tolerance: 1e-6 absolute + 1e-3 relative."""
    return 1e-6 + 1e-3 * np.abs(kl_ref)


def assert_kl_close(got, want, where=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    fin = np.isfinite(want)
    assert np.array_equal(np.isnan(got), np.isnan(want)), f"{where}: NaN pattern differs"
    assert np.array_equal(np.isposinf(got), np.isposinf(want)), f"{where}: +inf pattern differs"
    err = np.abs(got[fin] - want[fin])
    tol = kl_tol(want[fin])
    bad = np.flatnonzero(err > tol)
    assert bad.size == 0, f"{where}: KL off at {bad[:8]}: got {got[fin][bad[:4]]} want {want[fin][bad[:4]]}"
    assert np.all(got[fin] >= 0) and not np.any(np.signbit(got[fin]))


def assert_mean_rel(got, want, rel=1e-4, where=""):
    g, w = float(np.mean(got)), float(np.mean(want))
    assert abs(g - w) <= rel * abs(w) + 1e-12, f"{where}: mean KL {g} vs {w}"


def assert_nll_close(got, want, where=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want)), f"{where}: NaN pattern differs"
    fin = np.isfinite(want)
    err = np.abs(got[fin] - want[fin])
    assert np.all(err <= 1e-5 * np.maximum(1.0, np.abs(want[fin]))), f"{where}: NLL max err {err.max()}"


def _threads():
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_rows(a, b, target=None, k=None, block=8):
    """oracle.score_rows over row blocks on a thread pool (numpy releases the
    GIL in the row arithmetic and sorts); the per-row results are the
    oracle's own, concatenated in row order."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle

    n = a.shape[0]
    starts = list(range(0, n, block))

    def one(s):
        t = None if target is None else target[s:s + block]
        return oracle.score_rows(a[s:s + block], b[s:s + block], t, k=k)

    with ThreadPoolExecutor(_threads()) as ex:
        parts = list(ex.map(one, starts))
    return {key: np.concatenate([p[key] for p in parts]) for key in parts[0]}


def top_gaps(z, idx):
    """Per row of z (f64 logits [n, v]): z_(i) - z_(i+1) of the descending
    order for each 1-based rank i in idx (e.g. (1,) for the argmax gap,
    (64,) for the top-64 set gap)."""
    kth = sorted({v - 1 for v in idx} | {v for v in idx})
    part = -np.partition(-z, kth, axis=1)
    return {i: part[:, i - 1] - part[:, i] for i in idx}


def host_quantiles(kl, qs):
    """Type-7 quantiles of the given f32 values with the arithmetic the
    device summary documents: h = q (n - 1) in f64, lo = floor(h), the two
    order statistics widened to f64, lo + (h - lo) (hi - lo)."""
    x = np.sort(np.asarray(kl, np.float32)).astype(np.float64)
    n = x.shape[0]
    res = []
    for q in qs:
        h = float(q) * float(n - 1)
        lo = min(int(h), n - 1)
        hi = min(lo + 1, n - 1)
        res.append(x[lo] + (h - float(lo)) * (x[hi] - x[lo]))
    return res
