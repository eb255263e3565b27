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
