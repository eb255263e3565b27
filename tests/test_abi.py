"""CPU-only checks of the C-ABI library: it loads, exports every symbol that
include/kld.h declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import full_vocab_kl_amd as kld
from full_vocab_kl_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "kld.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kld_\w+|topk_export)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert {"kld_from_logits", "kld_fused_head", "topk_export", "kld_topk_tail", "kld_summary",
            "kld_workspace_size", "kld_status_str", "kld_abi_version"} <= set(names)
    lib = kld.lib()
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(binding.EXPORTED)


def test_abi_version_and_status_strings():
    assert kld.kld_abi_version() == 1
    assert kld.kld_status_str(0) == "KLD_OK"
    for c in range(1, 8):
        assert kld.kld_status_str(c).startswith("KLD_E")


def test_workspace_sizes():
    assert kld.kld_workspace_size(0, 512, 248_320) > 0
    assert kld.kld_workspace_size(0, -1, 10) == 0
    assert kld.kld_workspace_size(99, 1, 10) == 0
    assert kld.kld_workspace_size(0, 0, 10) == 0


def _rows(kl=16):
    return binding._Rows(kl, None, None, None, None, None, None)


def _call_from_logits(ref=16, cand=16, dtype=0, n=4, v=100, ld_ref=100, ld_cand=100, target=None,
                      rows=None, topk=None, ws=16, ws_bytes=1 << 30):
    rows = rows if rows is not None else _rows()
    return kld.lib().kld_from_logits(ref, cand, dtype, n, v, ld_ref, ld_cand, target,
                                     ctypes.byref(rows), topk, ws, ws_bytes, None, None)


def test_from_logits_validation_fails_closed():
    # every case fails validation, so nothing reaches the GPU (fake pointers are never touched)
    assert _call_from_logits(dtype=7) == 3
    assert _call_from_logits(n=-1) == 1
    assert _call_from_logits(ref=None) == 1
    assert _call_from_logits(cand=None) == 1
    assert _call_from_logits(rows=_rows(kl=None)) == 1
    assert _call_from_logits(ld_ref=99) == 2
    assert _call_from_logits(ld_cand=50) == 2
    assert _call_from_logits(v=0) == 2
    nll_rows = binding._Rows(16, 16, None, None, None, None, None)
    assert _call_from_logits(rows=nll_rows, target=None) == 1
    assert _call_from_logits(ws=None) == 4
    assert _call_from_logits(ws_bytes=3) == 4
    tk = binding._Topk(16, 16, 16, 16)
    assert _call_from_logits(v=63, ld_ref=63, ld_cand=63, topk=ctypes.byref(tk)) == 2
    # n == 0 is a valid no-op
    assert _call_from_logits(n=0) == 0


def test_summary_validation_fails_closed():
    lib = kld.lib()
    qs = (ctypes.c_double * 3)(0.5, 0.99, 0.999)
    bad_q = (ctypes.c_double * 1)(1.5)
    call = lambda **k: lib.kld_summary(k.get("kl", 16), k.get("ar", None), k.get("ac", None),  # noqa: E731
                                       k.get("nr", None), k.get("nc", None), k.get("n", 10),
                                       k.get("q", qs), k.get("nq", 3), k.get("out", 16),
                                       k.get("ws", 16), k.get("wsb", 1 << 30), None)
    assert call(kl=None) == 1
    assert call(out=None) == 1
    assert call(ar=16) == 1
    assert call(nc=16) == 1
    assert call(nq=17) == 2
    assert call(q=bad_q, nq=1) == 2
    assert call(q=None) == 1
    assert call(ws=None) == 4
    assert call(wsb=10) == 4
    assert call(n=-1) == 1
    assert call(n=0) == 0


def test_topk_and_tail_validation_fails_closed():
    lib = kld.lib()
    # topk_export(logits, dtype, n, v, ld, k, ids, lp, target, target_lp, ws, ws_bytes, stream)
    ok = dict(logits=16, dtype=0, n=4, v=100, ld=100, k=64, ids=16, lp=16, target=None, tlp=None,
              ws=16, wsb=1 << 30)

    def call(**kw):
        a = {**ok, **kw}
        return lib.topk_export(a["logits"], a["dtype"], a["n"], a["v"], a["ld"], a["k"], a["ids"],
                               a["lp"], a["target"], a["tlp"], a["ws"], a["wsb"], None)
    assert call(k=32) == 2
    assert call(v=63, ld=63) == 2
    assert call(ld=99) == 2
    assert call(dtype=5) == 3
    assert call(ids=None) == 1
    assert call(tlp=16) == 1
    assert call(ws=None) == 4
    assert call(n=0) == 0
    # kld_topk_tail(ids_p, lp_p, ids_q, lp_q, n, k, v, kl_tail, stream)
    assert lib.kld_topk_tail(16, 16, 16, 16, 4, 63, 1000, 16, None) == 2
    assert lib.kld_topk_tail(16, 16, 16, 16, 4, 64, 64, 16, None) == 2
    assert lib.kld_topk_tail(None, 16, 16, 16, 4, 64, 1000, 16, None) == 1
    assert lib.kld_topk_tail(16, 16, 16, 16, 0, 64, 1000, 16, None) == 0


def test_golden_and_coarse_validation_fails_closed():
    lib = kld.lib()
    # kld_golden_export(logits, dtype, n, v, ld, target, k, ids, lp, rec, stream)
    assert lib.kld_golden_export(16, 5, 4, 1000, 1000, None, 512, 16, 16, 16, None) == 3
    assert lib.kld_golden_export(16, 0, -1, 1000, 1000, None, 512, 16, 16, 16, None) == 1
    assert lib.kld_golden_export(16, 0, 4, 1000, 1000, None, 64, 16, 16, 16, None) == 2
    assert lib.kld_golden_export(16, 0, 4, 511, 511, None, 512, 16, 16, 16, None) == 2
    assert lib.kld_golden_export(16, 0, 4, 1000, 999, None, 512, 16, 16, 16, None) == 2
    assert lib.kld_golden_export(None, 0, 4, 1000, 1000, None, 512, 16, 16, 16, None) == 1
    assert lib.kld_golden_export(16, 0, 0, 1000, 1000, None, 512, None, None, None, None) == 0
    # kld_coarse_kl(cand, dtype, n, v, ld, ids, lp, rec, k, kl, stream)
    big = 1 << 30
    assert lib.kld_coarse_kl(16, 9, 4, 1000, 1000, 16, 16, 16, 512, 16, 16, big, None) == 3
    assert lib.kld_coarse_kl(16, 1, 4, 1000, 1000, 16, 16, 16, 100, 16, 16, big, None) == 2
    assert lib.kld_coarse_kl(16, 1, 4, 1000, 1000, 16, None, 16, 512, 16, 16, big, None) == 1
    assert lib.kld_coarse_kl(16, 1, 4, 1000, 1000, 16, 16, 16, 512, 16, None, 0, None) == 4
    assert lib.kld_coarse_kl(16, 1, 4, 1000, 1000, 16, 16, 16, 512, 16, 16, 8, None) == 4
    assert lib.kld_coarse_kl(16, 1, 0, 1000, 1000, None, None, None, 512, None, None, 0, None) == 0
    assert kld.kld_workspace_size(4, 512, 248_320) > 0


def test_window_summary_validation_fails_closed():
    lib = kld.lib()
    thr = (ctypes.c_float * 17)(*range(17))
    # kld_window_summary(kl, n, offsets, nseg, score_from, thr, nthr, seg_sum, seg_count,
    #                    seg_exceed, totals, stream)
    assert lib.kld_window_summary(16, 10, 16, 2, 0, thr, 17, 16, 16, 16, 16, None) == 2
    assert lib.kld_window_summary(16, 10, 16, 2, -1, thr, 1, 16, 16, 16, 16, None) == 1
    assert lib.kld_window_summary(16, -1, 16, 2, 0, thr, 1, 16, 16, 16, 16, None) == 1
    assert lib.kld_window_summary(16, 10, None, 2, 0, thr, 1, 16, 16, 16, 16, None) == 1
    assert lib.kld_window_summary(16, 10, 16, 2, 0, None, 1, 16, 16, 16, 16, None) == 1
    assert lib.kld_window_summary(16, 10, 16, 2, 0, thr, 1, None, 16, 16, 16, None) == 1
    assert lib.kld_window_summary(16, 10, 16, 2, 0, thr, 1, 16, 16, None, 16, None) == 1
    assert lib.kld_window_summary(16, 10, 16, 2, 0, thr, 1, 16, 16, 16, None, None) == 1
    assert lib.kld_window_summary(None, 10, 16, 2, 0, thr, 1, 16, 16, 16, 16, None) == 1


def test_paired_bootstrap_validation_fails_closed():
    lib = kld.lib()
    q = (ctypes.c_double * 17)(*([0.5] * 17))
    bad_q = (ctypes.c_double * 1)(1.5)
    ws = 1 << 20
    # kld_paired_bootstrap(sum_a, sum_b, count, nctx, cluster, nclust, draws, nrep, q, nq,
    #                      replicates, out, ws, ws_bytes, stream)
    assert lib.kld_paired_bootstrap(16, 16, 16, 8, 16, 3, 16, 10, q, 17, 16, 16, 16, ws, None) == 2
    assert lib.kld_paired_bootstrap(16, 16, 16, 8, 16, 3, 16, 16385, q, 2, 16, 16, 16, ws,
                                    None) == 2
    assert lib.kld_paired_bootstrap(16, 16, 16, 8, 16, 0, 16, 10, q, 2, 16, 16, 16, ws, None) == 2
    assert lib.kld_paired_bootstrap(16, 16, 16, -1, 16, 3, 16, 10, q, 2, 16, 16, 16, ws, None) == 1
    assert lib.kld_paired_bootstrap(16, 16, 16, 8, 16, 3, 16, 10, bad_q, 1, 16, 16, 16, ws,
                                    None) == 1
    assert lib.kld_paired_bootstrap(16, None, 16, 8, 16, 3, 16, 10, q, 2, 16, 16, 16, ws,
                                    None) == 1
    assert lib.kld_paired_bootstrap(16, 16, 16, 8, 16, 3, None, 10, q, 2, 16, 16, 16, ws,
                                    None) == 1
    assert lib.kld_paired_bootstrap(16, 16, 16, 8, 16, 3, 16, 10, q, 2, 16, None, 16, ws,
                                    None) == 1
    assert lib.kld_paired_bootstrap(16, 16, 16, 8, 16, 3, 16, 10, q, 2, 16, 16, None, 0,
                                    None) == 4
    assert lib.kld_paired_bootstrap(16, 16, 16, 8, 16, 3, 16, 10, q, 2, 16, 16, 16, 8, None) == 4
    # a workspace that is not 16-byte aligned
    assert lib.kld_paired_bootstrap(16, 16, 16, 8, 16, 3, 16, 10, q, 2, 16, 16, 24, ws, None) == 4
    assert kld.kld_workspace_size(5, 842, 10_000) >= 842 * 16 + 2 * 10_000 * 8


def test_coarse_fused_validation_fails_closed():
    lib = kld.lib()
    big = 1 << 30
    # kld_coarse_fused(W, v, d, h_cand, n, ids, lp, rec, k, kl, ws, ws_bytes, stream, opts)
    assert lib.kld_coarse_fused(16, 1000, 64, 16, 4, 16, 16, 16, 100, 16, 16, big, None, None) == 2
    assert lib.kld_coarse_fused(16, 511, 64, 16, 4, 16, 16, 16, 512, 16, 16, big, None, None) == 2
    assert lib.kld_coarse_fused(16, 1000, 0, 16, 4, 16, 16, 16, 512, 16, 16, big, None, None) == 2
    assert lib.kld_coarse_fused(16, 1000, 64, 16, -1, 16, 16, 16, 512, 16, 16, big, None, None) == 1
    assert lib.kld_coarse_fused(None, 1000, 64, 16, 4, 16, 16, 16, 512, 16, 16, big, None, None) == 1
    assert lib.kld_coarse_fused(16, 1000, 64, 16, 4, None, 16, 16, 512, 16, 16, big, None, None) == 1
    assert lib.kld_coarse_fused(16, 1000, 60, 16, 4, 16, 16, 16, 512, 16, 16, big, None, None) == 5
    assert lib.kld_coarse_fused(16, 1000, 64, 16, 4, 16, 16, 16, 512, 16, None, 0, None, None) == 4
    assert lib.kld_coarse_fused(16, 1000, 64, 16, 4, 16, 16, 16, 512, 16, 16, 8, None, None) == 4
    assert lib.kld_coarse_fused(None, 1000, 64, None, 0, None, None, None, 512, None, None, 0, None,
                                None) == 0
    assert kld.kld_workspace_size(6, 2047, 248_320, 5120) > 3 * 971 * 2048 * 4


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library every entry point raises: there is no other
    path to the results."""
    from full_vocab_kl_amd import binding
    monkeypatch.setattr(binding, "_LIB", None)
    monkeypatch.setattr(binding, "library_path", lambda: str(tmp_path / "libkld.so"))
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()
    with pytest.raises(RuntimeError, match="missing"):
        binding.kld_workspace_size(0, 4, 1000)


def _call_fused(W=16, v=1000, d=64, hr=16, hc=16, n=4, target=None, rows=None, topk=None, ws=16,
                ws_bytes=1 << 30):
    rows = rows if rows is not None else _rows()
    return kld.lib().kld_fused_head(W, v, d, hr, hc, n, target, ctypes.byref(rows), topk, ws,
                                    ws_bytes, None, None)


def test_fused_head_validation_fails_closed():
    # kld_fused_head(W, v, d, h_ref, h_cand, n, target, out, topk, ws, ws_bytes, stream, opts)
    assert _call_fused(W=None) == 1
    assert _call_fused(hr=None) == 1
    assert _call_fused(hc=None) == 1
    assert _call_fused(rows=_rows(kl=None)) == 1
    assert _call_fused(n=-1) == 1
    assert _call_fused(d=-8) == 1
    assert _call_fused(d=0) == 2
    assert _call_fused(d=(1 << 20) + 8) == 2
    assert _call_fused(v=0) == 2
    assert _call_fused(d=60) == 5                     # d % 8 != 0
    assert _call_fused(W=24) == 5                     # head not 16-byte aligned
    assert _call_fused(hr=40) == 5
    assert _call_fused(hc=8) == 5
    assert _call_fused(target=18) == 5                # int32 ids not 4-byte aligned
    assert _call_fused(rows=binding._Rows(18, None, None, None, None, None, None)) == 5
    nll_rows = binding._Rows(16, 16, None, None, None, None, None)
    assert _call_fused(rows=nll_rows, target=None) == 1   # NLL without a target
    tk = binding._Topk(16, 16, 16, 16)
    assert _call_fused(v=63, topk=ctypes.byref(tk)) == 2  # top-64 of fewer than 64 ids
    bad_tk = binding._Topk(16, 17, 16, 16)
    assert _call_fused(topk=ctypes.byref(bad_tk)) == 5   # fp16 list not 2-byte aligned
    need = kld.kld_workspace_size(1, 4, 1000, 64)
    assert need > 0
    assert _call_fused(ws=None) == 4
    assert _call_fused(ws_bytes=need - 1) == 4
    assert _call_fused(ws=24) == 4                    # workspace not 16-byte aligned
    need_topk = kld.kld_workspace_size(1, 4, 1000, 64, 1)
    assert need_topk > need
    assert _call_fused(topk=ctypes.byref(tk), ws_bytes=need) == 4
    assert _call_fused(n=0) == 0


def test_alignment_checked_everywhere():
    """Pointers must be aligned to their element size, workspaces to 16 bytes;
    misalignment is rejected before any launch."""
    lib = kld.lib()
    assert _call_from_logits(ref=18) == 5             # f32 rows need 4 bytes
    assert _call_from_logits(cand=17, dtype=1) == 5
    assert _call_from_logits(target=6) == 5
    assert _call_from_logits(rows=binding._Rows(16, None, None, 18, None, None, None)) == 5
    assert _call_from_logits(ws=40) == 4
    tk = binding._Topk(18, 16, 16, 16)
    assert _call_from_logits(topk=ctypes.byref(tk)) == 5
    # topk_export(logits, dtype, n, v, ld, k, ids, lp, target, target_lp, ws, ws_bytes, stream)
    assert lib.topk_export(16, 0, 4, 100, 100, 64, 18, 16, None, None, 16, 1 << 30, None) == 5
    assert lib.topk_export(16, 0, 4, 100, 100, 64, 16, 17, None, None, 16, 1 << 30, None) == 5
    assert lib.topk_export(16, 0, 4, 100, 100, 64, 16, 16, None, None, 8, 1 << 30, None) == 4
    # kld_topk_tail(ids_p, lp_p, ids_q, lp_q, n, k, v, kl_tail, stream)
    assert lib.kld_topk_tail(18, 16, 16, 16, 4, 64, 1000, 16, None) == 5
    assert lib.kld_topk_tail(16, 16, 16, 17, 4, 64, 1000, 16, None) == 5
    assert lib.kld_topk_tail(16, 16, 16, 16, 4, 64, 1000, 18, None) == 5
    # kld_summary(kl, ar, ac, nr, nc, n, q, nq, out, ws, ws_bytes, stream)
    qs = (ctypes.c_double * 1)(0.5)
    assert lib.kld_summary(18, None, None, None, None, 10, qs, 1, 16, 16, 1 << 30, None) == 5
    assert lib.kld_summary(16, None, None, None, None, 10, qs, 1, 20, 16, 1 << 30, None) == 5
    assert lib.kld_summary(16, None, None, None, None, 10, qs, 1, 16, 8, 1 << 30, None) == 4
    # kld_golden_export(logits, dtype, n, v, ld, target, k, ids, lp, rec, stream)
    assert lib.kld_golden_export(18, 0, 4, 1000, 1000, None, 512, 16, 16, 16, None) == 5
    assert lib.kld_golden_export(16, 0, 4, 1000, 1000, None, 512, 16, 16, 18, None) == 5
    # kld_coarse_kl(cand, dtype, n, v, ld, ids, lp, rec, k, kl, ws, ws_bytes, stream)
    assert lib.kld_coarse_kl(16, 1, 4, 1000, 1000, 18, 16, 16, 512, 16, 16, 1 << 30, None) == 5
    assert lib.kld_coarse_kl(16, 1, 4, 1000, 1000, 16, 16, 16, 512, 16, 24, 1 << 30, None) == 4
    # kld_window_summary(kl, n, offsets, nseg, score_from, thr, nthr, ...)
    thr = (ctypes.c_float * 1)(0.5)
    assert lib.kld_window_summary(16, 10, 20, 2, 0, thr, 1, 16, 16, 16, 16, None) == 5
    # kld_paired_bootstrap(sum_a, sum_b, count, nctx, cluster, nclust, draws, nrep, q, nq, ...)
    q = (ctypes.c_double * 1)(0.5)
    assert lib.kld_paired_bootstrap(20, 16, 16, 8, 16, 3, 16, 10, q, 1, 16, 16, 16, 1 << 20,
                                    None) == 5


def test_noalloc_validation_fails_closed():
    """kld_from_logits_noalloc checks every argument like kld_from_logits and
    rejects requests beyond its static scratch before any HIP call."""
    lib = kld.lib()

    def call(ref=16, cand=16, dtype=0, n=4, v=100, ld_ref=100, ld_cand=100, target=None,
             rows=None, topk=None):
        rows = rows if rows is not None else _rows()
        return lib.kld_from_logits_noalloc(ref, cand, dtype, n, v, ld_ref, ld_cand, target,
                                           ctypes.byref(rows), topk, None, None)
    assert call(dtype=4) == 3
    assert call(n=-1) == 1
    assert call(ref=None) == 1
    assert call(rows=_rows(kl=None)) == 1
    assert call(ld_cand=99) == 2
    assert call(ref=18) == 5
    nll_rows = binding._Rows(16, 16, None, None, None, None, None)
    assert call(rows=nll_rows) == 1
    tk = binding._Topk(16, 16, 16, 16)
    assert call(v=63, ld_ref=63, ld_cand=63, topk=ctypes.byref(tk)) == 2
    assert call(n=0) == 0
    # beyond the static scratch: 20,000 rows of V = 248,320 with top-64
    v = 248_320
    assert kld.kld_workspace_size(0, 20_000, v, 0, 1) > 16 << 20
    assert call(n=20_000, v=v, ld_ref=v, ld_cand=v, topk=ctypes.byref(tk)) == 7
    assert kld.kld_workspace_size(0, 4096, v, 0, 1) <= 16 << 20
