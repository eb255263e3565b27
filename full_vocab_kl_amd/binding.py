"""ctypes binding for libkld.so (include/kld.h).

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; every step of the computation runs in libkld's kernels.
There is no fallback path -- if libkld.so is missing or a call fails, an
exception is raised."""
from __future__ import annotations

import ctypes
import math
import os

import torch

TOPK = 64
KLD_F32, KLD_BF16 = 0, 1
(OP_FROM_LOGITS, OP_FUSED_HEAD, OP_TOPK_EXPORT, OP_SUMMARY, OP_COARSE_KL, OP_PAIRED,
 OP_COARSE_FUSED) = range(7)
FLAG_TOPK = 1
N_SUMMARY_FIXED = 8

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def library_path() -> str:
    return os.path.join(_HERE, "libkld.so")


class KldError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {kld_status_str(code)} ({code})")


class _Rows(ctypes.Structure):
    _fields_ = [("kl", ctypes.c_void_p), ("nll_ref", ctypes.c_void_p), ("nll_cand", ctypes.c_void_p),
                ("lse_ref", ctypes.c_void_p), ("lse_cand", ctypes.c_void_p),
                ("argmax_ref", ctypes.c_void_p), ("argmax_cand", ctypes.c_void_p)]


class _Topk(ctypes.Structure):
    _fields_ = [("ids_ref", ctypes.c_void_p), ("lp_ref", ctypes.c_void_p),
                ("ids_cand", ctypes.c_void_p), ("lp_cand", ctypes.c_void_p)]


class _Opts(ctypes.Structure):
    _fields_ = [("main_start", ctypes.c_void_p), ("main_stop", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGS = {
    "kld_workspace_size": (_SZ, [_I, _I64, _I64, _I64, _I]),
    "kld_from_logits": (_I, [_P, _P, _I, _I64, _I64, _I64, _I64, _P, ctypes.POINTER(_Rows),
                             ctypes.POINTER(_Topk), _P, _SZ, _P, ctypes.POINTER(_Opts)]),
    "kld_from_logits_noalloc": (_I, [_P, _P, _I, _I64, _I64, _I64, _I64, _P, ctypes.POINTER(_Rows),
                                     ctypes.POINTER(_Topk), _P, ctypes.POINTER(_Opts)]),
    "kld_fused_head": (_I, [_P, _I64, _I64, _P, _P, _I64, _P, ctypes.POINTER(_Rows),
                            ctypes.POINTER(_Topk), _P, _SZ, _P, ctypes.POINTER(_Opts)]),
    "topk_export": (_I, [_P, _I, _I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _SZ, _P]),
    "kld_topk_tail": (_I, [_P, _P, _P, _P, _I64, _I, _I64, _P, _P]),
    "kld_summary": (_I, [_P, _P, _P, _P, _P, _I64, _P, _I, _P, _P, _SZ, _P]),
    "kld_golden_export": (_I, [_P, _I, _I64, _I64, _I64, _P, _I, _P, _P, _P, _P]),
    "kld_coarse_kl": (_I, [_P, _I, _I64, _I64, _I64, _P, _P, _P, _I, _P, _P, _SZ, _P]),
    "kld_coarse_fused": (_I, [_P, _I64, _I64, _P, _I64, _P, _P, _P, _I, _P, _P, _SZ, _P,
                              ctypes.POINTER(_Opts)]),
    "kld_window_summary": (_I, [_P, _I64, _P, _I64, _I64, _P, _I, _P, _P, _P, _P, _P]),
    "kld_paired_bootstrap": (_I, [_P, _P, _P, _I64, _P, _I64, _P, _I64, _P, _I, _P, _P, _P, _SZ,
                                  _P]),
    "kld_status_str": (ctypes.c_char_p, [_I]),
    "kld_abi_version": (_I, []),
}
EXPORTED = tuple(_SIGS)


def lib():
    """Load libkld.so (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m full_vocab_kl_amd.build`")
        handle = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def kld_status_str(code: int) -> str:
    return lib().kld_status_str(int(code)).decode()


def kld_abi_version() -> int:
    return int(lib().kld_abi_version())


def kld_workspace_size(op: int, n: int, v: int, d: int = 0, flags: int = 0) -> int:
    return int(lib().kld_workspace_size(op, n, v, d, flags))


# ------------------------------------------------------------------ helpers

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _opts(events):
    """events: None or (start, stop) torch.cuda.Event pair to time the main kernel."""
    if events is None:
        return None
    start, stop = events
    for e in (start, stop):
        if e.cuda_event == 0:      # torch creates the HIP event lazily on first record
            e.record()
    return ctypes.byref(_Opts(start.cuda_event, stop.cuda_event))


def _check(code: int, where: str):
    if code != 0:
        raise KldError(code, where)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return KLD_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return KLD_BF16
    raise TypeError(f"logits must be float32 or bfloat16 (bit patterns), got {t.dtype}")


def _rows_ld(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("logits must be a 2-D tensor with unit stride along the vocabulary")
    return t.stride(0)


def _workspace(op, n, v, d, flags, device, ws):
    need = kld_workspace_size(op, n, v, d, flags)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return ws, need


def _alloc_rows(n, device, target):
    f = dict(dtype=torch.float32, device=device)
    out = {"kl": torch.empty(n, **f), "lse_ref": torch.empty(n, **f), "lse_cand": torch.empty(n, **f),
           "argmax_ref": torch.empty(n, dtype=torch.int32, device=device),
           "argmax_cand": torch.empty(n, dtype=torch.int32, device=device)}
    if target is not None:
        out["nll_ref"] = torch.empty(n, **f)
        out["nll_cand"] = torch.empty(n, **f)
    return out


def _rows_struct(out):
    return _Rows(*(out[k].data_ptr() if out.get(k) is not None else None
                   for k in ("kl", "nll_ref", "nll_cand", "lse_ref", "lse_cand", "argmax_ref",
                             "argmax_cand")))


_TOPK_KEYS = ("ids_ref", "lp_ref", "ids_cand", "lp_cand")


def _topk_from(out, n, device):
    """Reuse top-k buffers present in `out`, else allocate them."""
    if out is not None and all(out.get(k) is not None for k in _TOPK_KEYS):
        return {k: out[k] for k in _TOPK_KEYS}
    return _alloc_topk(n, device)


def _alloc_topk(n, device):
    return {"ids_ref": torch.empty((n, TOPK), dtype=torch.int32, device=device),
            "lp_ref": torch.empty((n, TOPK), dtype=torch.float16, device=device),
            "ids_cand": torch.empty((n, TOPK), dtype=torch.int32, device=device),
            "lp_cand": torch.empty((n, TOPK), dtype=torch.float16, device=device)}


def _topk_struct(tk):
    return _Topk(*(tk[k].data_ptr() if tk.get(k) is not None else None
                   for k in ("ids_ref", "lp_ref", "ids_cand", "lp_cand")))


# ------------------------------------------------------------------ entry points

def kld_from_logits(ref: torch.Tensor, cand: torch.Tensor, target: torch.Tensor | None = None,
                    topk: bool = False, out: dict | None = None, ws: torch.Tensor | None = None,
                    stream=None, events=None) -> dict:
    """Per-position KL(ref || cand), lse, argmax, NLL (with target) and the
    optional top-64 export, from two [n, v] logit tensors on the GPU."""
    n, v = ref.shape
    if cand.shape != ref.shape:
        raise ValueError("ref and cand must have the same shape")
    dt = _dtype_code(ref)
    if _dtype_code(cand) != dt:
        raise TypeError("ref and cand must have the same dtype")
    tk = _topk_from(out, n, ref.device) if topk else None
    out = out if out is not None else _alloc_rows(n, ref.device, target)
    ws, need = _workspace(OP_FROM_LOGITS, n, v, 0, FLAG_TOPK if topk else 0, ref.device, ws)
    rows = _rows_struct(out)
    tks = _topk_struct(tk) if tk else None
    code = lib().kld_from_logits(_ptr(ref), _ptr(cand), dt, n, v, _rows_ld(ref), _rows_ld(cand),
                                 _ptr(target), ctypes.byref(rows),
                                 ctypes.byref(tks) if tks else None, _ptr(ws), ws.numel(),
                                 _stream(stream), _opts(events))
    _check(code, "kld_from_logits")
    if tk:
        out.update(tk)
    return out


def kld_from_logits_noalloc(ref: torch.Tensor, cand: torch.Tensor,
                            target: torch.Tensor | None = None, topk: bool = False,
                            out: dict | None = None, stream=None, events=None) -> dict:
    """kld_from_logits without a workspace: the library's static device
    scratch serves instead.  Pass preallocated outputs in `out` (the rows and,
    with topk, the four top-64 arrays) for a call that allocates nothing."""
    n, v = ref.shape
    if cand.shape != ref.shape:
        raise ValueError("ref and cand must have the same shape")
    dt = _dtype_code(ref)
    if _dtype_code(cand) != dt:
        raise TypeError("ref and cand must have the same dtype")
    tk = _topk_from(out, n, ref.device) if topk else None
    out = out if out is not None else _alloc_rows(n, ref.device, target)
    rows = _rows_struct(out)
    tks = _topk_struct(tk) if tk else None
    code = lib().kld_from_logits_noalloc(_ptr(ref), _ptr(cand), dt, n, v, _rows_ld(ref),
                                         _rows_ld(cand), _ptr(target), ctypes.byref(rows),
                                         ctypes.byref(tks) if tks else None, _stream(stream),
                                         _opts(events))
    _check(code, "kld_from_logits_noalloc")
    if tk:
        out.update(tk)
    return out


def kld_fused_head(W: torch.Tensor, h_ref: torch.Tensor, h_cand: torch.Tensor,
                   target: torch.Tensor | None = None, topk: bool = False, out: dict | None = None,
                   ws: torch.Tensor | None = None, stream=None, events=None) -> dict:
    """Per-position scores from hidden states [n, d] through one shared bf16
    head W [v, d]; logits are never written to memory."""
    v, d = W.shape
    n = h_ref.shape[0]
    for t in (W, h_ref, h_cand):
        if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or not t.is_contiguous():
            raise TypeError("W and hidden states must be contiguous bf16 (or 16-bit bit-pattern) tensors")
    if h_ref.shape != (n, d) or h_cand.shape != (n, d):
        raise ValueError("hidden states must be [n, d] with d = W.shape[1]")
    tk = _topk_from(out, n, W.device) if topk else None
    out = out if out is not None else _alloc_rows(n, W.device, target)
    ws, need = _workspace(OP_FUSED_HEAD, n, v, d, FLAG_TOPK if topk else 0, W.device, ws)
    rows = _rows_struct(out)
    tks = _topk_struct(tk) if tk else None
    code = lib().kld_fused_head(_ptr(W), v, d, _ptr(h_ref), _ptr(h_cand), n, _ptr(target),
                                ctypes.byref(rows), ctypes.byref(tks) if tks else None, _ptr(ws),
                                ws.numel(), _stream(stream), _opts(events))
    _check(code, "kld_fused_head")
    if tk:
        out.update(tk)
    return out


def topk_export(logits: torch.Tensor, target: torch.Tensor | None = None, k: int = TOPK,
                ws: torch.Tensor | None = None, stream=None) -> dict:
    """Top-64 ids (int32) and fp16 log-probs of each row, most likely first,
    plus the true-token log-prob when a target is given."""
    n, v = logits.shape
    dt = _dtype_code(logits)
    ids = torch.empty((n, k), dtype=torch.int32, device=logits.device)
    lp = torch.empty((n, k), dtype=torch.float16, device=logits.device)
    tlp = torch.empty(n, dtype=torch.float32, device=logits.device) if target is not None else None
    ws, need = _workspace(OP_TOPK_EXPORT, n, v, 0, FLAG_TOPK, logits.device, ws)
    code = lib().topk_export(_ptr(logits), dt, n, v, _rows_ld(logits), k, _ptr(ids), _ptr(lp),
                             _ptr(target), _ptr(tlp), _ptr(ws), ws.numel(), _stream(stream))
    _check(code, "topk_export")
    res = {"ids": ids, "lp": lp}
    if tlp is not None:
        res["target_lp"] = tlp
    return res


def kld_topk_tail(ids_p, lp_p, ids_q, lp_q, v: int, k: int = TOPK, out=None, stream=None):
    """Top-64 + one tail bucket KLD per position from two exported lists."""
    n = ids_p.shape[0]
    out = out if out is not None else torch.empty(n, dtype=torch.float32, device=ids_p.device)
    code = lib().kld_topk_tail(_ptr(ids_p), _ptr(lp_p), _ptr(ids_q), _ptr(lp_q), n, k, v, _ptr(out),
                               _stream(stream))
    _check(code, "kld_topk_tail")
    return out


GOLDEN_TOPK = 512


def kld_golden_export(logits: torch.Tensor, target: torch.Tensor | None = None, out: dict | None = None,
                      stream=None) -> dict:
    """Golden records of [n, v] reference logits: ids [n, 512] int32, lp
    [n, 512] f32, rec [n, 3] f32 (NLL of target, entropy, tail mass)."""
    n, v = logits.shape
    dt = _dtype_code(logits)
    if out is None:
        dev = logits.device
        out = {"ids": torch.empty((n, GOLDEN_TOPK), dtype=torch.int32, device=dev),
               "lp": torch.empty((n, GOLDEN_TOPK), dtype=torch.float32, device=dev),
               "rec": torch.empty((n, 3), dtype=torch.float32, device=dev)}
    code = lib().kld_golden_export(_ptr(logits), dt, n, v, _rows_ld(logits), _ptr(target), GOLDEN_TOPK,
                                   _ptr(out["ids"]), _ptr(out["lp"]), _ptr(out["rec"]), _stream(stream))
    _check(code, "kld_golden_export")
    return out


def kld_coarse_kl(cand: torch.Tensor, ids: torch.Tensor, lp: torch.Tensor, rec: torch.Tensor,
                  out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                  stream=None) -> torch.Tensor:
    """513-cell coarsened KL of [n, v] candidate logits against golden records."""
    n, v = cand.shape
    dt = _dtype_code(cand)
    out = out if out is not None else torch.empty(n, dtype=torch.float32, device=cand.device)
    ws, need = _workspace(OP_COARSE_KL, n, v, 0, 0, cand.device, ws)
    code = lib().kld_coarse_kl(_ptr(cand), dt, n, v, _rows_ld(cand), _ptr(ids), _ptr(lp), _ptr(rec),
                               GOLDEN_TOPK, _ptr(out), _ptr(ws), ws.numel(), _stream(stream))
    _check(code, "kld_coarse_kl")
    return out


def kld_coarse_fused(W: torch.Tensor, h_cand: torch.Tensor, ids: torch.Tensor, lp: torch.Tensor,
                     rec: torch.Tensor, out: torch.Tensor | None = None,
                     ws: torch.Tensor | None = None, stream=None, events=None) -> torch.Tensor:
    """513-cell coarsened KL of candidate hidden states [n, d], through the
    shared bf16 head W [v, d], against golden records; logits are never
    written to memory."""
    v, d = W.shape
    n = h_cand.shape[0]
    for t in (W, h_cand):
        if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or not t.is_contiguous():
            raise TypeError("W and hidden states must be contiguous bf16 (or 16-bit bit-pattern) tensors")
    if h_cand.shape != (n, d):
        raise ValueError("hidden states must be [n, d] with d = W.shape[1]")
    out = out if out is not None else torch.empty(n, dtype=torch.float32, device=W.device)
    ws, need = _workspace(OP_COARSE_FUSED, n, v, d, 0, W.device, ws)
    code = lib().kld_coarse_fused(_ptr(W), v, d, _ptr(h_cand), n, _ptr(ids), _ptr(lp), _ptr(rec),
                                  GOLDEN_TOPK, _ptr(out), _ptr(ws), ws.numel(), _stream(stream),
                                  _opts(events))
    _check(code, "kld_coarse_fused")
    return out


def kld_window_summary(kl: torch.Tensor, offsets: torch.Tensor, score_from: int = 0,
                       thresholds=(), out: dict | None = None, stream=None) -> dict:
    """Scored-window statistics: per-segment sums, counts and exceedance
    counts past score_from, the mean over every scored position and the
    exact exceedance counts over all of them."""
    n = kl.shape[0]
    nseg = max(offsets.shape[0] - 1, 0)
    nthr = len(thresholds)
    dev = kl.device
    if out is None:
        out = {"seg_sum": torch.empty(nseg, dtype=torch.float64, device=dev),
               "seg_count": torch.empty(nseg, dtype=torch.int64, device=dev),
               "seg_exceed": torch.empty((nseg, nthr), dtype=torch.int64, device=dev),
               "totals": torch.empty(2 + nthr, dtype=torch.float64, device=dev)}
    th = (ctypes.c_float * max(nthr, 1))(*thresholds)
    code = lib().kld_window_summary(_ptr(kl), n, _ptr(offsets), nseg, int(score_from), th, nthr,
                                    _ptr(out["seg_sum"]), _ptr(out["seg_count"]),
                                    _ptr(out["seg_exceed"]), _ptr(out["totals"]), _stream(stream))
    _check(code, "kld_window_summary")
    return out


def kld_paired_bootstrap(sum_a: torch.Tensor, sum_b: torch.Tensor, count: torch.Tensor,
                         cluster: torch.Tensor, draws: torch.Tensor,
                         quantiles=(0.025, 0.975), ws: torch.Tensor | None = None,
                         stream=None) -> dict:
    """Paired per-context comparison of two candidates with a source-cluster
    bootstrap: the position-weighted difference, contexts won and tied, the
    replicates and their percentiles."""
    nctx = sum_a.shape[0]
    nrep, nclust = draws.shape
    dev = sum_a.device
    reps = torch.empty(nrep, dtype=torch.float64, device=dev)
    out = torch.empty(4 + len(quantiles), dtype=torch.float64, device=dev)
    qs = (ctypes.c_double * max(len(quantiles), 1))(*quantiles)
    ws, need = _workspace(OP_PAIRED, nclust, nrep, 0, 0, dev, ws)
    code = lib().kld_paired_bootstrap(_ptr(sum_a), _ptr(sum_b), _ptr(count), nctx, _ptr(cluster),
                                      nclust, _ptr(draws), nrep, qs, len(quantiles), _ptr(reps),
                                      _ptr(out), _ptr(ws), ws.numel(), _stream(stream))
    _check(code, "kld_paired_bootstrap")
    return {"diff": out[0], "a_wins": out[1], "b_wins": out[2], "ties": out[3],
            "quantiles": out[4:], "replicates": reps, "out": out}


def kld_summary(kl, argmax_ref=None, argmax_cand=None, nll_ref=None, nll_cand=None,
                quantiles=(0.5, 0.99, 0.999), ws=None, out=None, stream=None) -> torch.Tensor:
    """Aggregate per-position scores on the device; returns a float64 device
    tensor laid out as in include/kld.h (see summary_dict)."""
    n = kl.shape[0]
    qs = (ctypes.c_double * len(quantiles))(*quantiles)
    out = out if out is not None else torch.empty(N_SUMMARY_FIXED + len(quantiles),
                                                  dtype=torch.float64, device=kl.device)
    ws, need = _workspace(OP_SUMMARY, n, 0, 0, 0, kl.device, ws)
    code = lib().kld_summary(_ptr(kl), _ptr(argmax_ref), _ptr(argmax_cand), _ptr(nll_ref),
                             _ptr(nll_cand), n, qs, len(quantiles), _ptr(out), _ptr(ws), ws.numel(),
                             _stream(stream))
    _check(code, "kld_summary")
    return out


def summary_dict(vals, quantiles=(0.5, 0.99, 0.999)) -> dict:
    v = [float(x) for x in (vals.cpu().tolist() if hasattr(vals, "cpu") else vals)]
    keys = ("mean_kl", "top1", "mean_nll_ref", "mean_nll_cand", "ppl_ref", "ppl_cand", "ppl_ratio",
            "n_nonfinite")
    d = dict(zip(keys, v[:N_SUMMARY_FIXED]))
    d["quantiles"] = {float(q): v[N_SUMMARY_FIXED + i] for i, q in enumerate(quantiles)}
    return d
