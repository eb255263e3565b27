"""Throughput of the libkld hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload fused_window]

Default workload: one 2047-position window through the shared head
(d = 5120, V = 248,320, bf16 head and hidden states, f32 softmax).  One step
is the whole path over that window: kld_fused_head (logits, KL, argmax, NLL,
lse and the top-64 export of every position, both sides), kld_topk_tail (the
top-64 + tail-bucket KLD from those exports) and kld_summary (mean KL, top-1,
perplexities, median / p99 / p99.9 KL).  Inputs are seeded synthetic data
already resident in HBM when the timed region starts.

Prints one JSON line: positions/s over K timed steps, the roofline of the
dominant kernel (its average duration from HIP events recorded around it on
the launch stream during the timed steps), a parity block (the GPU's values
at the oracle's sampled positions against the oracle's), the f64 CPU oracle
timed on a bounded sample of the same workload on this host, and the other
workloads (`secondary`): the f32 logits rows, the 32,752-row bf16 top-64
stream, the 32,752-position fused batch, the 262,144-position long trace and
the ranked-next rows.

Measurement helpers (no scoring): --copy-calibration (a plain 1 GiB device
copy, for scaling the FETCH_SIZE / WRITE_SIZE counters), --gemm-calibration
(the vendor library's bf16 GEMM at the head's shape, for comparison),
--read-calibration (torch reductions and a copy over 4 GiB, for comparison),
--record-traffic DIR (turn rocprofv3 FETCH_SIZE / WRITE_SIZE runs into
profiles/traffic.json) and --counter-table DIR (per-kernel averages of any
rocprofv3 counter run).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "scored positions/sec at V=248,320 (fused head d=5120) + % of MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
QUANTILES = (0.5, 0.99, 0.999)
GAP = 1e-3                     # fused-path exemption: oracle top gap below this

WORKLOADS = ("fused_window", "logits_f32", "bf16_topk_stream", "fused_batch", "long_trace",
             "golden_f32", "windows_paired", "coarse_fused_window")


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="fused_window", choices=WORKLOADS)
    p.add_argument("--cpu-sample", type=int, default=None,
                   help="positions the CPU oracle scores for the baseline (0 = skip)")
    p.add_argument("--no-secondary", action="store_true",
                   help="skip the secondary workloads")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (counter calibration)")
    p.add_argument("--read-calibration", action="store_true",
                   help="only time torch reductions and a copy over 4 GiB (comparison)")
    p.add_argument("--gemm-calibration", action="store_true",
                   help="only time the vendor bf16 GEMM at the head's shape (comparison)")
    p.add_argument("--record-traffic", metavar="DIR",
                   help="write profiles/traffic.json from rocprofv3 counter runs under DIR")
    p.add_argument("--counter-table", metavar="DIR",
                   help="print per-kernel averages of the rocprofv3 counter runs under DIR")
    return p.parse_args()


# Dominant kernel of each workload whose traffic the counters record:
# workload -> (traffic key, substring of the kernel's name in rocprofv3 output,
# source file it is built from).
TRAFFIC_KERNELS = {
    "fused_window": ("fused_head_kernel<1>", "fused_head_kernel<1>",
                     "full_vocab_kl_amd/csrc/kld_fused.hip"),
    "long_trace": ("fused_head_kernel<1>@8192", "fused_head_kernel<1>",
                   "full_vocab_kl_amd/csrc/kld_fused.hip"),
    "fused_batch": ("fused_head_kernel<0>", "fused_head_kernel<0>",
                    "full_vocab_kl_amd/csrc/kld_fused.hip"),
    "coarse_fused_window": ("fused_head_kernel<2>", "fused_head_kernel<2>",
                            "full_vocab_kl_amd/csrc/kld_fused.hip"),
    "logits_f32": ("logits_partial_kernel_f32", "logits_partial_kernel<float",
                   "full_vocab_kl_amd/csrc/kld_logits.hip"),
    "bf16_topk_stream": ("logits_partial_kernel_bf16_topk", "logits_partial_kernel<unsigned short",
                         "full_vocab_kl_amd/csrc/kld_logits.hip"),
    "golden_f32": ("coarse_partial_kernel_f32", "coarse_partial_kernel<float",
                   "full_vocab_kl_amd/csrc/kld_golden.hip"),
    "windows_paired": ("window_seg_kernel", "window_seg", "full_vocab_kl_amd/csrc/kld_window.hip"),
}
KERNEL_SOURCES = {key: src for key, _, src in TRAFFIC_KERNELS.values()}


def _code_text(src):
    """The source with comments removed and whitespace collapsed, so that a
    comment edit leaves a kernel's recorded traffic valid (string and
    character literals are kept as written)."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def _sha(path):
    """sha256 of a kernel source's code (_code_text)."""
    import hashlib
    with open(os.path.join(ROOT, path), encoding="utf-8") as f:
        return hashlib.sha256(_code_text(f.read()).encode()).hexdigest()


def _traffic(kernel_key):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel
    calibration) from profiles/traffic.json, or None when missing or when the
    kernel's source has changed since the counters were taken."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f)["kernels"][kernel_key]
        digest = _sha(KERNEL_SOURCES[kernel_key])
    except (OSError, ValueError, KeyError):
        return None
    return rec["bytes_per_launch"] if rec.get("source_sha256") == digest else None


def _cores():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    return max(1, min(n, int(env)) if env and env.isdigit() else n)


def _pool_map(fn, items):
    """fn over items on a pool of _cores() threads (the oracle's numpy row
    arithmetic and sorts release the GIL), results in order."""
    from concurrent.futures import ThreadPoolExecutor
    items = list(items)
    with ThreadPoolExecutor(_cores()) as ex:
        return list(ex.map(fn, items))


def _oracle_scores(za, zb, t, k=None, block=4):
    """oracle.score_rows over row blocks on the thread pool."""
    import numpy as np
    import oracle
    starts = range(0, za.shape[0], block)
    parts = _pool_map(lambda s: oracle.score_rows(za[s:s + block], zb[s:s + block],
                                                  None if t is None else t[s:s + block], k=k),
                      starts)
    return {key: np.concatenate([p[key] for p in parts]) for key in parts[0]}


_HIP = None


def _hip():
    """The HIP runtime this process already uses (the one torch loaded)."""
    global _HIP
    if _HIP is None:
        import ctypes
        import torch
        torch.cuda.init()
        with open("/proc/self/maps") as f:
            path = next(l.split()[-1] for l in f if "libamdhip64" in l)
        h = ctypes.CDLL(path)
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                          ctypes.c_void_p]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
        _HIP = h
    return _HIP


class TimingEvent:
    """A HIP timing event created with hipEventDisableSystemFence: recording it
    takes a timestamp without the system-scope cache writeback and
    invalidation a default event performs, which would slow the kernels that
    follow it (a default event pair around each launch costs a ~200 us step
    about 24 us).  Used only to time kernels; `cuda_event` is the raw handle
    the library records around its dominant kernel."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        h = ctypes.c_void_p()
        if _hip().hipEventCreateWithFlags(ctypes.byref(h), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.cuda_event = h.value

    def record(self):
        import torch
        if _hip().hipEventRecord(self.cuda_event, torch.cuda.current_stream().cuda_stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end):
        import ctypes
        ms = ctypes.c_float()
        if _hip().hipEventElapsedTime(ctypes.byref(ms), self.cuda_event, end.cuda_event) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if _HIP is not None and getattr(self, "cuda_event", None):
            _HIP.hipEventDestroy(self.cuda_event)


_STREAMS = []


def _streams():
    """Two HIP streams (default priority) that consecutive steps alternate on."""
    import torch
    if not _STREAMS:
        _STREAMS.extend(torch.cuda.Stream() for _ in range(2))
    return _STREAMS


class _Chain:
    """The launches of a step made of several calls (chunks, batches), spread
    over the two streams: launch g runs on stream g % 2 and first waits for the
    end of launch g - 1's dominant kernel, so the dominant kernels run one at
    a time while a launch's closing kernels run beside the next launch's
    dominant kernel -- within a step as across steps.  A launch's workspace
    goes by g % 2 (launch g + 2, on the same stream, runs after launch g's
    closing kernels).  One chain serves every step of a workload.  serial:
    every launch on the first stream, one after the other."""

    def __init__(self, serial=False):
        self.serial = serial
        self.g = 0
        self.prev = None
        self.spare = [(TimingEvent(), TimingEvent()) for _ in range(4)]   # untimed launches
        self.tail = [TimingEvent() for _ in range(2)]

    def launch(self, fn, ev=None):
        """fn(parity, (start, stop)) issues one call with the event pair
        around its dominant kernel, on the current stream."""
        import torch
        s = _streams()[0 if self.serial else self.g % 2]
        if (not self.serial and self.prev is not None and
                _hip().hipStreamWaitEvent(s.cuda_stream, self.prev, 0) != 0):
            raise RuntimeError("hipStreamWaitEvent failed")
        pair = ev if ev is not None else self.spare[self.g % len(self.spare)]
        with torch.cuda.stream(s):
            fn(self.g % 2, pair)
        self.prev = pair[1].cuda_event
        self.g += 1

    def join(self):
        """The stream of the last launch, after the other stream's work so
        far: what closes a step (its summary) runs there."""
        ss = _streams()
        if self.serial:
            return ss[0]
        last, other = ss[(self.g - 1) % 2], ss[self.g % 2]
        t = self.tail[self.g % 2]
        if (_hip().hipEventRecord(t.cuda_event, other.cuda_stream) != 0 or
                _hip().hipStreamWaitEvent(last.cuda_stream, t.cuda_event, 0) != 0):
            raise RuntimeError("stream join failed")
        return last


def _timeit(step, steps, warmup, n_ev=1, serial=False):
    """Run warmup untimed steps, then `steps` timed ones; step(i, evs) gets a
    list of n_ev (start, stop) event pairs for the dominant kernel's launches
    (None during warmup).  Step i runs on stream i % 2 and must use buffers
    of its own parity.  Each timed step first waits for the end of the
    previous step's last dominant launch, so the dominant kernels run one at
    a time (each event pair brackets one launch) while one step's small
    closing kernels (finalize, top-64 select, tail KLD, summary) overlap the
    next step's dominant kernel, as a scorer fed batch after batch would run
    them.  serial: every step on the first stream, one after the other.
    Returns (elapsed seconds, mean dominant-kernel ms per launch)."""
    import torch
    evs = [[(TimingEvent(), TimingEvent()) for _ in range(n_ev)] for _ in range(steps)]
    ss = _streams()
    for i in range(warmup):   # one at a time: warmup steps never overlap
        with torch.cuda.stream(ss[0 if serial else i % 2]):
            step(i, None)
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if (not serial and i > 0 and
                _hip().hipStreamWaitEvent(ss[i % 2].cuda_stream, evs[i - 1][-1][1].cuda_event,
                                          0) != 0):
            raise RuntimeError("hipStreamWaitEvent failed")
        with torch.cuda.stream(ss[0 if serial else i % 2]):
            step(i, evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kms = [a.elapsed_time(b) for e in evs for a, b in e]
    return elapsed, sum(kms) / len(kms)


def _roofline(bound, kernel, key, per_launch, kernel_ms, unit_desc):
    if bound == "mfma":
        ach = per_launch / (kernel_ms * 1e-3) / 1e12
        peak, unit = PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        ach = per_launch / (kernel_ms * 1e-3) / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
    return {"bound": bound, "kernel": kernel, "achieved": round(ach, 1), "peak": peak, "unit": unit,
            "frac": round(ach / peak, 4), "traffic": _traffic(key) if key else None,
            "kernel_ms": round(kernel_ms, 4), "algorithmic": unit_desc}


def _bf(x, dev):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)


def _fused_parity(got, want, z, v):
    """GPU values at the oracle's sampled positions against the oracle's:
    KL (max error, error against the per-position bar, relative error of the
    mean), argmax and top-64 sets outside the gap exemption, NLL, and the tail
    KLD on rows whose exported lists equal the oracle's."""
    import numpy as np
    import oracle
    kl = np.asarray(got["kl"], np.float64)
    err = np.abs(kl - want["kl"])
    res = {"positions": int(len(kl)), "max_abs_dkl": float(err.max()),
           "max_dkl_over_bar": float(np.max(err / (1e-6 + 1e-3 * np.abs(want["kl"])))),
           "mean_kl_rel_err": float(abs(kl.mean() - want["kl"].mean()) / abs(want["kl"].mean()))}
    for s in ("ref", "cand"):
        part = -np.partition(-z[s], [0, 1, 63, 64], axis=1)
        g1, g64 = part[:, 0] - part[:, 1], part[:, 63] - part[:, 64]
        ok = g1 >= GAP
        res[f"argmax_{s}_mismatch_outside_exemption"] = int(np.sum(
            got[f"argmax_{s}"][ok] != want[f"argmax_{s}"][ok]))
        if f"ids_{s}" in got and f"ids_{s}" in want:
            differ = np.array([set(got[f"ids_{s}"][i].tolist()) != set(want[f"ids_{s}"][i].tolist())
                               for i in range(len(kl))])
            res[f"top64_{s}_mismatch_outside_exemption"] = int(np.sum(differ & (g64 >= GAP)))
            res[f"top64_{s}_exempt"] = int(np.sum(g64 < GAP))
            res[f"top64_{s}_exempt_differ"] = int(np.sum(differ & (g64 < GAP)))
        if f"nll_{s}" in got and np.isfinite(want[f"nll_{s}"]).all():
            res[f"max_abs_dnll_{s}"] = float(np.max(np.abs(got[f"nll_{s}"] - want[f"nll_{s}"])))
    if "tail" in got and "ids_ref" in want:
        same = [i for i in range(len(kl)) if all(
            np.array_equal(got[f"ids_{s}"][i], want[f"ids_{s}"][i]) and
            np.array_equal(got[f"lp_{s}"][i].view(np.uint16), want[f"lp_{s}"][i])
            for s in ("ref", "cand"))]
        if same:
            wt = np.array([oracle.tail_kld_row(want["ids_ref"][i], want["lp_ref"][i],
                                               want["ids_cand"][i], want["lp_cand"][i], v)
                           for i in same])
            res["tail_rows_compared"] = len(same)
            res["tail_max_abs_err"] = float(np.max(np.abs(got["tail"][same] - wt)))
    return res


def _oracle_fused(w_np, hr, hc, t, k):
    """f64 oracle of sampled fused positions: both sides' logits through the
    head in one product (BLAS threads), then the row definitions on the
    thread pool.  Returns (scores, logits by side, seconds)."""
    import numpy as np
    import oracle
    t0 = time.perf_counter()
    m = hr.shape[0]
    z = oracle.head_logits(w_np, np.concatenate([hr, hc]))
    za, zb = z[:m], z[m:]
    s = _oracle_scores(za, zb, t, k=k)
    if k:
        s["tail"] = np.array(_pool_map(lambda i: oracle.tail_kld_row(
            s["ids_ref"][i], s["lp_ref"][i], s["ids_cand"][i], s["lp_cand"][i], w_np.shape[0]),
            range(m)))
    oracle.summarize(s["kl"], s["argmax_ref"], s["argmax_cand"],
                     s["nll_ref"] if t is not None else None,
                     s["nll_cand"] if t is not None else None)
    return s, {"ref": za, "cand": zb}, time.perf_counter() - t0


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

def fused_window(steps, warmup, cpu_sample):
    """Configuration 1: one 2047-position window with top-64 export, tail KLD
    and summary per step."""
    import numpy as np
    import torch

    import full_vocab_kl_amd as kld
    import synth

    n, v, d = synth.WINDOW_POSITIONS, synth.VOCAB, synth.HIDDEN
    wl = synth.FUSED_WINDOW
    w_np = synth.head_weight(wl, v, d)
    hr_np, hc_np = synth.hidden_rows(wl, range(n), d, 0.01)
    t_np = synth.targets(wl, range(n), v)
    dev = torch.device("cuda:0")
    W, hr, hc = _bf(w_np, dev), _bf(hr_np, dev), _bf(hc_np, dev)
    tg = torch.from_numpy(t_np).to(dev)
    # per stream parity: workspaces and outputs
    ws = [torch.empty(kld.kld_workspace_size(1, n, v, d, 1), dtype=torch.uint8, device=dev)
          for _ in range(2)]
    ws_s = [torch.empty(kld.kld_workspace_size(3, n, 0), dtype=torch.uint8, device=dev)
            for _ in range(2)]
    summs = [torch.empty(8 + len(QUANTILES), dtype=torch.float64, device=dev) for _ in range(2)]
    tails = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(2)]
    outs = [None, None]

    def step(i, ev):
        k = i % 2
        outs[k] = kld.kld_fused_head(W, hr, hc, tg, topk=True, ws=ws[k], out=outs[k],
                                     events=ev[0] if ev else None)
        o = outs[k]
        kld.kld_topk_tail(o["ids_ref"], o["lp_ref"], o["ids_cand"], o["lp_cand"], v, out=tails[k])
        kld.kld_summary(o["kl"], o["argmax_ref"], o["argmax_cand"], o["nll_ref"], o["nll_cand"],
                        quantiles=QUANTILES, ws=ws_s[k], out=summs[k])

    elapsed, kernel_ms = _timeit(step, steps, warmup)
    flops = 4.0 * n * d * v
    summ, tail, box = summs[0], tails[0], {"out": outs[0]}
    summary = kld.summary_dict(summ, QUANTILES)
    res = {
        "value": n * steps / elapsed, "unit": "positions/s", "ms_per_step": elapsed * 1e3 / steps,
        "dtype": "bf16",
        "config": {"workload": "kld_fused_head (+top-64 export) + kld_topk_tail + kld_summary: "
                               "one window, N=2047 positions, d=5120, V=248,320, bf16 head "
                               "W~N(0,0.02^2), hidden RMS-normalised, cand noise 0.01, f32 "
                               "accumulate and softmax",
                   "positions": n, "d": d, "V": v},
        "roofline": _roofline("mfma", "fused_head_kernel<1>", "fused_head_kernel<1>", flops,
                              kernel_ms, f"4*N*d*V = {flops:.4e} flop per launch"),
        "result": {"mean_kl": summary["mean_kl"], "mean_tail_kl": float(tail.double().mean()),
                   "top1": summary["top1"],
                   "ppl_ref": summary["ppl_ref"], "ppl_cand": summary["ppl_cand"],
                   "p99": summary["quantiles"][0.99], "p999": summary["quantiles"][0.999]},
    }
    if cpu_sample:
        rows = synth.subset(wl, n, cpu_sample)
        want, z, dt = _oracle_fused(w_np, hr_np[rows], hc_np[rows], t_np[rows], 64)
        o = box["out"]
        ridx = torch.from_numpy(rows).to(dev)
        got = {k: x[ridx].cpu().numpy() for k, x in o.items()}
        got["tail"] = tail[ridx].cpu().numpy().astype(np.float64)
        res["parity"] = _fused_parity(got, want, z, v)
        res["cpu_baseline"] = {
            "value": len(rows) / dt, "unit": "positions/s", "cores": _cores(), "kind": "oracle",
            "sample": f"{len(rows)} of the 2047 positions of the window: head logits "
                      f"in f64 for both sides over all 248,320 ids (one BLAS product), then KL, "
                      f"argmax, NLL, top-64 and tail KLD per row on {_cores()} threads, and the "
                      f"summary; {dt:.1f} s"}
    return res


def fused_batch(steps, warmup, cpu_sample):
    """Configuration 3: 16 windows = 32,752 positions (candidate noise 0.02)
    through one kld_fused_head call (no top-64), then kld_summary."""
    import torch

    import full_vocab_kl_amd as kld
    import synth

    n, v, d = 16 * synth.WINDOW_POSITIONS, synth.VOCAB, synth.HIDDEN
    w_np = synth.head_weight(synth.FUSED_WINDOW, v, d)
    hr_np, hc_np = synth.hidden_rows(synth.FUSED_BATCH, range(n), d, 0.02)
    t_np = synth.targets(synth.FUSED_BATCH, range(n), v)
    dev = torch.device("cuda:0")
    W, hr, hc = _bf(w_np, dev), _bf(hr_np, dev), _bf(hc_np, dev)
    tg = torch.from_numpy(t_np).to(dev)
    ws = [torch.empty(kld.kld_workspace_size(1, n, v, d, 0), dtype=torch.uint8, device=dev)
          for _ in range(2)]
    ws_s = [torch.empty(kld.kld_workspace_size(3, n, 0), dtype=torch.uint8, device=dev)
            for _ in range(2)]
    summs = [torch.empty(8 + len(QUANTILES), dtype=torch.float64, device=dev) for _ in range(2)]
    outs = [None, None]

    def step(i, ev):
        k = i % 2
        outs[k] = kld.kld_fused_head(W, hr, hc, tg, ws=ws[k], out=outs[k],
                                     events=ev[0] if ev else None)
        o = outs[k]
        kld.kld_summary(o["kl"], o["argmax_ref"], o["argmax_cand"], o["nll_ref"], o["nll_cand"],
                        quantiles=QUANTILES, ws=ws_s[k], out=summs[k])

    elapsed, kernel_ms = _timeit(step, steps, warmup)
    summ, box = summs[0], {"out": outs[0]}
    flops = 4.0 * n * d * v
    summary = kld.summary_dict(summ, QUANTILES)
    res = {
        "value": n * steps / elapsed, "unit": "positions/s", "ms_per_step": elapsed * 1e3 / steps,
        "dtype": "bf16",
        "config": {"workload": "kld_fused_head + kld_summary: 16 windows x 2047 = 32,752 "
                               "positions in one call, d=5120, V=248,320, cand noise 0.02",
                   "positions": n, "d": d, "V": v},
        "roofline": _roofline("mfma", "fused_head_kernel<0>", "fused_head_kernel<0>", flops,
                              kernel_ms, f"4*N*d*V = {flops:.4e} flop per launch"),
        "target_ms": 110.3,
        "result": {"mean_kl": summary["mean_kl"], "top1": summary["top1"],
                   "ppl_ratio": summary["ppl_ratio"], "p99": summary["quantiles"][0.99],
                   "p999": summary["quantiles"][0.999]},
    }
    if cpu_sample:
        import numpy as np
        per = max(1, cpu_sample // 16)
        rows = np.concatenate([wi * synth.WINDOW_POSITIONS + synth.subset(
            synth.FUSED_BATCH * 1000 + wi, synth.WINDOW_POSITIONS, per) for wi in range(16)])
        want, z, dt = _oracle_fused(w_np, hr_np[rows], hc_np[rows], t_np[rows], None)
        ridx = torch.from_numpy(rows).to(dev)
        got = {k: x[ridx].cpu().numpy() for k, x in box["out"].items()}
        res["parity"] = _fused_parity(got, want, z, v)
        res["cpu_baseline"] = {
            "value": len(rows) / dt, "unit": "positions/s", "cores": _cores(), "kind": "oracle",
            "sample": f"{len(rows)} seeded positions ({per} per window): head logits in f64, "
                      f"KL, argmax, NLL, summary; {dt:.1f} s"}
    return res


def long_trace(steps, warmup, cpu_sample):
    """Configuration 4: 262,144 positions in 32 chunks of 8192 rows through
    the head with top-64 export (candidate noise rising linearly from 0.005
    to 0.05 over the chunks); a step is the 32 chunk calls plus kld_summary
    over every position."""
    import numpy as np
    import torch

    import full_vocab_kl_amd as kld
    import synth

    chunk, nchunk = 8192, 32
    n, v, d = chunk * nchunk, synth.VOCAB, synth.HIDDEN
    w_np = synth.head_weight(synth.FUSED_WINDOW, v, d)
    dev = torch.device("cuda:0")
    W = _bf(w_np, dev)
    hr = torch.empty((n, d), dtype=torch.bfloat16, device=dev)
    hc = torch.empty((n, d), dtype=torch.bfloat16, device=dev)
    per = max(1, cpu_sample // nchunk) if cpu_sample else 0
    rows, keep_r, keep_c = [], [], []
    for c in range(nchunk):   # generated chunk by chunk, all resident before timing
        a, b = synth.hidden_rows(synth.LONG_TRACE, range(c * chunk, (c + 1) * chunk), d,
                                 synth.long_trace_noise)
        hr[c * chunk:(c + 1) * chunk] = _bf(a, dev)
        hc[c * chunk:(c + 1) * chunk] = _bf(b, dev)
        if per:   # the oracle's sample, kept from the generated host rows
            sel = synth.subset(synth.LONG_TRACE * 1000 + c, chunk, per)
            rows.append(c * chunk + sel)
            keep_r.append(a[sel])
            keep_c.append(b[sel])
    t_np = synth.targets(synth.LONG_TRACE, range(n), v)
    tg = torch.from_numpy(t_np).to(dev)
    ws = [torch.empty(kld.kld_workspace_size(1, chunk, v, d, 1), dtype=torch.uint8, device=dev)
          for _ in range(2)]
    ws_s = [torch.empty(kld.kld_workspace_size(3, n, 0), dtype=torch.uint8, device=dev)
            for _ in range(2)]
    summs = [torch.empty(8 + len(QUANTILES), dtype=torch.float64, device=dev) for _ in range(2)]

    def outputs():
        o = {k: torch.empty(n, dtype=dt, device=dev) for k, dt in (
            ("kl", torch.float32), ("nll_ref", torch.float32), ("nll_cand", torch.float32),
            ("lse_ref", torch.float32), ("lse_cand", torch.float32), ("argmax_ref", torch.int32),
            ("argmax_cand", torch.int32))}
        o.update({"ids_ref": torch.empty((n, 64), dtype=torch.int32, device=dev),
                  "ids_cand": torch.empty((n, 64), dtype=torch.int32, device=dev),
                  "lp_ref": torch.empty((n, 64), dtype=torch.float16, device=dev),
                  "lp_cand": torch.empty((n, 64), dtype=torch.float16, device=dev)})
        return o
    outs = [outputs() for _ in range(2)]
    views = [[{k: x[c * chunk:(c + 1) * chunk] for k, x in o.items()} for c in range(nchunk)]
             for o in outs]

    chain = _Chain()   # chunk calls alternate streams: a chunk's closing kernels overlap the next

    def step(i, ev):
        k = i % 2
        for c in range(nchunk):
            sl = slice(c * chunk, (c + 1) * chunk)
            chain.launch(lambda p, e: kld.kld_fused_head(W, hr[sl], hc[sl], tg[sl], topk=True,
                                                         ws=ws[p], out=views[k][c], events=e),
                         ev[c] if ev else None)
        o = outs[k]
        with torch.cuda.stream(chain.join()):
            kld.kld_summary(o["kl"], o["argmax_ref"], o["argmax_cand"], o["nll_ref"],
                            o["nll_cand"], quantiles=QUANTILES, ws=ws_s[k], out=summs[k])

    elapsed, kernel_ms = _timeit(step, steps, warmup, n_ev=nchunk)
    summ, out = summs[0], outs[0]
    flops = 4.0 * chunk * d * v
    summary = kld.summary_dict(summ, QUANTILES)
    res = {
        "value": n * steps / elapsed, "unit": "positions/s", "ms_per_step": elapsed * 1e3 / steps,
        "dtype": "bf16",
        "config": {"workload": "kld_fused_head (+top-64 export) x 32 chunks of 8192 + kld_summary: "
                               "262,144 positions, d=5120, V=248,320, cand noise 0.005..0.05 "
                               "over the chunks",
                   "positions": n, "d": d, "V": v, "chunk": chunk},
        "roofline": _roofline("mfma", "fused_head_kernel<1>", "fused_head_kernel<1>@8192", flops,
                              kernel_ms, f"4*chunk*d*V = {flops:.4e} flop per launch (8192 rows)"),
        "target_ms": 883.0,
        "result": {"mean_kl": summary["mean_kl"], "top1": summary["top1"],
                   "ppl_ratio": summary["ppl_ratio"], "p99": summary["quantiles"][0.99],
                   "p999": summary["quantiles"][0.999]},
    }
    if per:
        rows = np.concatenate(rows)
        ridx = torch.from_numpy(rows).to(dev)
        want, z, dt = _oracle_fused(w_np, np.concatenate(keep_r), np.concatenate(keep_c),
                                    t_np[rows], 64)
        got = {k: x[ridx].cpu().numpy() for k, x in out.items()}
        res["parity"] = _fused_parity(got, want, z, v)
        res["cpu_baseline"] = {
            "value": len(rows) / dt, "unit": "positions/s", "cores": _cores(), "kind": "oracle",
            "sample": f"{len(rows)} seeded positions ({per} per chunk): head logits in f64, KL, "
                      f"argmax, NLL, top-64, tail KLD, summary; {dt:.1f} s"}
    return res


def logits_f32(steps, warmup, cpu_sample):
    """Configuration 0: 512 f32 rows, kld_from_logits + kld_summary."""
    import numpy as np
    import torch

    import full_vocab_kl_amd as kld
    import synth

    n, v = 512, synth.VOCAB
    wl = synth.LOGITS_F32
    a_np, b_np = synth.logit_rows(wl, range(n), v)
    t_np = synth.targets(wl, range(n), v)
    dev = torch.device("cuda:0")
    # two copies rotate so that one step's rows are not still in the 256 MB cache
    sets = [(torch.from_numpy(a_np).to(dev), torch.from_numpy(b_np).to(dev)) for _ in range(2)]
    tg = torch.from_numpy(t_np).to(dev)
    ws = [torch.empty(kld.kld_workspace_size(0, n, v), dtype=torch.uint8, device=dev)
          for _ in range(2)]
    ws_s = [torch.empty(kld.kld_workspace_size(3, n, 0), dtype=torch.uint8, device=dev)
            for _ in range(2)]
    summs = [torch.empty(8 + len(QUANTILES), dtype=torch.float64, device=dev) for _ in range(2)]
    outs = [None, None]

    def step(i, ev):
        k = i % 2
        ra, rb = sets[k]
        outs[k] = kld.kld_from_logits(ra, rb, tg, ws=ws[k], out=outs[k],
                                      events=ev[0] if ev else None)
        o = outs[k]
        kld.kld_summary(o["kl"], o["argmax_ref"], o["argmax_cand"], o["nll_ref"], o["nll_cand"],
                        quantiles=QUANTILES, ws=ws_s[k], out=summs[k])

    elapsed, kernel_ms = _timeit(step, steps, warmup)
    box = {"out": outs[0]}
    nbytes = 8.0 * n * v
    res = {
        "value": n * steps / elapsed, "unit": "positions/s", "ms_per_step": elapsed * 1e3 / steps,
        "dtype": "f32",
        "config": {"workload": "kld_from_logits + kld_summary: N=512 rows, V=248,320 f32 logits",
                   "positions": n, "V": v},
        "roofline": _roofline("hbm", "logits_partial_kernel", "logits_partial_kernel_f32", nbytes,
                              kernel_ms, f"8*N*V = {nbytes:.4e} bytes per launch"),
        "target_positions_per_s": 2.82e6,
    }
    if cpu_sample:
        rows = np.arange(min(cpu_sample, n))
        t0 = time.perf_counter()
        want = _oracle_scores(a_np[rows], b_np[rows], t_np[rows])
        dt = time.perf_counter() - t0
        o = box["out"]
        got = {k: x.cpu().numpy()[rows] for k, x in o.items()}
        err = np.abs(got["kl"] - want["kl"])
        res["parity"] = {"positions": int(len(rows)), "max_abs_dkl": float(err.max()),
                         "max_dkl_over_bar": float(np.max(err / (1e-6 + 1e-3 * want["kl"]))),
                         "mean_kl_rel_err": float(abs(got["kl"].astype(np.float64).mean() -
                                                      want["kl"].mean()) / want["kl"].mean()),
                         "argmax_mismatch": int(np.sum(got["argmax_ref"] != want["argmax_ref"]) +
                                                np.sum(got["argmax_cand"] != want["argmax_cand"]))}
        res["cpu_baseline"] = {"value": len(rows) / dt, "unit": "positions/s", "cores": _cores(),
                               "kind": "oracle",
                               "sample": f"rows 0..{len(rows) - 1} (KL, lse, argmax, NLL) on "
                                         f"{_cores()} threads, {dt:.1f} s"}
    return res


def bf16_topk_stream(steps, warmup, cpu_sample):
    """Configuration 2: the 16-window bf16 stream (32,752 rows) in 4096-row
    batches (7 x 4096 + 4080), all resident; a step is every batch's pass
    (full KL + both sides' top-64) and tail KLD, then the summary of the
    whole stream."""
    import numpy as np
    import torch

    import full_vocab_kl_amd as kld
    import synth

    total, bsz, v = 16 * synth.WINDOW_POSITIONS, 4096, synth.VOCAB
    wl = synth.LOGITS_BF16_TOPK
    dev = torch.device("cuda:0")
    batches = []
    for r0 in range(0, total, bsz):
        nb = min(bsz, total - r0)
        a, b = synth.logit_rows(wl, range(r0, r0 + nb), v, dtype="bf16")
        batches.append((r0, nb, _bf(a, dev), _bf(b, dev)))
        del a, b
    ws = [torch.empty(kld.kld_workspace_size(0, bsz, v, 0, 1), dtype=torch.uint8, device=dev)
          for _ in range(2)]
    ws_s = [torch.empty(kld.kld_workspace_size(3, total, 0), dtype=torch.uint8, device=dev)
            for _ in range(2)]
    summs = [torch.empty(8 + len(QUANTILES), dtype=torch.float64, device=dev) for _ in range(2)]

    def outputs():
        o = {k: torch.empty(total, dtype=dt, device=dev) for k, dt in (
            ("kl", torch.float32), ("lse_ref", torch.float32), ("lse_cand", torch.float32),
            ("argmax_ref", torch.int32), ("argmax_cand", torch.int32))}
        o.update({"ids_ref": torch.empty((total, 64), dtype=torch.int32, device=dev),
                  "ids_cand": torch.empty((total, 64), dtype=torch.int32, device=dev),
                  "lp_ref": torch.empty((total, 64), dtype=torch.float16, device=dev),
                  "lp_cand": torch.empty((total, 64), dtype=torch.float16, device=dev)})
        return o
    outs = [outputs() for _ in range(2)]
    tails = [torch.empty(total, dtype=torch.float32, device=dev) for _ in range(2)]
    views = [[{k: x[r0:r0 + nb] for k, x in o.items()} for r0, nb, _, _ in batches] for o in outs]

    # The batches run back to back on one stream: beside the next batch's pass,
    # a batch's closing kernels (merge, tail KLD, finalize; ~0.04 ms) had
    # slowed that pass by more than their own time (0.69 against 0.665 ms per
    # pass, 5.63 against 5.54-5.58 ms per stream, interleaved on one box).
    chain = _Chain(serial=True)

    def step(i, ev):
        k = i % 2
        for j, (r0, nb, ra, rb) in enumerate(batches):
            def call(p, e):
                o = kld.kld_from_logits(ra, rb, None, topk=True, ws=ws[p], out=views[k][j],
                                        events=e)
                kld.kld_topk_tail(o["ids_ref"], o["lp_ref"], o["ids_cand"], o["lp_cand"], v,
                                  out=tails[k][r0:r0 + nb])
            chain.launch(call, ev[j] if ev else None)
        o = outs[k]
        with torch.cuda.stream(chain.join()):
            kld.kld_summary(o["kl"], o["argmax_ref"], o["argmax_cand"], quantiles=QUANTILES,
                            ws=ws_s[k], out=summs[k])   # no targets in this workload: no NLL

    elapsed, kernel_ms = _timeit(step, steps, warmup, n_ev=len(batches), serial=True)
    summ, out, tail = summs[0], outs[0], tails[0]
    nbytes = 4.0 * bsz * v
    mean_ms = kernel_ms
    achieved_bytes = 4.0 * total * v / len(batches)   # average launch
    res = {
        "value": total * steps / elapsed, "unit": "positions/s",
        "ms_per_step": elapsed * 1e3 / steps, "dtype": "bf16",
        "config": {"workload": "kld_from_logits (+top-64 export) + kld_topk_tail per 4096-row "
                               "batch, + kld_summary: 32,752 bf16 rows (16 windows), V=248,320",
                   "positions": total, "V": v, "batches": len(batches)},
        "roofline": _roofline("hbm", "logits_partial_kernel", "logits_partial_kernel_bf16_topk",
                              achieved_bytes, mean_ms,
                              f"4*N*V = {nbytes:.4e} bytes per 4096-row launch "
                              f"({achieved_bytes:.4e} on average over the 8 launches)"),
        "target_ms_per_stream": 5.81,
        "result": {"mean_kl": kld.summary_dict(summ, QUANTILES)["mean_kl"],
                   "mean_tail_kl": float(tail.double().mean()),
                   "top1": kld.summary_dict(summ, QUANTILES)["top1"]},
    }
    if cpu_sample:
        import oracle
        rows = synth.subset(wl * 1000 + 99, total, cpu_sample)
        a, b = synth.logit_rows(wl, rows, v, dtype="bf16")
        t0 = time.perf_counter()
        za, zb = oracle.bf16_bits_to_f64(a), oracle.bf16_bits_to_f64(b)
        want = _oracle_scores(za, zb, None, k=64)
        want["tail"] = np.array(_pool_map(lambda i: oracle.tail_kld_row(
            want["ids_ref"][i], want["lp_ref"][i], want["ids_cand"][i], want["lp_cand"][i], v),
            range(len(rows))))
        dt = time.perf_counter() - t0
        ridx = torch.from_numpy(rows).to(dev)
        got = {k: x[ridx].cpu().numpy() for k, x in out.items()}
        got["tail"] = tail[ridx].cpu().numpy().astype(np.float64)
        err = np.abs(got["kl"] - want["kl"])
        same = [i for i in range(len(rows)) if all(
            np.array_equal(got[f"lp_{s}"][i].view(np.uint16), want[f"lp_{s}"][i]) for s in ("ref", "cand"))]
        res["parity"] = {
            "positions": int(len(rows)), "max_abs_dkl": float(err.max()),
            "max_dkl_over_bar": float(np.max(err / (1e-6 + 1e-3 * want["kl"]))),
            "mean_kl_rel_err": float(abs(got["kl"].astype(np.float64).mean() - want["kl"].mean()) /
                                     want["kl"].mean()),
            "top64_ids_mismatch": int(sum(not np.array_equal(got[f"ids_{s}"][i], want[f"ids_{s}"][i])
                                          for i in range(len(rows)) for s in ("ref", "cand"))),
            "tail_rows_compared": len(same),
            "tail_max_abs_err": float(np.max(np.abs(got["tail"][same] - want["tail"][same])))
            if same else None}
        res["cpu_baseline"] = {"value": len(rows) / dt, "unit": "positions/s", "cores": _cores(),
                               "kind": "oracle",
                               "sample": f"{len(rows)} seeded rows of the stream (KL, argmax, lse, "
                                         f"top-64 + tail KLD) on {_cores()} threads, {dt:.1f} s"}
    return res


def golden_f32(steps, warmup, cpu_sample):
    """The 512 f32 rows of the logits workload scored the challenge's way: the
    reference rows' golden records (512 listed ids + NLL, entropy, tail mass;
    written once, timed apart) and, per step, the candidate rows' 513-cell
    coarsened KL against them plus the summary."""
    import numpy as np
    import torch

    import full_vocab_kl_amd as kld
    import synth

    n, v = 512, synth.VOCAB
    wl = synth.LOGITS_F32
    a_np, b_np = synth.logit_rows(wl, range(n), v)
    t_np = synth.targets(wl, range(n), v)
    dev = torch.device("cuda:0")
    ra, rb = torch.from_numpy(a_np).to(dev), torch.from_numpy(b_np).to(dev)
    tg = torch.from_numpy(t_np).to(dev)
    rec = kld.kld_golden_export(ra, tg)
    ws = [torch.empty(kld.kld_workspace_size(4, n, v), dtype=torch.uint8, device=dev)
          for _ in range(2)]
    ws_s = [torch.empty(kld.kld_workspace_size(3, n, 0), dtype=torch.uint8, device=dev)
            for _ in range(2)]
    summs = [torch.empty(8 + len(QUANTILES), dtype=torch.float64, device=dev) for _ in range(2)]
    kls = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(2)]

    def step(i, ev):
        k = i % 2
        if ev:
            ev[0][0].record()
        kld.kld_coarse_kl(rb, rec["ids"], rec["lp"], rec["rec"], out=kls[k], ws=ws[k])
        if ev:
            ev[0][1].record()
        kld.kld_summary(kls[k], quantiles=QUANTILES, ws=ws_s[k], out=summs[k])

    torch.cuda.synchronize()
    e0, e1 = TimingEvent(), TimingEvent()
    e0.record()
    kld.kld_golden_export(ra, tg, out=rec)
    e1.record()
    torch.cuda.synchronize()
    export_ms = e0.elapsed_time(e1)
    elapsed, kernel_ms = _timeit(step, steps, warmup)   # (warmup on both streams)
    nbytes = 4.0 * n * v
    summary = kld.summary_dict(summs[0], QUANTILES)
    res = {
        "value": n * steps / elapsed, "unit": "positions/s", "ms_per_step": elapsed * 1e3 / steps,
        "dtype": "f32",
        "config": {"workload": "kld_coarse_kl + kld_summary against golden records "
                               "(kld_golden_export, 512 listed ids): N=512 rows, V=248,320 f32",
                   "positions": n, "V": v},
        "roofline": _roofline("hbm", "coarse_partial_kernel + coarse_finalize_kernel",
                              "coarse_partial_kernel_f32", nbytes, kernel_ms,
                              f"4*N*V = {nbytes:.4e} bytes per call (candidate rows once)"),
        "export_ms": round(export_ms, 4),
        "result": {"mean_coarse_kl": summary["mean_kl"],
                   "mean_tail_mass": float(rec["rec"][:, 2].double().mean())},
    }
    if cpu_sample:
        import oracle
        rows = np.arange(min(cpu_sample, n))
        t0 = time.perf_counter()

        def one(i):
            g = oracle.golden_rows(a_np[i:i + 1], t_np[i:i + 1])
            return oracle.coarse_kl_rows(g["ids"], g["lp"], g["rec"], b_np[i:i + 1])
        _pool_map(one, rows)
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": len(rows) / dt, "unit": "positions/s", "cores": _cores(),
                               "kind": "oracle",
                               "sample": f"first {len(rows)} rows (golden record + coarsened score) "
                                         f"on {_cores()} threads, {dt:.1f} s"}
    return res


def windows_paired(steps, warmup, cpu_sample):
    """The ten-shard ladder's aggregation: 10,480,640 scored positions as
    5,120 contexts of 2,047 positions in 842 source clusters.  One step is
    kld_window_summary over each of two candidates' per-position scores
    (per-context sums and counts, overall mean, exceedance counts against
    seven thresholds) and kld_paired_bootstrap (the paired difference, wins
    and ties, 10,000 cluster-bootstrap replicates and their 2.5 / 50 / 97.5 %
    percentiles)."""
    import numpy as np
    import torch

    import full_vocab_kl_amd as kld
    import synth

    nctx, per, nclust, nrep = 5120, 2047, 842, 10_000
    n = nctx * per
    thr = (0.0, 0.01, 0.1, 0.5, 1.0, 2.0, 5.0)
    qs = (0.025, 0.5, 0.975)
    a_np, b_np = synth.kl_score_pair(synth.LOGITS_F32, n)
    lab_np = synth.cluster_labels(synth.LOGITS_F32, nctx, nclust)
    dr_np = synth.bootstrap_draws(synth.LOGITS_F32, nrep, nclust)
    off_np = np.arange(0, n + 1, per, dtype=np.int64)
    dev = torch.device("cuda:0")
    a, b = torch.from_numpy(a_np).to(dev), torch.from_numpy(b_np).to(dev)
    off, lab, dr = (torch.from_numpy(x).to(dev) for x in (off_np, lab_np, dr_np))

    def wout():
        return {"seg_sum": torch.empty(nctx, dtype=torch.float64, device=dev),
                "seg_count": torch.empty(nctx, dtype=torch.int64, device=dev),
                "seg_exceed": torch.empty((nctx, len(thr)), dtype=torch.int64, device=dev),
                "totals": torch.empty(2 + len(thr), dtype=torch.float64, device=dev)}
    was, wbs = [wout() for _ in range(2)], [wout() for _ in range(2)]
    ws_p = [torch.empty(kld.kld_workspace_size(5, nclust, nrep), dtype=torch.uint8, device=dev)
            for _ in range(2)]
    ev_p = [(TimingEvent(), TimingEvent()) for _ in range(steps)]
    box = {"k": 0}

    def step(i, ev):
        k = i % 2
        wa, wb = was[k], wbs[k]
        if ev:
            ev[0][0].record()
        kld.kld_window_summary(a, off, 0, thr, out=wa)
        kld.kld_window_summary(b, off, 0, thr, out=wb)
        if ev:
            ev[0][1].record()
            ev_p[i][0].record()
        box["p"] = kld.kld_paired_bootstrap(wa["seg_sum"], wb["seg_sum"], wa["seg_count"], lab,
                                            dr, qs, ws=ws_p[k])
        if ev:
            ev_p[i][1].record()

    elapsed, w_ms = _timeit(step, steps, warmup)
    p_ms = sum(x.elapsed_time(y) for x, y in ev_p) / steps
    nbytes = 2 * (4.0 * n + 8.0 * (nctx + 1) + (16.0 + 8.0 * len(thr)) * nctx)
    out = box["p"]["out"].cpu().numpy()
    wtr = _traffic("window_seg_kernel")
    roof = _roofline("hbm", "window_seg_wave_kernel + window_total_kernel (two candidates)", None,
                     nbytes, w_ms, "2 x (4 B per position + 8 B per offset + 16 B + 8 B per "
                                   f"threshold per context of output) = {nbytes:.4e} bytes")
    roof["traffic"] = None if wtr is None else 2 * wtr
    res = {
        "value": n * steps / elapsed, "unit": "positions/s", "ms_per_step": elapsed * 1e3 / steps,
        "dtype": "f64",
        "config": {"workload": "kld_window_summary x 2 + kld_paired_bootstrap: 10,480,640 scored "
                               "positions = 5,120 contexts x 2,047, 842 clusters, 10,000 replicates",
                   "positions": n, "contexts": nctx, "clusters": nclust, "replicates": nrep},
        "roofline": roof,
        "paired_ms": round(p_ms, 4),
        "result": {"diff": float(out[0]), "a_wins": int(out[1]), "b_wins": int(out[2]),
                   "interval_95": [float(out[4]), float(out[6])]},
    }
    if cpu_sample:
        import oracle
        sub = min(cpu_sample, nrep)
        t0 = time.perf_counter()
        oa = oracle.window_summary(a_np, off_np, 0, thr)
        ob = oracle.window_summary(b_np, off_np, 0, thr)
        t1 = time.perf_counter()
        oracle.paired_bootstrap(oa["seg_sum"], ob["seg_sum"], oa["seg_count"], lab_np,
                                dr_np[:sub], qs)
        t2 = time.perf_counter()
        per_step = (t1 - t0) + (t2 - t1) * nrep / sub
        res["cpu_baseline"] = {"value": n / per_step, "unit": "positions/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"both window summaries in full ({t1 - t0:.1f} s) and "
                                         f"{sub} of the {nrep} replicates ({t2 - t1:.1f} s), "
                                         "scaled to the full step; one thread"}
    return res


def coarse_fused_window(steps, warmup, cpu_sample):
    """One 2047-position window of a candidate given as hidden states (d =
    5120) through the shared bf16 head (V = 248,320), scored against stored
    golden records (512 listed ids + tail): one step is kld_coarse_fused and
    kld_summary.  Records are seeded stand-ins of the golden format."""
    import numpy as np
    import torch

    import full_vocab_kl_amd as kld
    import synth

    n, v, d = synth.WINDOW_POSITIONS, synth.VOCAB, synth.HIDDEN
    wl = synth.FUSED_WINDOW
    w_np = synth.head_weight(wl, v, d)
    _, hc_np = synth.hidden_rows(wl, range(n), d, 0.01)
    ids_np, lp_np, rec_np = synth.sparse_records(wl, n, v)
    dev = torch.device("cuda:0")
    W, hc = _bf(w_np, dev), _bf(hc_np, dev)
    ids, lp, rec = (torch.from_numpy(x).to(dev) for x in (ids_np, lp_np, rec_np))
    ws = [torch.empty(kld.kld_workspace_size(6, n, v, d), dtype=torch.uint8, device=dev)
          for _ in range(2)]
    ws_s = [torch.empty(kld.kld_workspace_size(3, n, 0), dtype=torch.uint8, device=dev)
            for _ in range(2)]
    summs = [torch.empty(8 + len(QUANTILES), dtype=torch.float64, device=dev) for _ in range(2)]
    kls = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(2)]

    def step(i, ev):
        k = i % 2
        kld.kld_coarse_fused(W, hc, ids, lp, rec, out=kls[k], ws=ws[k],
                             events=ev[0] if ev else None)
        kld.kld_summary(kls[k], quantiles=QUANTILES, ws=ws_s[k], out=summs[k])

    elapsed, kernel_ms = _timeit(step, steps, warmup)
    summ = summs[0]
    flops = 2.0 * n * d * v
    summary = kld.summary_dict(summ, QUANTILES)
    res = {
        "value": n * steps / elapsed, "unit": "positions/s", "ms_per_step": elapsed * 1e3 / steps,
        "dtype": "bf16",
        "config": {"workload": "kld_coarse_fused + kld_summary: one window, N=2047 candidate "
                               "positions as hidden states, d=5120, V=248,320 through the shared "
                               "bf16 head, scored against 512-id golden records + tail",
                   "positions": n, "d": d, "V": v},
        "roofline": _roofline("mfma", "fused_head_kernel<2> (sparse mode)", "fused_head_kernel<2>",
                              flops, kernel_ms,
                              f"2*N*d*V = {flops:.4e} flop per launch (candidate side only)"),
        "result": {"mean_coarse_kl_vs_stand_in_records": summary["mean_kl"]},
    }
    if cpu_sample:
        import oracle
        rows = synth.subset(wl, n, cpu_sample)
        t0 = time.perf_counter()
        zb = oracle.head_logits(w_np, hc_np[rows])
        _pool_map(lambda i: oracle.coarse_kl_rows(ids_np[rows[i:i + 1]], lp_np[rows[i:i + 1]],
                                                  rec_np[rows[i:i + 1]], zb[i:i + 1]),
                  range(len(rows)))
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": len(rows) / dt, "unit": "positions/s", "cores": _cores(),
                               "kind": "oracle",
                               "sample": f"{len(rows)} seeded positions of the window (head logits "
                                         f"in f64 over all 248,320 ids, 513-cell score), {dt:.1f} s"}
    return res


FUNCS = {"fused_window": fused_window, "logits_f32": logits_f32,
         "bf16_topk_stream": bf16_topk_stream, "fused_batch": fused_batch,
         "long_trace": long_trace, "golden_f32": golden_f32, "windows_paired": windows_paired,
         "coarse_fused_window": coarse_fused_window}
# default oracle sample per workload when it runs on its own / as a secondary entry
CPU_SAMPLE = {"fused_window": (2047, None), "logits_f32": (512, 512),
              "bf16_topk_stream": (2048, 2048), "fused_batch": (768, 768), "long_trace": (768, 768),
              "golden_f32": (64, 0), "windows_paired": (10_000, 0), "coarse_fused_window": (64, 0)}
SECONDARY_STEPS = {"long_trace": 3, "fused_batch": 3, "bf16_topk_stream": 5}


# --------------------------------------------------------------------------
# measurement helpers
# --------------------------------------------------------------------------

def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device copy of known size, for scaling the FETCH_SIZE /
    WRITE_SIZE counters (run under rocprofv3 --pmc)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def gemm_calibration(reps=10):
    """The vendor library's bf16 GEMM (torch.matmul, hipBLASLt) at the head's
    shape: [248,320 x 5120] x [5120 x N] for N = 4096 (both sides of a window)
    and 8192, bf16 output, no epilogue.  A comparison point for the fused
    kernel's MFMA rate on the same chip, not part of the path."""
    import torch
    dev = torch.device("cuda:0")
    m, k = 248_320, 5120
    res = []
    g = torch.Generator(device=dev)
    g.manual_seed(20261203)
    W = (torch.randn(m, k, device=dev, generator=g) * 0.02).to(torch.bfloat16)
    for n in (4096, 8192):
        H = torch.randn(k, n, device=dev, generator=g).to(torch.bfloat16).contiguous()
        for _ in range(3):
            C = torch.matmul(W, H)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            C = torch.matmul(W, H)
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
        res.append({"gemm": f"{m}x{n}x{k} bf16", "ms": round(ms, 4), "tflops": round(tf, 1),
                    "frac_of_2500": round(tf / PEAK_BF16_TFLOPS, 4)})
        del H, C
    print(json.dumps({"gemm_calibration": res}), flush=True)


def read_calibration(reps=10):
    """Library streaming rates on the same chip, for comparison with the
    logits passes: torch.sum and torch.amax over a resident 4 GiB f32 tensor
    (read once) and torch's clone of it (read and write).  Not part of the
    path."""
    import torch
    dev = torch.device("cuda:0")
    n = (4 << 30) // 4
    x = torch.randn(n, device=dev)
    res = []
    for name, fn, moved in (("sum", lambda: x.sum(), 4 * n), ("amax", lambda: x.amax(), 4 * n),
                            ("clone", lambda: x.clone(), 8 * n)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        gbs = moved / (ms * 1e-3) / 1e9
        res.append({"op": f"torch.{name}, 4 GiB f32", "ms": round(ms, 4), "GB/s": round(gbs, 1),
                    "frac_of_8000": round(gbs / PEAK_HBM_GBS, 4)})
    print(json.dumps({"read_calibration": res}), flush=True)


def _read_counter_csv(d):
    """Rows of every rocprofv3 counter_collection CSV under d."""
    import csv
    import glob
    rows = []
    for p in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(p) as f:
            rows.extend(csv.DictReader(f))
    return rows


def _per_dispatch(rows, counter, part):
    """Per-dispatch values of one counter for kernels whose name contains
    `part` (summed over the counter's instances)."""
    from collections import defaultdict
    acc = defaultdict(float)
    for r in rows:
        if r.get("Counter_Name") == counter and part in r.get("Kernel_Name", ""):
            acc[r.get("Dispatch_Id")] += float(r["Counter_Value"])
    return [acc[k] for k in sorted(acc, key=lambda x: int(x))]


def record_traffic(d):
    """profiles/traffic.json from rocprofv3 --pmc runs under d: for each
    workload w run on its own, d/w/pmc_FETCH_SIZE and d/w/pmc_WRITE_SIZE, and
    for the calibration d/cal_FETCH_SIZE and d/cal_WRITE_SIZE
    (--copy-calibration).  Bytes per launch of w's dominant kernel = its
    average FETCH_SIZE x (copy bytes / the copy's FETCH_SIZE) + the same for
    WRITE_SIZE."""
    copy_kib = (1 << 30) / 1024.0
    scale = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        vals = _per_dispatch(_read_counter_csv(os.path.join(d, f"cal_{c}")), c, "")
        vals = [x for x in vals if x > 0.25 * copy_kib]
        scale[c] = copy_kib / (sum(vals) / len(vals))
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {"kernels": {}}
    rec["note"] = ("HBM-side bytes per launch of each workload's dominant kernel: FETCH_SIZE and "
                   "WRITE_SIZE (rocprofv3 --pmc, one counter per run, the workload run on its "
                   "own) scaled by the same counters on a plain copy of known size. "
                   "source_sha256: of the kernel source with comments removed and whitespace "
                   "collapsed.")
    for wl, (key, part, src) in TRAFFIC_KERNELS.items():
        f = _per_dispatch(_read_counter_csv(os.path.join(d, wl, "pmc_FETCH_SIZE")), "FETCH_SIZE",
                          part)
        w = _per_dispatch(_read_counter_csv(os.path.join(d, wl, "pmc_WRITE_SIZE")), "WRITE_SIZE",
                          part)
        if not f or not w:
            continue
        fk, wk = sum(f) / len(f), sum(w) / len(w)
        rec["kernels"][key] = {
            "bytes_per_launch": int(round((fk * scale["FETCH_SIZE"] + wk * scale["WRITE_SIZE"]) * 1024)),
            "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
            "dispatches": len(f), "fetch_scale": round(scale["FETCH_SIZE"], 4),
            "write_scale": round(scale["WRITE_SIZE"], 4), "workload": wl,
            "source_sha256": _sha(src)}
        print(f"{key} ({wl}): {rec['kernels'][key]['bytes_per_launch'] / 1e9:.4f} GB per launch "
              f"(FETCH {fk:.1f} KiB, WRITE {wk:.1f} KiB, {len(f)} dispatches)")
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(f"copy scale: FETCH {scale['FETCH_SIZE']:.4f}, WRITE {scale['WRITE_SIZE']:.4f}")


def counter_table(d):
    """Per-kernel averages of every counter in the rocprofv3 counter runs
    under d (rows already summed over the counter's instances), with the
    kernel duration and, where GRBM_GUI_ACTIVE and SQ_VALU_MFMA_BUSY_CYCLES
    were collected, the shader clock (GRBM_GUI_ACTIVE summed over the 8 XCDs,
    / 8, over the duration) and the MFMA utilisation (busy cycles summed over
    the 1,024 SIMDs over 1,024 x the per-XCD active cycles)."""
    from collections import defaultdict
    rows = _read_counter_csv(d)
    vals = defaultdict(lambda: defaultdict(float))
    dur, name = {}, {}
    for r in rows:
        key = (f'{r.get("Kernel_Name", "")[:60]} grid={r.get("Grid_Size", "?")}', r["Dispatch_Id"])
        vals[key][r["Counter_Name"]] += float(r["Counter_Value"])
        dur[key] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    by_kernel = defaultdict(list)
    for (k, disp), c in vals.items():
        by_kernel[k].append((dur[(k, disp)], c))
    for k, lst in sorted(by_kernel.items()):
        if max(x[0] for x in lst) < 20_000:   # skip launches under 20 us
            continue
        ns = sum(x[0] for x in lst) / len(lst)
        avg = defaultdict(float)
        for _, c in lst:
            for cn, v in c.items():
                avg[cn] += v / len(lst)
        line = f"{k} n={len(lst)} avg_ms={ns / 1e6:.3f}"
        for cn in sorted(avg):
            line += f" {cn}={avg[cn]:.5g}"
        if "GRBM_GUI_ACTIVE" in avg and ns >= 1e6:   # clocks only for launches of 1 ms or more
            per_xcd = avg["GRBM_GUI_ACTIVE"] / 8.0
            line += f" clock_GHz={per_xcd / ns:.3f}"
            if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
                line += f" mfma_util={avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (per_xcd * 1024):.3f}"
        print(line)


# --------------------------------------------------------------------------

def main():
    args = _args()
    if args.record_traffic:
        record_traffic(args.record_traffic)
        return
    if args.counter_table:
        counter_table(args.counter_table)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: libkld scores on one GPU; --gpus must be 1 (sharding positions over "
              "several GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.read_calibration:
        read_calibration()
        return
    if args.gemm_calibration:
        gemm_calibration()
        return
    import full_vocab_kl_amd as kld
    kld.lib()   # fails loudly if libkld.so is missing

    cpu = CPU_SAMPLE[args.workload][0] if args.cpu_sample is None else args.cpu_sample
    res = FUNCS[args.workload](args.steps, args.warmup, cpu)

    line = {"metric": METRIC, "value": round(res["value"], 1), "unit": res["unit"], "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": res["dtype"],
            "data": "synthetic", "config": res["config"], "roofline": res["roofline"]}
    for k in ("parity", "cpu_baseline", "result", "export_ms", "paired_ms", "target_ms",
              "target_ms_per_stream", "target_positions_per_s"):
        if k in res:
            line[k] = res[k]
    if args.workload == "fused_window" and not args.no_secondary:
        line["secondary"] = []
        for name in ("logits_f32", "bf16_topk_stream", "fused_batch", "long_trace", "golden_f32",
                     "windows_paired", "coarse_fused_window"):
            cs = CPU_SAMPLE[name][1] if args.cpu_sample is None else min(args.cpu_sample,
                                                                         CPU_SAMPLE[name][1])
            steps = SECONDARY_STEPS.get(name, max(5, args.steps))
            print(f"bench: secondary {name}", file=sys.stderr, flush=True)
            sec = FUNCS[name](steps, min(args.warmup, 2), cs)
            entry = {"workload": sec["config"]["workload"], "value": round(sec["value"], 1),
                     "unit": sec["unit"], "ms_per_step": round(sec["ms_per_step"], 4),
                     "steps": steps, "roofline": sec["roofline"]}
            for k in ("parity", "cpu_baseline", "export_ms", "paired_ms", "target_ms",
                      "target_ms_per_stream", "target_positions_per_s"):
                if k in sec:
                    entry[k] = sec[k]
            line["secondary"].append(entry)
            torch.cuda.empty_cache()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
