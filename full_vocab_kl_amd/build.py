"""Build libkld.so in-tree with hipcc for gfx950.

    python -m full_vocab_kl_amd.build

Every source under csrc/ is compiled to an object (in parallel), then linked
into full_vocab_kl_amd/libkld.so.  Packed-fp32 VALU forms are disabled for
all device code."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkld.so")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-ffp-contract=off",  # every fused multiply-add is written out explicitly (fmaf / fma)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libkld")
    return h


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def build(verbose: bool = False, extra_flags=()) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        cmd = [hipcc, *CFLAGS, *extra_flags, "-c", src, "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                         if "packed-fp32-ops" not in l and l.strip())
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
        if verbose and msgs:
            print(msgs, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
