"""Build librnn.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m gru_layer_fwd_amd.build [--jobs N] [--only main|timers]

Each source is compiled to an object in _build/ (in parallel), then linked
into gru_layer_fwd_amd/librnn.so. The same sources are also built with
RNN_STEP_TIMERS into librnn_timers.so, the debug build whose persistent
kernels record per-step timestamps (include/rnn_debug.h); nothing but the
step-timer tool loads it. Always rebuilds.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "librnn.so")
OUT_TIMERS = os.path.join(PKG, "librnn_timers.so")
BUILD = os.path.join(ROOT, "_build")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Wno-unused-command-line-argument",
    # packed fp32 VALU forms stay off (the compiler would otherwise form them
    # from plain float code)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def hipcc():
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return p


def _compile(src: str, variant: str = "main") -> str:
    obj = os.path.join(BUILD, variant, os.path.basename(src) + ".o")
    extra = ["-DRNN_STEP_TIMERS"] if variant == "timers" else []
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc()] + COMMON + extra + lang + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs: int | None = None, verbose: bool = False, only: str | None = None) -> str:
    variants = [v for v in ("main", "timers") if only in (None, v)]
    for v in variants:
        os.makedirs(os.path.join(BUILD, v), exist_ok=True)
    srcs = sources()
    work = [(s, v) for v in variants for s in srcs]
    jobs = jobs or min(len(work), os.cpu_count() or 4, 16)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda sv: _compile(*sv), work))
    for v in variants:
        out = OUT if v == "main" else OUT_TIMERS
        _link([o for o, (_, vv) in zip(objs, work) if vv == v], out)
        if verbose:
            print(f"built {out}")
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--only", choices=("main", "timers"), default=None)
    args = ap.parse_args()
    try:
        build(args.jobs, verbose=True, only=args.only)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
