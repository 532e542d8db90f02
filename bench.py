#!/usr/bin/env python3
"""One-GPU benchmark of the LSTM/GRU layer engine.

A step is one pass of the whole layer on one batch of seeded synthetic input
already resident in HBM: rnn_fwd (input projection + persistent forward),
rnn_bwd_data (persistent BPTT + dx) and rnn_bwd_weights (dW, db). The default
workload is the single-layer bf16 LSTM at T=256, B=64, I=H=1024.

Prints one JSON line: the throughput in timestep*batch/s, the algorithmic
TFLOP/s, a roofline entry for the kernel that takes the most time per step
(timed live with HIP events on the library's stream through the
rnn_profile_* hook, in a second pass over the same K steps so that the
event records stay out of the throughput), and the CPU oracle timed on a
bounded sample of the same workload on the host cores.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

# dense MFMA ceilings on MI355X for the arithmetic each storage type runs on:
# bf16 products at the published 2.5 PFLOP/s; fp32 products run as six
# bf16 MFMAs on exact three-piece splits of their operands, so their ceiling
# is the bf16 peak over six (the published fp32 matrix peak, 157.3 TFLOP/s,
# is what the fp32 MFMA instructions would give and lies below it)
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 2500.0 / 6}
PEAK_HBM_GBS = 8000.0


def _layer_work(wl, li):
    """(flops, bytes) per label for one layer and direction (one launch
    group), from the algorithmic counts: every GEMM-shaped product
    2*M*N*K; bytes = the tensors each step must read and write once."""
    from gru_layer_fwd_amd.synth import n_gates
    G = n_gates(wl.mode)
    dirs = 2 if wl.bidir else 1
    I = wl.I if li == 0 else wl.H * dirs
    T, B, H = wl.T, wl.B, wl.H
    s = 2 if wl.dtype == "bf16" else 4
    TB = T * B
    GZ = 4 if (wl.mode == "gru" and wl.reset_after) else G
    cst = H if wl.mode == "lstm" else 0
    return {
        "proj_gemm": (2.0 * TB * G * H * I, s * (TB * I + G * H * I + TB * G * H)),
        # persistent forward: read P, write y, gates (+c); W_hh stays resident
        "rec_fwd": (2.0 * TB * G * H * H, s * TB * (G * H + H + GZ * H + cst)),
        # persistent BPTT: read dy, gates (+c twice, y), write dG
        "rec_bwd": (2.0 * TB * G * H * H, s * TB * (H + GZ * H + 2 * cst + H + G * H)),
        "dx_gemm": (2.0 * TB * G * H * I, s * (TB * G * H + G * H * I + TB * I)),
        "dw_gemm": (2.0 * TB * G * H * (I + H), s * (2 * TB * G * H + TB * (I + H) + G * H * (I + H))),
        "db_colsum": (2.0 * TB * G * H, s * 2 * TB * G * H),
    }


def _work(wl):
    tot = {}
    dirs = 2 if wl.bidir else 1
    for li in range(wl.layers):
        for _ in range(dirs):
            for k, (f, b) in _layer_work(wl, li).items():
                f0, b0 = tot.get(k, (0.0, 0.0))
                tot[k] = (f0 + f, b0 + b)
    return tot


KERNEL_SOURCES = ("gru_layer_fwd_amd/csrc/recurrent.hip", "gru_layer_fwd_amd/csrc/gemm.hip",
                  "gru_layer_fwd_amd/csrc/rnn_internal.hpp")


def kernel_hash() -> str:
    """Hash of the kernel sources, so that stored counter readings are only
    used for the kernels they were taken on."""
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for f in KERNEL_SOURCES:
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, label: str):
    """HBM bytes per launch of `label` from profiles/traffic.json (two
    rocprofv3 --pmc passes, FETCH_SIZE and WRITE_SIZE, scaled by a copy
    kernel of known size), or None when absent or taken on other kernels."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic.json")
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    e = t.get(workload, {}).get(label)
    if not e or e.get("kernel_hash") != kernel_hash():
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(wl, inp, rows: int):
    """The oracle as it stands, on the first `rows` batch rows of the same
    workload (all T steps, every layer/direction), timed on the host."""
    import numpy as np

    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    sub = lambda a: None if a is None else a[:rows]  # noqa: E731
    x = inp["x"][:, :rows]
    g = inp["g"][:, :rows]
    order = wl.gate_order()
    t0 = time.perf_counter()
    if wl.layers == 1 and not wl.bidir:
        p = inp["params"][0][0]
        fw = O.layer_forward(wl.mode, x, sub(inp["h0"]), sub(inp["c0"]), p, order, False, wl.reset_after)
        O.layer_backward(wl.mode, fw, g)
    else:
        recs, _ = O.stack_forward(wl.mode, x, inp["params"], order, wl.bidir, wl.reset_after)
        O.stack_backward(wl.mode, recs, g)
    dt = time.perf_counter() - t0
    units = wl.T * rows
    return {"value": units / dt, "unit": "timestep*batch/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 numpy oracle (library matmul, BLAS threads = cores), fwd+bwd_data+bwd_weights "
                      f"over all T={wl.T} steps on {rows} of {wl.B} batch rows ({dt:.2f} s)",
            "seconds": dt, "np": np.__version__, "host": host_cpu()}


def host_cpu():
    """CPU model, logical CPUs of the host and those this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--cpu-rows", type=int, default=0, help="batch rows the CPU oracle runs (0 = all)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--ragged", action="store_true",
                    help="single-layer workloads: per-row sequence lengths drawn uniformly from [1, T] "
                         "(the timed work still covers all T steps; value counts T*B)")
    ap.add_argument("--recompute", action="store_true",
                    help="LSTM workloads: keep only the gates between forward and backward and rebuild the "
                         "cell states in the backward call")
    ap.add_argument("--att", action="store_true",
                    help="GRU workloads: AUGRU attention scores drawn uniformly from [0, 1], and their gradient")
    ap.add_argument("--separate-dw", action="store_true",
                    help="single-layer workloads: dW_hh from the separate product even where the BPTT kernel "
                         "could accumulate it (dw_hh_mode 1)")
    ap.add_argument("--stepwise", action="store_true",
                    help="single-layer workloads: the per-step recurrence instead of the persistent kernels")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed region, run one plain device copy of this many MiB (a known-size "
                         "kernel for calibrating rocprofv3 FETCH_SIZE/WRITE_SIZE readings)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the layer shards over "
              "batch rows with one dW all-reduce, which is not built here)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from gru_layer_fwd_amd import _lib as L
    from gru_layer_fwd_amd import synth
    from gru_layer_fwd_amd.api import RnnLayer, RnnStack

    name = args.workload or synth.HEADLINE
    wl = synth.WORKLOADS[name]
    inp = synth.make_inputs(wl)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[wl.dtype]
    dev = lambda a: None if a is None else torch.from_numpy(a).to("cuda", dt)  # noqa: E731
    x = dev(inp["x"])
    g = dev(inp["g"])
    # per layer, each parameter of all directions in one [dirs, ...] tensor;
    # params[l][d] are views of it (a bidirectional layer reads both at once)
    def stacked(per):
        ts = [torch.stack([dev(getattr(p, k)) for p in per]) for k in ("W_ih", "W_hh", "b_ih", "b_hh")]
        return [tuple(t[d] for t in ts) for d in range(len(per))]

    params = [stacked(per) for per in inp["params"]]
    grads = []
    for per in params:
        gts = [torch.empty((len(per),) + tuple(t.shape), dtype=t.dtype, device=t.device) for t in per[0]]
        grads.append([tuple(t[d] for t in gts) for d in range(len(per))])
    order = wl.gate_order()

    if (args.ragged or args.att or args.recompute or args.separate_dw or args.stepwise) and (wl.layers != 1 or wl.bidir):
        raise SystemExit("--ragged / --att / --recompute / --separate-dw / --stepwise apply to single-layer workloads")
    if args.recompute and wl.mode != "lstm":
        raise SystemExit("--recompute applies to LSTM workloads")
    if args.att and wl.mode != "gru":
        raise SystemExit("--att applies to GRU workloads")
    extra_rng = np.random.Generator(np.random.PCG64(wl.seed + 500))
    lengths = att = datt = None
    if args.ragged:
        lengths = torch.from_numpy(extra_rng.integers(1, wl.T + 1, size=wl.B).astype(np.int32)).to("cuda")
    if args.att:
        att = dev(synth.round_to(extra_rng.uniform(0.0, 1.0, (wl.T, wl.B)), wl.dtype))
        datt = torch.empty_like(att)

    if wl.layers == 1 and not wl.bidir:
        lay = RnnLayer(wl.mode, wl.T, wl.B, wl.I, wl.H, wl.dtype, reset_after=wl.reset_after, gate_order=order,
                       lengths=lengths, att=att, recompute=args.recompute, dw_hh_mode=int(args.separate_dw),
                       stepwise=args.stepwise)
        h0, c0 = dev(inp["h0"]), dev(inp["c0"])
        y = torch.empty(wl.T, wl.B, wl.H, dtype=dt, device="cuda")
        hT = torch.empty(wl.B, wl.H, dtype=dt, device="cuda")
        cT = torch.empty_like(hT) if wl.mode == "lstm" else None
        dx = torch.empty_like(x)
        dh0 = torch.empty_like(hT)
        dc0 = torch.empty_like(hT) if wl.mode == "lstm" else None
        W_ih, W_hh, b_ih, b_hh = params[0][0]

        def step():
            lay.fwd(x, h0, c0, W_ih, W_hh, b_ih, b_hh, y, hT, cT)
            lay.bwd_data(W_ih, W_hh, h0, c0, y, g, None, None, dx, dh0, dc0, datt=datt)
            lay.bwd_weights(x, h0, y, *grads[0][0])

        status = lambda: lay.device_status()  # noqa: E731
    else:
        st = RnnStack(wl.mode, wl.T, wl.B, wl.I, wl.H, wl.dtype, wl.layers, wl.bidir, wl.reset_after, order)
        dx = torch.empty_like(x)

        def step():
            st.fwd(x, params)
            st.bwd(x, params, g, dx, grads)

        status = lambda: max((lay.device_status() for lay in st.layers), key=abs)  # noqa: E731

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if status() != 0:
        raise SystemExit(f"device status {status()} after warm-up")
    # The K steps are timed twice: once as they run (the throughput), then
    # once more with a HIP event pair around every library step on its
    # stream (per-kernel durations, the roofline). The event records cost
    # about 60 us per layer step at the headline shape, so they stay out of
    # the throughput figure.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if status() != 0:
        raise SystemExit(f"device status {status()} in the timed region")
    L.rnn_profile_read(reset=True)
    L.rnn_profile_enable(True)
    torch.cuda.synchronize()
    tp0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    tp1 = time.perf_counter()
    L.rnn_profile_enable(False)
    prof = L.rnn_profile_read(reset=True)
    if status() != 0:
        raise SystemExit(f"device status {status()} in the timed region")

    ms = (t1 - t0) * 1e3 / args.steps
    ms_timed = (tp1 - tp0) * 1e3 / args.steps
    units = wl.T * wl.B
    value = units / (ms / 1e3)
    tflops = wl.flops_gemm() / (ms / 1e3) / 1e12
    work = _work(wl)
    kern = {k: {"ms_per_step": v[1] / args.steps, "launches_per_step": v[0] / args.steps} for k, v in prof.items()}
    # dominant kernel = most time per step; its roofline from the algorithmic work
    dom = max((k for k in kern if k in work), key=lambda k: kern[k]["ms_per_step"])
    f_step, b_step = work[dom]
    t_step = kern[dom]["ms_per_step"] / 1e3
    t_mfma = f_step / (PEAK_TFLOPS[wl.dtype] * 1e12)
    t_hbm = b_step / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": f_step / t_step / 1e12, "peak": PEAK_TFLOPS[wl.dtype],
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": b_step / t_step / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = stored_traffic(name, dom)
    roof["kernel"] = dom
    roof["launch_ms"] = kern[dom]["ms_per_step"] / max(kern[dom]["launches_per_step"], 1)
    for k in kern:
        if k in work:
            f, b = work[k]
            tk = kern[k]["ms_per_step"] / 1e3
            kern[k]["tflops"] = f / tk / 1e12 if tk > 0 else None
            kern[k]["mfma_frac"] = (f / tk / 1e12) / PEAK_TFLOPS[wl.dtype] if tk > 0 else None
    rec = {}
    dirs = (2 if wl.bidir else 1) * wl.layers
    for k in ("rec_fwd", "rec_bwd"):
        if k in kern:
            rec[k] = kern[k]["ms_per_step"] * 1e3 / (wl.T * dirs)

    out = {
        "metric": "LSTM/GRU fwd+bwd timestep*batch/s and TFLOP/s at H=1024 B=64 T=256",
        "value": value,
        "unit": "timestep*batch/s",
        "tflops": tflops,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": name, "cell": wl.mode + ("" if wl.mode == "lstm" else
                                                       ("_reset_after" if wl.reset_after else "_basic")),
                   "T": wl.T, "B": wl.B, "I": wl.I, "H": wl.H, "layers": wl.layers,
                   "bidirectional": wl.bidir, "storage": wl.dtype, "accumulate": "f32",
                   **({"lengths": "uniform [1, T] per row"} if args.ragged else {}),
                   **({"augru_scores": "uniform [0, 1]"} if args.att else {}),
                   **({"cell_states": "recomputed in the backward call"} if args.recompute else {}),
                   **({"dw_hh": "separate product"} if args.separate_dw else {}),
                   **({"recurrence": "per-step kernels"} if args.stepwise else {})},
        "roofline": roof,
        "recurrent_us_per_step": rec,
        "kernels": kern,
        "kernels_pass_ms_per_step": ms_timed,
    }
    # the exchange alone on the persistent kernels' own grids: the floor the
    # step handshake puts under a step (rnn_handshake_probe)
    floor = {}
    probe_lay = lay if (wl.layers == 1 and not wl.bidir) else st.layers[0]
    cs = torch.cuda.current_stream()
    for pass_, label in ((0, "rec_fwd"), (1, "rec_bwd")):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record(cs)
        rc = 0
        for _ in range(reps):
            rc = L.rnn_handshake_probe(probe_lay.desc, pass_, probe_lay.workspace.data_ptr(), probe_lay.ws_bytes,
                                       cs.cuda_stream)
            if rc != 0:
                break
        e1.record(cs)
        torch.cuda.synchronize()
        if rc == 0 and probe_lay.device_status() == 0:
            floor[label] = e0.elapsed_time(e1) * 1e3 / (reps * wl.T)
    out["handshake_floor_us_per_step"] = floor or None
    if args.copy_mib:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_probe_bytes"] = 2 * (args.copy_mib << 20)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, inp, min(args.cpu_rows or wl.B, wl.B))
    print(json.dumps(out), flush=True)
    # explicit teardown before the interpreter exits: every queued kernel
    # done, the library's profiling events released (profiling is off and
    # read), torch's cached device memory returned
    torch.cuda.synchronize()
    del step
    torch.cuda.empty_cache()
    torch.cuda.synchronize()


if __name__ == "__main__":
    main()
