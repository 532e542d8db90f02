"""Where a persistent step's time goes: per-phase table from the debug build.

    python -m gru_layer_fwd_amd.step_timers [--workload NAME] [--out FILE]

Loads librnn_timers.so (built with RNN_STEP_TIMERS, see include/rnn_debug.h)
instead of librnn.so, runs the layer of the workload (seeded synthetic
inputs), and after one forward and one backward-data call reads the
timestamps thread 0 of every workgroup wrote at eight points of every step.
Reported per pass, in ns, averaged over the workgroups and the steps away
from both ends of the sequence:

    wait      step start -> the step counters of wave 0's producers seen
    contract  -> the contraction's loads and MFMAs issued
    spill     -> partial sums written to LDS (the MFMA results are in)
    barrier   -> past the workgroup barrier
    epilogue  -> gate arithmetic done, exchange stores issued
    publish   -> stores acknowledged, barrier, step counter written
    stores    -> stores for later kernels issued
    loop      -> next step's start

plus the whole step, the time from kernel start to the first step, the
first step, and the exchange-only probe (rnn_handshake_probe) on the same
grid: the floor the step exchange puts under a step.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys

import numpy as np

PHASES = ("wait", "contract", "spill", "barrier", "epilogue", "publish", "stores", "loop")
# basic GRU: two exchanges per step (A: r, u from h_{t-1}; B: the candidate
# from r*h_{t-1}; backward: A the carried gradient, B the one through r*h)
PHASES_GRUB = ("waitA", "contractA", "epilogueA", "publishA", "waitB", "contractB", "epilogueB", "publishB")


def _timers(lib):
    w, s, p = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    assert lib.rnn_step_timers_shape(ctypes.byref(w), ctypes.byref(s), ctypes.byref(p)) == 0
    t = np.zeros(w.value * s.value * p.value, dtype=np.uint64)
    c = np.zeros(w.value * 4, dtype=np.uint64)
    st = lib.rnn_step_timers_read(t.ctypes.data_as(ctypes.c_void_p), c.ctypes.data_as(ctypes.c_void_p))
    assert st == 0, st
    # the kernels keep the low 32 bits of the clock per step: unwrap them;
    # points a step does not pass (zero: e.g. the wait of the backward's
    # first step) take the previous point's time first
    t = t.reshape(w.value, s.value, p.value).astype(np.int64)
    flat = t.reshape(w.value, -1)
    idx = np.where(flat != 0, np.arange(flat.shape[1])[None, :], 0)
    np.maximum.accumulate(idx, axis=1, out=idx)
    flat = np.take_along_axis(flat, idx, axis=1)
    d = np.diff(flat, axis=1)
    d[d < -(1 << 31)] += 1 << 32
    flat[:, 1:] = flat[:, :1] + np.cumsum(d, axis=1)
    return flat.reshape(t.shape), c.reshape(w.value, 4).astype(np.int64)


def analyse(t, cal, nblocks, nsteps, skip=8, phases=PHASES):
    """Per-phase means (ns) over the blocks among [0, nblocks) that ran (nonzero
    calibration pairs) and steps [skip, nsteps - skip)."""
    nblocks = min(nblocks, t.shape[0])
    nsteps = min(nsteps, t.shape[1])
    skip = min(skip, max(1, nsteps // 4))  # short sequences: fewer steps left out at the ends
    ran = np.nonzero(cal[:nblocks, 0] != 0)[0]
    t, cal = t[ran, :nsteps], cal[ran]
    nwg = len(ran)
    # s_memtime ticks per ns from each workgroup's start/end pairs (s_memrealtime: 100 MHz)
    ticks_per_ns = float(np.median((cal[:, 2] - cal[:, 0]) / ((cal[:, 3] - cal[:, 1]) * 10.0)))
    lo, hi = skip, max(skip + 1, nsteps - skip)
    seg = t[:, lo:hi + 1]
    out = {}
    for p in range(7):
        out[phases[p]] = float(np.mean(seg[:, :-1, p + 1] - seg[:, :-1, p])) / ticks_per_ns
    out[phases[7]] = float(np.mean(seg[:, 1:, 0] - seg[:, :-1, 7])) / ticks_per_ns
    out["step"] = float(np.mean(seg[:, 1:, 0] - seg[:, :-1, 0])) / ticks_per_ns
    out["startup"] = float(np.mean((t[:, 0, 0] - (cal[:, 0] & 0xFFFFFFFF)) % (1 << 32))) / ticks_per_ns
    out["first_step"] = float(np.mean(t[:, 1, 0] - t[:, 0, 0])) / ticks_per_ns
    out["clock_ghz"] = ticks_per_ns
    out["steps_averaged"] = int(hi - lo)
    out["steps_skipped"] = int(skip)
    out["workgroups"] = int(nwg)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--out", default=None, help="write the markdown table here as well")
    ap.add_argument("--json", default=None, help="write the numbers as JSON here")
    ap.add_argument("--separate-dw", action="store_true",
                    help="dW_hh from the separate product (dw_hh_mode 1), not accumulated in the BPTT kernel")
    args = ap.parse_args()

    # torch first: the library then binds to the HIP runtime torch has loaded
    import torch

    from . import _lib as L
    from . import synth
    L.select(os.path.join(os.path.dirname(os.path.abspath(__file__)), "librnn_timers.so"))
    lib = L.lib()
    for name in ("rnn_step_timers_shape", "rnn_step_timers_read", "rnn_step_timers_reset"):
        getattr(lib, name).restype = ctypes.c_int

    from .api import RnnLayer
    name = args.workload or synth.HEADLINE
    wl = synth.WORKLOADS[name]
    if wl.layers != 1 or wl.bidir:
        raise SystemExit("single-layer workloads only")
    inp = synth.make_inputs(wl)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[wl.dtype]
    dev = lambda a: None if a is None else torch.from_numpy(a).to("cuda", dt)  # noqa: E731
    p = inp["params"][0][0]
    W = [dev(getattr(p, k)) for k in ("W_ih", "W_hh", "b_ih", "b_hh")]
    x, g, h0, c0 = dev(inp["x"]), dev(inp["g"]), dev(inp["h0"]), dev(inp["c0"])
    lay = RnnLayer(wl.mode, wl.T, wl.B, wl.I, wl.H, wl.dtype, reset_after=wl.reset_after,
                   gate_order=wl.gate_order(), dw_hh_mode=int(args.separate_dw))
    y = torch.empty(wl.T, wl.B, wl.H, dtype=dt, device="cuda")
    dx = torch.empty_like(x)
    grads = [torch.empty_like(w) for w in W]
    for _ in range(2):
        lay.fwd(x, h0, c0, *W, y)
        lay.bwd_data(W[0], W[1], h0, c0, y, g, None, None, dx)
        lay.bwd_weights(x, h0, y, *grads)
    torch.cuda.synchronize()
    res = {"workload": name, "dw_hh_mode": int(args.separate_dw)}
    phases = PHASES_GRUB if (wl.mode == "gru" and not wl.reset_after) else PHASES
    for pass_, label in ((0, "forward"), (1, "backward")):
        torch.cuda.synchronize()
        assert lib.rnn_step_timers_reset() == 0
        if pass_ == 0:
            lay.fwd(x, h0, c0, *W, y)
        else:
            lay.bwd_data(W[0], W[1], h0, c0, y, g, None, None, dx)
        torch.cuda.synchronize()
        assert lay.device_status() == 0
        st, plan = L.rnn_plan_query(lay.desc, pass_)
        assert st == 0
        t, cal = _timers(lib)
        res[label] = analyse(t, cal, plan.blocks, wl.T + pass_, phases=phases)
        res[label]["plan"] = {k: getattr(plan, k) for k, _ in plan._fields_}
        # the exchange alone on the same grid
        s = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record(s)
        for _ in range(reps):
            st = L.rnn_handshake_probe(lay.desc, pass_, lay.workspace.data_ptr(), lay.ws_bytes, s.cuda_stream)
            if st != 0:
                break
        e1.record(s)
        torch.cuda.synchronize()
        if st == 0 and lay.device_status() == 0:
            res[label]["exchange_only_us_per_step"] = e0.elapsed_time(e1) * 1e3 / (reps * wl.T)
    lines = [f"Per-step phases of the persistent kernels, {name}"
             + (", dW_hh by the separate product" if args.separate_dw else "")
             + " (debug build with step timers; ns, mean over workgroups and over the steps away from both"
             " ends of the sequence)", "",
             "| pass | " + " | ".join(phases) + " | step | first step | start-up | exchange only |",
             "|---" * (len(phases) + 5) + "|"]
    for label in ("forward", "backward"):
        r = res[label]
        ex = r.get("exchange_only_us_per_step")
        lines.append(f"| {label} | " + " | ".join(f"{r[k]:.0f}" for k in phases)
                     + f" | {r['step']:.0f} | {r['first_step']:.0f} | {r['startup']:.0f} | "
                     + (f"{ex * 1e3:.0f}" if ex is not None else "-") + " |")
    lines += ["", "Produced by (from the repository root, library built with `python -m gru_layer_fwd_amd.build`):",
              "", "```", "python -m gru_layer_fwd_amd.step_timers " + " ".join(sys.argv[1:]), "```"]
    text = "\n".join(lines)
    print(text, flush=True)
    print(json.dumps(res), flush=True)
    if args.out:
        with open(args.out, "w") as fh:
            fh.write(text + "\n")
    if args.json:
        with open(args.json, "w") as fh:
            json.dump(res, fh, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
