"""Shared pieces of the GPU parity tests: run one layer through the C ABI and
through the oracle on the same seeded inputs, and compare.

Tolerances (per tensor, max_i |gpu_i - ref_i| / max_i |ref_i|): 1e-4 for the
fp32 forward outputs, 1e-3 for fp32 gradients, 2e-2 for bf16 storage with
fp32 accumulation.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from gru_layer_fwd_amd.api import RnnLayer, RnnStack

TOL = {("f32", "fwd"): 1e-4, ("f32", "grad"): 1e-3, ("bf16", "fwd"): 2e-2, ("bf16", "grad"): 2e-2}
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


def dev(a, dtype, device="cuda"):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=TDT[dtype])


def host(t):
    return None if t is None else t.detach().to(torch.float64).cpu().numpy()


def gpu_layer(mode, dtype, params, x, h0, c0, dy, dhT=None, dcT=None, direction=0, reset_after=True,
              order=None, xpad=0, ypad=0, want_dx=True, acc=False, repeat=1, lengths=None, att=None,
              recompute=False, dw_hh_mode=0, stepwise=False):
    """Forward, backward-data and backward-weights of one layer on the GPU.
    xpad/ypad > 0 store x/dx and y/dy with a larger row stride; lengths is
    an optional host array of B per-row step counts, att optional [T, B]
    AUGRU attention scores (GRU)."""
    T, B, I = x.shape
    H = params.W_hh.shape[1]
    ldx, ldy = I + xpad, H + ypad
    lens = None if lengths is None else torch.as_tensor(np.asarray(lengths), dtype=torch.int32).to("cuda")
    dt = TDT[dtype]
    attd = None if att is None else dev(att, dtype)
    lay = RnnLayer(mode, T, B, I, H, dtype, direction=direction, reset_after=reset_after,
                   gate_order=order, ldx=ldx, ldy=ldy, lengths=lens, att=attd, recompute=recompute,
                   dw_hh_mode=dw_hh_mode, stepwise=stepwise)
    datt = None if att is None else torch.zeros(T, B, dtype=dt, device="cuda")
    xs = torch.zeros(T, B, ldx, dtype=dt, device="cuda")
    xs[:, :, :I] = dev(x, dtype)
    ys = torch.full((T, B, ldy), float("nan"), dtype=dt, device="cuda")
    dys = torch.zeros(T, B, ldy, dtype=dt, device="cuda")
    dys[:, :, :H] = dev(dy, dtype)
    W_ih, W_hh, b_ih, b_hh = (dev(a, dtype) for a in (params.W_ih, params.W_hh, params.b_ih, params.b_hh))
    h0d, c0d = dev(h0, dtype), dev(c0, dtype) if mode == "lstm" else None
    dhTd, dcTd = dev(dhT, dtype), dev(dcT, dtype) if mode == "lstm" else None
    hT = torch.empty(B, H, dtype=dt, device="cuda")
    cT = torch.empty(B, H, dtype=dt, device="cuda") if mode == "lstm" else None
    dxs = torch.zeros(T, B, ldx, dtype=dt, device="cuda") if want_dx else None
    dh0 = torch.empty(B, H, dtype=dt, device="cuda")
    dc0 = torch.empty(B, H, dtype=dt, device="cuda") if mode == "lstm" else None
    G = W_hh.shape[0]
    dW_ih = torch.zeros(G, I, dtype=dt, device="cuda")
    dW_hh = torch.zeros(G, H, dtype=dt, device="cuda")
    db_ih = torch.zeros(G, dtype=dt, device="cuda")
    db_hh = torch.zeros(G, dtype=dt, device="cuda")
    out = []
    for _ in range(repeat):
        lay.fwd(xs, h0d, c0d, W_ih, W_hh, b_ih, b_hh, ys, hT, cT)
        lay.bwd_data(W_ih, W_hh, h0d, c0d, ys, dys, dhTd, dcTd, dxs, dh0, dc0, accumulate=acc, datt=datt)
        lay.bwd_weights(xs, h0d, ys, dW_ih, dW_hh, db_ih, db_hh, accumulate=acc)
        torch.cuda.synchronize()
        st = lay.device_status()
        assert st == 0, f"device status {st}"
        r = dict(y=host(ys[:, :, :H]), hT=host(hT), dh0=host(dh0), dW_ih=host(dW_ih), dW_hh=host(dW_hh),
                 db_ih=host(db_ih), db_hh=host(db_hh), ypad=host(ys[:, :, H:]))
        if want_dx:
            r["dx"] = host(dxs[:, :, :I])
            r["dxpad"] = host(dxs[:, :, I:])
        if mode == "lstm":
            r["cT"], r["dc0"] = host(cT), host(dc0)
        if datt is not None:
            r["datt"] = host(datt)
        out.append(r)
    return out if repeat > 1 else out[0]


def oracle_layer(mode, params, x, h0, c0, dy, dhT=None, dcT=None, direction=0, reset_after=True, order=None,
                 lengths=None, att=None):
    if order is None:
        order = (0, 1, 2, 3) if mode == "lstm" else (0, 1, 2)
    fw = O.layer_forward(mode, x, h0, c0, params, order, reverse=bool(direction), reset_after=reset_after,
                         lengths=lengths, att=att)
    gr = O.layer_backward(mode, fw, dy, dhT, dcT)
    r = dict(y=fw["y"], hT=fw["hT"], dx=gr["dx"], dh0=gr["dh0"], dW_ih=gr["dW_ih"], dW_hh=gr["dW_hh"],
             db_ih=gr["db_ih"], db_hh=gr["db_hh"])
    if mode == "lstm":
        r["cT"], r["dc0"] = fw["cT"], gr["dc0"]
    if "datt" in gr:
        r["datt"] = gr["datt"]
    return r


FWD_KEYS = ("y", "hT", "cT")
GRAD_KEYS = ("dx", "dh0", "dc0", "dW_ih", "dW_hh", "db_ih", "db_hh", "datt")


def compare(got, ref, dtype, keys=None, rows=None, extra=""):
    """Assert every tensor within tolerance; returns the error table."""
    errs = {}
    for k in (keys or FWD_KEYS + GRAD_KEYS):
        if k not in ref or k not in got:
            continue
        g, r = got[k], ref[k]
        if rows is not None and k in ("y", "dx", "datt"):
            g = g[:, rows]
        elif rows is not None and k in ("hT", "cT", "dh0", "dc0"):
            g = g[rows]
        e = O.rel_err(g, r)
        errs[k] = e
    bad = {k: e for k, e in errs.items()
           if not (e <= TOL[(dtype, "fwd" if k in FWD_KEYS else "grad")])}
    assert not bad, f"{extra} out of tolerance: {bad} (all: {errs})"
    return errs


class Params:
    def __init__(self, W_ih, W_hh, b_ih, b_hh):
        self.W_ih, self.W_hh, self.b_ih, self.b_hh = W_ih, W_hh, b_ih, b_hh

    def rows_of(self):
        return self


def sub_params(p):
    return Params(p.W_ih, p.W_hh, p.b_ih, p.b_hh)


__all__ = ["gpu_layer", "oracle_layer", "compare", "dev", "host", "Params", "RnnStack", "TOL"]
