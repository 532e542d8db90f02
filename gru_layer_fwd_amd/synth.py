"""Seeded synthetic inputs for the LSTM/GRU layer engine.

This module holds no arithmetic of the recurrent method itself: it only draws
random numbers in a fixed order, rounds them to the storage type, and names the
workloads. Both the HIP path (through the binding) and the CPU oracle consume
exactly the arrays produced here.

Workloads follow the shapes and distributions the layer API implies for
single-layer and stacked bidirectional LSTM/GRU layers (time-major [T, B, I]
sequences, [G*H, I] input weights and [G*H, H] recurrent weights grouped by
gate, as in the popnn Lstm.cpp/Gru.cpp pages, "createWeightsKernel").

Draw order per layer and direction: W_ih, W_hh, b_ih, b_hh, then (first layer
only) x, h0, c0, and last the upstream gradient g used as dy.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

LSTM, GRU = "lstm", "gru"
F32, BF16 = "f32", "bf16"

# gate ids (named, independent of storage order)
LSTM_I, LSTM_F, LSTM_G, LSTM_O = 0, 1, 2, 3
GRU_R, GRU_U, GRU_C = 0, 1, 2

ORDER_IFGO = (LSTM_I, LSTM_F, LSTM_G, LSTM_O)   # p1 kernel lane order
ORDER_FIGO = (LSTM_F, LSTM_I, LSTM_G, LSTM_O)   # popnn default cell order
ORDER_RUC = (GRU_R, GRU_U, GRU_C)               # popnn default GRU order


def n_gates(mode: str) -> int:
    return 4 if mode == LSTM else 3


@dataclass(frozen=True)
class Workload:
    """A named layer workload: shapes, dtype and the init recipe."""
    name: str
    mode: str                 # "lstm" | "gru"
    dtype: str                # "f32" | "bf16" (storage; accumulation is fp32)
    T: int
    B: int
    I: int
    H: int
    w_scale: float            # weights and biases ~ U(-w_scale, w_scale)
    h0_std: float             # 0.0 -> zero initial state (passed as NULL)
    c0_std: float
    seed: int
    layers: int = 1
    bidir: bool = False
    reset_after: bool = True  # GRU only
    order: tuple = field(default=None)

    def gate_order(self):
        if self.order is not None:
            return tuple(self.order)
        return ORDER_IFGO if self.mode == LSTM else ORDER_RUC

    def flops_gemm(self) -> float:
        """Algorithmic GEMM FLOPs of fwd + bwd-data + bwd-weights.

        6*T*B*G*H*(I+H) per layer and direction: the input projection, the
        recurrent product, their two data-gradient products and the two
        weight-gradient products, each 2*T*B*G*H*K (non-linearities excluded,
        as the popnn FLOP counters on the Lstm.cpp/Gru.cpp pages do)."""
        G = n_gates(self.mode)
        tot = 0.0
        dirs = 2 if self.bidir else 1
        for layer in range(self.layers):
            I = self.I if layer == 0 else self.H * dirs
            tot += dirs * 6.0 * self.T * self.B * G * self.H * (I + self.H)
        return tot


def _wl(name, mode, dtype, T, B, I, H, w_scale, h0_std, c0_std, seed, **kw):
    return Workload(name, mode, dtype, T, B, I, H, w_scale, h0_std, c0_std, seed, **kw)


WORKLOADS = {
    w.name: w for w in [
        _wl("lstm_f32_t8_b2_i16_h32", LSTM, F32, 8, 2, 16, 32,
            1 / math.sqrt(32), 1.0, 1.0, 1001),
        _wl("gru_f32_t64_b16_i256_h256", GRU, F32, 64, 16, 256, 256,
            1 / 16, 0.0, 0.0, 1002, reset_after=False),
        _wl("grura_f32_t64_b16_i256_h256", GRU, F32, 64, 16, 256, 256,
            1 / 16, 0.0, 0.0, 1002, reset_after=True),
        _wl("lstm_bf16_t256_b64_i1024_h1024", LSTM, BF16, 256, 64, 1024, 1024,
            1 / 32, 0.1, 0.1, 1003),
        _wl("bilstm2_f32_t512_b32_i512_h512", LSTM, F32, 512, 32, 512, 512,
            1 / math.sqrt(512), 0.0, 0.0, 1004, layers=2, bidir=True),
        _wl("lstm_bf16_t128_b128_i2048_h2048", LSTM, BF16, 128, 128, 2048, 2048,
            1 / 45, 0.0, 0.0, 1005),
        _wl("grura_bf16_t128_b128_i2048_h2048", GRU, BF16, 128, 128, 2048, 2048,
            1 / 45, 0.0, 0.0, 1005, reset_after=True),
    ]
}

HEADLINE = "lstm_bf16_t256_b64_i1024_h1024"


def round_to(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to the storage type (round-to-nearest-even) and
    return them as fp64, so that both sides consume identical values."""
    a32 = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == F32:
        return a32.astype(np.float64)
    bits = a32.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    out = (rounded & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    # NaN/Inf are never drawn here; keep the rule simple
    return out.astype(np.float64)


@dataclass
class LayerParams:
    W_ih: np.ndarray
    W_hh: np.ndarray
    b_ih: np.ndarray
    b_hh: np.ndarray


def make_inputs(wl: Workload, seed: int | None = None, with_grad: bool = True):
    """Draw every tensor of a workload in the fixed order.

    Returns a dict with fp64 arrays already rounded to wl.dtype:
      params: list over layers of list over directions of LayerParams
      x [T,B,I], h0/c0 [B,H] or None (per layer and direction: lists),
      g [T,B,H*dirs] (upstream gradient of the last layer's output).
    """
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    G = n_gates(wl.mode)
    dirs = 2 if wl.bidir else 1
    k = wl.w_scale
    params = []
    for layer in range(wl.layers):
        I = wl.I if layer == 0 else wl.H * dirs
        per_dir = []
        for _ in range(dirs):
            W_ih = rng.uniform(-k, k, size=(G * wl.H, I))
            W_hh = rng.uniform(-k, k, size=(G * wl.H, wl.H))
            b_ih = rng.uniform(-k, k, size=(G * wl.H,))
            b_hh = rng.uniform(-k, k, size=(G * wl.H,))
            per_dir.append(LayerParams(*(round_to(a, wl.dtype) for a in (W_ih, W_hh, b_ih, b_hh))))
        params.append(per_dir)
    x = round_to(rng.standard_normal((wl.T, wl.B, wl.I)), wl.dtype)
    h0 = c0 = None
    if wl.h0_std > 0:
        h0 = round_to(wl.h0_std * rng.standard_normal((wl.B, wl.H)), wl.dtype)
    if wl.mode == LSTM and wl.c0_std > 0:
        c0 = round_to(wl.c0_std * rng.standard_normal((wl.B, wl.H)), wl.dtype)
    out = dict(params=params, x=x, h0=h0, c0=c0)
    if with_grad:
        out["g"] = round_to(rng.standard_normal((wl.T, wl.B, wl.H * dirs)), wl.dtype)
    return out


def small(wl: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (sizes for quick cases)."""
    return replace(wl, **changes)
