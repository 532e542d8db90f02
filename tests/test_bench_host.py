"""Host logic of bench.py: the algorithmic work per launch, the MFMA
ceilings and the rule that stored HBM traffic is only reported for the
kernel sources it was measured on. No device work."""
import json
import os

import pytest

import bench
from gru_layer_fwd_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_headline_algorithmic_flops():
    wl = synth.WORKLOADS["lstm_bf16_t256_b64_i1024_h1024"]
    w = bench._work(wl)
    TB, G, H, I = 256 * 64, 4, 1024, 1024
    # M*N*K products: projection and input gradient TB x 4H x I, each
    # persistent kernel TB x 4H x H, weight gradients 4H x (I+H) x TB
    assert w["proj_gemm"][0] == 2.0 * TB * G * H * I == pytest.approx(137.4e9, rel=1e-3)
    assert w["dx_gemm"][0] == w["proj_gemm"][0]
    assert w["rec_fwd"][0] == w["rec_bwd"][0] == 2.0 * TB * G * H * H
    assert w["dw_gemm"][0] == 2.0 * TB * G * H * (I + H) == pytest.approx(274.9e9, rel=1e-3)
    # the step's work per timestep*batch element: 6*G*H*(I+H) FLOPs
    step = sum(w[k][0] for k in ("proj_gemm", "rec_fwd", "rec_bwd", "dx_gemm", "dw_gemm"))
    assert step / TB == 6 * G * H * (I + H)


def test_stacked_bidirectional_work_counts_every_layer_and_direction():
    wl = synth.WORKLOADS["bilstm2_f32_t512_b32_i512_h512"]
    w = bench._work(wl)
    TB, G, H = 512 * 32, 4, 512
    # layer 1 reads I = 512, layer 2 the concatenated 1024; two directions each
    proj = 2 * (2.0 * TB * G * H * 512) + 2 * (2.0 * TB * G * H * 1024)
    assert w["proj_gemm"][0] == proj
    assert w["rec_fwd"][0] == 4 * 2.0 * TB * G * H * H


def test_mfma_ceilings():
    # bf16 at the published dense peak; fp32 products run as six bf16 MFMAs
    # on split operands, so their ceiling is that peak over six, above the
    # published fp32 matrix peak
    assert bench.PEAK_TFLOPS["bf16"] == 2500.0
    assert bench.PEAK_TFLOPS["f32"] == pytest.approx(2500.0 / 6)
    assert 157.3 < bench.PEAK_TFLOPS["f32"] < bench.PEAK_TFLOPS["bf16"]


def test_stored_traffic_only_for_the_measured_sources(monkeypatch):
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
        t = json.load(fh)
    name = "lstm_bf16_t256_b64_i1024_h1024"
    e = t[name]["rec_bwd"]
    monkeypatch.setattr(bench, "kernel_hash", lambda: e["kernel_hash"])
    assert bench.stored_traffic(name, "rec_bwd") == e["bytes_per_launch"]
    assert bench.stored_traffic(name, "no_such_kernel") is None
    assert bench.stored_traffic("no_such_workload", "rec_bwd") is None
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0" * 16)
    assert bench.stored_traffic(name, "rec_bwd") is None


def test_kernel_hash_covers_the_kernel_sources():
    h = bench.kernel_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    for f in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, f)), f
