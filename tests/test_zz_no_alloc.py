"""rnn_fwd_noalloc: the forward entry point whose workspace is the library's
static device array. Called through the C ABI and compared with rnn_fwd
(same kernels, caller-owned workspace): the outputs must be bit-identical,
on two calls in a row, the second with a smaller input (the array keeps the
first call's contents)."""
import numpy as np
import pytest
import torch

from gru_layer_fwd_amd import _lib as L
from gru_layer_fwd_amd import synth

TDT = {L.RNN_F32: torch.float32, L.RNN_BF16: torch.bfloat16}


def _tensors(mode, T, B, I, H, dtype, seed):
    rng = np.random.default_rng(seed)
    G = 4 if mode == L.RNN_LSTM else 3
    k = 1.0 / np.sqrt(H)
    dt = TDT[dtype]
    r = lambda a: torch.from_numpy(synth.round_to(a, "bf16" if dtype == L.RNN_BF16 else "f32")).to("cuda", dt)  # noqa: E731
    return dict(x=r(rng.standard_normal((T, B, I))), h0=r(0.3 * rng.standard_normal((B, H))),
                c0=r(0.3 * rng.standard_normal((B, H))) if mode == L.RNN_LSTM else None,
                W_ih=r(rng.uniform(-k, k, (G * H, I))), W_hh=r(rng.uniform(-k, k, (G * H, H))),
                b_ih=r(rng.uniform(-k, k, G * H)), b_hh=r(rng.uniform(-k, k, G * H)))


def _p(t):
    return 0 if t is None else t.data_ptr()


def _forward(desc, t, noalloc):
    T, B, H = desc.T, desc.B, desc.H
    dt = t["x"].dtype
    y = torch.full((T, B, H), float("nan"), dtype=dt, device="cuda")
    hT = torch.full((B, H), float("nan"), dtype=dt, device="cuda")
    cT = torch.full((B, H), float("nan"), dtype=dt, device="cuda") if desc.mode == L.RNN_LSTM else None
    s = torch.cuda.current_stream().cuda_stream
    args = [_p(t[k]) for k in ("x", "h0", "c0", "W_ih", "W_hh", "b_ih", "b_hh")] + [_p(y), _p(hT), _p(cT)]
    if noalloc:
        st = L.rnn_fwd_noalloc(desc, *args, s)
        ws = None
    else:
        n = L.rnn_workspace_bytes(desc)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        st = L.rnn_fwd(desc, *args, ws.data_ptr(), n, s)
    assert st == L.RNN_OK, L.rnn_status_string(st)
    torch.cuda.synchronize()
    if ws is not None:
        assert L.rnn_last_device_status(ws.data_ptr()) == L.RNN_OK
    out = {"y": y, "hT": hT}
    if cT is not None:
        out["cT"] = cT
    return {k: v.float().cpu().numpy() for k, v in out.items()}


@pytest.mark.gpu
def test_noalloc_forward_matches_rnn_fwd_on_two_calls():
    cases = [
        # first call: ring path, 24 rows, H = 256 (about 6 MiB of the array)
        (L.RNN_LSTM, 16, 24, 64, 256, L.RNN_BF16, 0, 1),
        # second call, smaller: fewer steps, rows and units, other direction
        (L.RNN_LSTM, 6, 5, 32, 128, L.RNN_BF16, 1, 2),
        # a third, smaller still, another cell: reset-after GRU in fp32
        (L.RNN_GRU, 5, 3, 16, 32, L.RNN_F32, 0, 3),
    ]
    for mode, T, B, I, H, dtype, direction, seed in cases:
        print(f"[noalloc] mode={mode} T={T} B={B} I={I} H={H} dtype={dtype} dir={direction}", flush=True)
        desc = L.make_desc(mode, T, B, I, H, dtype, direction, 1)
        assert L.rnn_workspace_bytes(desc) <= L.RNN_NOALLOC_SCRATCH_BYTES
        t = _tensors(mode, T, B, I, H, dtype, seed)
        ref = _forward(desc, t, noalloc=False)
        got = _forward(desc, t, noalloc=True)
        for k in ref:
            assert np.all(np.isfinite(got[k])), k
            np.testing.assert_array_equal(got[k], ref[k], err_msg=k)


def test_noalloc_refuses_descriptors_beyond_the_array():
    # the headline shape needs about 206 MiB of workspace: refused on the
    # host, before the device is touched
    d = L.make_desc(L.RNN_LSTM, 256, 64, 1024, 1024, L.RNN_BF16)
    assert L.rnn_workspace_bytes(d) > L.RNN_NOALLOC_SCRATCH_BYTES
    assert L.rnn_fwd_noalloc(d, 16, 0, 0, 16, 16, 16, 16, 16, 0, 0, 0) == L.RNN_ERR_WORKSPACE_TOO_SMALL
    bad = L.make_desc(L.RNN_LSTM, 0, 64, 1024, 1024, L.RNN_BF16)
    assert L.rnn_fwd_noalloc(bad, 16, 0, 0, 16, 16, 16, 16, 16, 0, 0, 0) == L.RNN_ERR_INVALID_ARG
