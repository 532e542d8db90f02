"""Torch-facing marshalling over the C ABI: tensors in, device addresses out.

PyTorch provides device memory and the stream; every step of the layer runs
in the HIP kernels of librnn.so. Nothing here computes.
"""
from __future__ import annotations

import torch

from . import _lib as L

TORCH_DT = {L.RNN_F32: torch.float32, L.RNN_BF16: torch.bfloat16}
DT_OF = {"f32": L.RNN_F32, "bf16": L.RNN_BF16}
MODE_OF = {"lstm": L.RNN_LSTM, "gru": L.RNN_GRU}


def _p(t) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(st: int, where: str):
    if st != L.RNN_OK:
        raise L.RnnError(st, where)


class RnnLayer:
    """One layer and direction: descriptor plus its workspace."""

    def __init__(self, mode: str, T: int, B: int, I: int, H: int, dtype: str, direction: int = 0,
                 reset_after: bool = True, gate_order=None, ldx: int = 0, ldy: int = 0, device="cuda",
                 lengths=None, att=None, recompute=False, dw_hh_mode=0, stepwise=False):
        """`lengths`: optional int32 device tensor [B] of per-row sequence
        lengths; `att`: optional [T, B] device tensor of AUGRU attention
        scores in the layer's dtype (GRU only). Both are kept referenced by
        the layer; the three calls read them. `recompute` (LSTM): keep only
        the gates between the forward and backward calls. `dw_hh_mode` 1:
        the recurrent-weight gradient from the separate product, never
        accumulated inside the BPTT kernel. `stepwise`: the per-step
        recurrence even where a persistent plan fits."""
        self.mode, self.dtype = mode, dtype
        self.T, self.B, self.I, self.H = T, B, I, H
        if lengths is not None:
            assert lengths.dtype == torch.int32 and lengths.is_cuda and tuple(lengths.shape) == (B,)
            lengths = lengths.contiguous()
        if att is not None:
            assert mode == "gru" and att.is_cuda and tuple(att.shape) == (T, B)
            assert att.dtype == TORCH_DT[DT_OF[dtype]]
            att = att.contiguous()
        self.lengths, self.att = lengths, att
        self.desc = L.make_desc(MODE_OF[mode], T, B, I, H, DT_OF[dtype], direction,
                                int(bool(reset_after)), gate_order, ldx, ldy, _p(lengths), _p(att),
                                int(bool(recompute)), int(dw_hh_mode), int(bool(stepwise)))
        self.ws_bytes = L.rnn_workspace_bytes(self.desc)
        if self.ws_bytes == 0:
            raise L.RnnError(L.RNN_ERR_INVALID_ARG, "rnn_workspace_bytes")
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)

    @property
    def torch_dtype(self):
        return TORCH_DT[DT_OF[self.dtype]]

    def fwd(self, x, h0, c0, W_ih, W_hh, b_ih, b_hh, y, hT=None, cT=None, stream=None):
        _check(L.rnn_fwd(self.desc, _p(x), _p(h0), _p(c0), _p(W_ih), _p(W_hh), _p(b_ih), _p(b_hh),
                         _p(y), _p(hT), _p(cT), _p(self.workspace), self.ws_bytes, _stream(stream)),
               "rnn_fwd")

    def bwd_data(self, W_ih, W_hh, h0, c0, y, dy, dhT, dcT, dx, dh0=None, dc0=None, accumulate=False,
                 stream=None, datt=None):
        _check(L.rnn_bwd_data(self.desc, _p(W_ih), _p(W_hh), _p(h0), _p(c0), _p(y), _p(dy), _p(dhT),
                              _p(dcT), _p(dx), _p(dh0), _p(dc0), _p(datt), int(bool(accumulate)),
                              _p(self.workspace), self.ws_bytes, _stream(stream)),
               "rnn_bwd_data")

    def bwd_weights(self, x, h0, y, dW_ih, dW_hh, db_ih, db_hh, accumulate=False, stream=None):
        _check(L.rnn_bwd_weights(self.desc, _p(x), _p(h0), _p(y), _p(dW_ih), _p(dW_hh), _p(db_ih),
                                 _p(db_hh), int(bool(accumulate)), _p(self.workspace), self.ws_bytes,
                                 _stream(stream)),
               "rnn_bwd_weights")

    def device_status(self) -> int:
        return L.rnn_last_device_status(_p(self.workspace))


class RnnStack:
    """Stacked, optionally bidirectional layers over one [T, B, I] input.

    Layer l writes [T, B, dirs*H]: the forward direction in columns [0, H),
    the reverse one in [H, 2H) (row stride dirs*H), and layer l+1 reads that
    tensor as its input. A bidirectional layer is one direction-2 layer of
    the C ABI: both directions share one persistent launch per pass.
    Backward: the input gradient of layer l+1 (both directions summed) is the
    output gradient of layer l.
    Parameters: params[l][d] = (W_ih, W_hh, b_ih, b_hh) device tensors; for
    a bidirectional layer the two directions' tensors are passed without a
    copy when they already sit back to back in one [2, ...] tensor (views of
    it), and are stacked into a temporary otherwise. The same holds for the
    weight gradients grads[l][d]. h0/c0 ([B, H]) apply to every layer and
    direction.
    """

    def __init__(self, mode, T, B, I, H, dtype, layers, bidir, reset_after=True, gate_order=None,
                 device="cuda", lengths=None, stepwise=False):
        self.dirs = 2 if bidir else 1
        self.T, self.B, self.I, self.H = T, B, I, H
        self.layers = []
        for layer in range(layers):
            Il = I if layer == 0 else H * self.dirs
            self.layers.append(RnnLayer(mode, T, B, Il, H, dtype, direction=2 if bidir else 0,
                                        reset_after=reset_after, gate_order=gate_order, ldx=Il,
                                        ldy=H * self.dirs, device=device, lengths=lengths,
                                        stepwise=stepwise))
        dt = self.layers[0].torch_dtype
        self.ys = [torch.empty(T, B, H * self.dirs, dtype=dt, device=device) for _ in range(layers)]
        # input gradients of layers 1.. (the output gradients of the layer below)
        self.dxs = [None] + [torch.empty(T, B, H * self.dirs, dtype=dt, device=device)
                             for _ in range(layers - 1)]

    @staticmethod
    def _pair(a, b):
        """([2, ...] tensor holding a and b, whether it is a view of them)."""
        if (a.shape == b.shape and a.dtype == b.dtype and a.is_contiguous() and b.is_contiguous()
                and a.untyped_storage().data_ptr() == b.untyped_storage().data_ptr()
                and b.storage_offset() == a.storage_offset() + a.numel()):
            return torch.as_strided(a, (2,) + tuple(a.shape), (a.numel(),) + tuple(a.stride()),
                                    a.storage_offset()), True
        return torch.stack([a, b]), False

    def _layer_params(self, li, params):
        if self.dirs == 1:
            return params[li][0]
        return tuple(self._pair(params[li][0][i], params[li][1][i])[0] for i in range(4))

    def _state(self, t):
        if t is None or self.dirs == 1:
            return t
        return torch.stack([t, t])

    @staticmethod
    def _on(stream):
        """Context that makes `stream` torch's current stream: the stacked
        temporaries and copy-backs of a bidirectional layer are then ordered
        with the library's kernels on it (a raw stream handle is refused,
        since torch could not order its own work with it)."""
        import contextlib
        if stream is None:
            return contextlib.nullcontext()
        if not isinstance(stream, torch.cuda.Stream):
            raise TypeError("RnnStack takes a torch.cuda.Stream (or None for the current stream)")
        return torch.cuda.stream(stream)

    def fwd(self, x, params, h0=None, c0=None, stream=None):
        with self._on(stream):
            return self._fwd(x, params, h0, c0)

    def bwd(self, x, params, dy, dx=None, grads=None, h0=None, c0=None, stream=None):
        """dy: gradient of the last layer's output. grads[l][d] = (dW_ih, dW_hh, db_ih, db_hh)
        (or None to skip the weight gradients)."""
        with self._on(stream):
            return self._bwd(x, params, dy, dx, grads, h0, c0)

    def _fwd(self, x, params, h0, c0):
        inp = x
        h0s, c0s = self._state(h0), self._state(c0)
        for li, lay in enumerate(self.layers):
            W_ih, W_hh, b_ih, b_hh = self._layer_params(li, params)
            lay.fwd(inp, h0s, c0s, W_ih, W_hh, b_ih, b_hh, self.ys[li])
            inp = self.ys[li]
        return self.ys[-1]

    def _bwd(self, x, params, dy, dx, grads, h0, c0):
        d_out = dy
        h0s, c0s = self._state(h0), self._state(c0)
        for li in range(len(self.layers) - 1, -1, -1):
            lay = self.layers[li]
            d_in = dx if li == 0 else self.dxs[li]
            W_ih, W_hh, _, _ = self._layer_params(li, params)
            lay.bwd_data(W_ih, W_hh, h0s, c0s, self.ys[li], d_out, None, None, d_in)
            if grads is not None:
                inp = x if li == 0 else self.ys[li - 1]
                if self.dirs == 1:
                    lay.bwd_weights(inp, h0s, self.ys[li], *grads[li][0])
                else:
                    pairs = [self._pair(grads[li][0][i], grads[li][1][i]) for i in range(4)]
                    lay.bwd_weights(inp, h0s, self.ys[li], *(t for t, _ in pairs))
                    for i, (t, view) in enumerate(pairs):
                        if not view:
                            grads[li][0][i].copy_(t[0])
                            grads[li][1][i].copy_(t[1])
            d_out = d_in
        return dx
