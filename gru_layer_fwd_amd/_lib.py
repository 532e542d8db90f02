"""ctypes binding of librnn.so (include/rnn.h). Argument marshalling only.

The functions keep the C names and arguments; tensor arguments are passed as
integer device addresses (0 = NULL) and `stream` as an integer hipStream_t.
Loading fails loudly when the library has not been built: there is no other
implementation behind these names.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librnn.so")

RNN_LSTM, RNN_GRU = 0, 1
RNN_F32, RNN_BF16 = 0, 1

RNN_OK = 0
RNN_ERR_INVALID_ARG = -1
RNN_ERR_WORKSPACE_TOO_SMALL = -2
RNN_ERR_UNSUPPORTED = -3
RNN_ERR_DEVICE = -4
RNN_ERR_TIMEOUT = -5

# every function the header declares, with its C signature
_c = ctypes
_P = _c.c_void_p
_SIGS = {
    "rnn_workspace_bytes": (_c.c_size_t, [_P]),
    "rnn_fwd": (_c.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _c.c_size_t, _P]),
    "rnn_fwd_noalloc": (_c.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "rnn_bwd_data": (_c.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _c.c_int, _P, _c.c_size_t,
                                _P]),
    "rnn_bwd_weights": (_c.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _c.c_int, _P, _c.c_size_t, _P]),
    "rnn_last_device_status": (_c.c_int, [_P]),
    "rnn_status_string": (_c.c_char_p, [_c.c_int]),
    "rnn_set_handshake_timeout": (_c.c_int, [_c.c_double]),
    "rnn_plan_query": (_c.c_int, [_P, _c.c_int, _c.c_int, _c.c_int, _P]),
    "rnn_handshake_probe": (_c.c_int, [_P, _c.c_int, _P, _c.c_size_t, _P]),
    "rnn_profile_enable": (_c.c_int, [_c.c_int]),
    "rnn_profile_read": (_c.c_int, [_P, _c.c_int, _c.c_int]),
}


class RnnDesc(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int),
        ("direction", ctypes.c_int),
        ("reset_after", ctypes.c_int),
        ("gate_order", ctypes.c_int * 4),
        ("dtype", ctypes.c_int),
        ("T", ctypes.c_int),
        ("B", ctypes.c_int),
        ("I", ctypes.c_int),
        ("H", ctypes.c_int),
        ("ldx", ctypes.c_longlong),
        ("ldy", ctypes.c_longlong),
        ("lengths", ctypes.c_void_p),
        ("att", ctypes.c_void_p),
        ("recompute", ctypes.c_int),
        ("dw_hh_mode", ctypes.c_int),
        ("stepwise", ctypes.c_int),
    ]


class RnnPlan(ctypes.Structure):
    _fields_ = [
        ("groups", ctypes.c_int),
        ("rows", ctypes.c_int),
        ("slices", ctypes.c_int),
        ("units", ctypes.c_int),
        ("waves", ctypes.c_int),
        ("workgroups", ctypes.c_int),
        ("dual", ctypes.c_int),
        ("ring", ctypes.c_int),
        ("xcd_span", ctypes.c_int),
        ("model_us_per_step", ctypes.c_double),
        ("blocks", ctypes.c_int),
        ("fused_dw", ctypes.c_int),
        ("stepwise", ctypes.c_int),
    ]


class RnnKernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_longlong), ("total_ms", ctypes.c_double)]


_lib = None


def select(path: str):
    """Load another build of the library (e.g. the step-timer debug build)
    instead of librnn.so; only before the first call into the library."""
    global LIB_PATH
    if _lib is not None and os.path.abspath(path) != os.path.abspath(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is already loaded")
    LIB_PATH = path


def lib():
    """The loaded librnn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m gru_layer_fwd_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class RnnError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib().rnn_status_string(status).decode()
        super().__init__(f"{where}: {msg} ({status})")
        self.status = status


def make_desc(mode: int, T: int, B: int, I: int, H: int, dtype: int, direction: int = 0,
              reset_after: int = 1, gate_order=None, ldx: int = 0, ldy: int = 0, lengths: int = 0,
              att: int = 0, recompute: int = 0, dw_hh_mode: int = 0, stepwise: int = 0) -> RnnDesc:
    """`lengths`: device address of int32[B] sequence lengths (0 = all T);
    `att`: device address of the [T][B] AUGRU attention scores (0 = none);
    `recompute`: 1 = LSTM cell states rebuilt in the backward pass;
    `dw_hh_mode`: 1 = dW_hh from the separate product, never fused into BPTT;
    `stepwise`: 1 = the per-step recurrence even where a persistent plan fits."""
    d = RnnDesc()
    d.mode, d.direction, d.reset_after, d.dtype = mode, direction, reset_after, dtype
    d.T, d.B, d.I, d.H, d.ldx, d.ldy = T, B, I, H, ldx, ldy
    d.lengths = lengths or None
    d.att = att or None
    d.recompute = recompute
    d.dw_hh_mode = dw_hh_mode
    d.stepwise = stepwise
    if gate_order is None:
        gate_order = (0, 1, 2, 3) if mode == RNN_LSTM else (0, 1, 2)
    order = list(gate_order) + [0] * (4 - len(gate_order))
    for k in range(4):
        d.gate_order[k] = order[k]
    return d


def rnn_workspace_bytes(desc: RnnDesc) -> int:
    return int(lib().rnn_workspace_bytes(ctypes.byref(desc)))


def rnn_fwd(desc, x, h0, c0, W_ih, W_hh, b_ih, b_hh, y, hT, cT, workspace, ws_bytes, stream) -> int:
    return lib().rnn_fwd(ctypes.byref(desc), x, h0, c0, W_ih, W_hh, b_ih, b_hh, y, hT, cT,
                         workspace, ws_bytes, stream)


RNN_NOALLOC_SCRATCH_BYTES = 64 << 20


def rnn_fwd_noalloc(desc, x, h0, c0, W_ih, W_hh, b_ih, b_hh, y, hT, cT, stream) -> int:
    return lib().rnn_fwd_noalloc(ctypes.byref(desc), x, h0, c0, W_ih, W_hh, b_ih, b_hh, y, hT, cT, stream)


def rnn_bwd_data(desc, W_ih, W_hh, h0, c0, y, dy, dhT, dcT, dx, dh0, dc0, datt, accumulate,
                 workspace, ws_bytes, stream) -> int:
    return lib().rnn_bwd_data(ctypes.byref(desc), W_ih, W_hh, h0, c0, y, dy, dhT, dcT, dx, dh0, dc0,
                              datt, accumulate, workspace, ws_bytes, stream)


def rnn_bwd_weights(desc, x, h0, y, dW_ih, dW_hh, db_ih, db_hh, accumulate, workspace, ws_bytes,
                    stream) -> int:
    return lib().rnn_bwd_weights(ctypes.byref(desc), x, h0, y, dW_ih, dW_hh, db_ih, db_hh, accumulate,
                                 workspace, ws_bytes, stream)


def rnn_last_device_status(workspace) -> int:
    return lib().rnn_last_device_status(workspace)


def rnn_status_string(status: int) -> str:
    return lib().rnn_status_string(status).decode()


def rnn_set_handshake_timeout(seconds: float) -> int:
    """Handshake time-out for later calls (0: default; < 0: give up at once)."""
    return lib().rnn_set_handshake_timeout(float(seconds))


def rnn_plan_query(desc, pass_: int, cu_count: int = 0, wg_per_cu: int = 0):
    """(status, RnnPlan) of the persistent kernel of pass 0 (forward) or 1
    (backward); cu_count/wg_per_cu > 0 inject the device's CU count and the
    kernel's co-resident workgroups per CU (then no device is touched)."""
    out = RnnPlan()
    st = lib().rnn_plan_query(ctypes.byref(desc), int(pass_), int(cu_count), int(wg_per_cu), ctypes.byref(out))
    return st, out


def rnn_handshake_probe(desc, pass_: int, workspace, ws_bytes, stream) -> int:
    return lib().rnn_handshake_probe(ctypes.byref(desc), int(pass_), workspace, ws_bytes, stream)


def rnn_profile_enable(on: bool) -> int:
    return lib().rnn_profile_enable(int(bool(on)))


def rnn_profile_read(reset: bool = True) -> dict:
    """{label: (launches, total_ms)} of the kernels queued while enabled."""
    n = lib().rnn_profile_read(None, 0, 0)
    if n < 0:
        raise RnnError(n, "rnn_profile_read")
    buf = (RnnKernelTime * max(n, 1))()
    n = lib().rnn_profile_read(ctypes.cast(buf, ctypes.c_void_p), n, int(bool(reset)))
    if n < 0:
        raise RnnError(n, "rnn_profile_read")
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(n)}
