"""CPU oracle of the LSTM and GRU layer equations (fp64, numpy).

TEST INFRASTRUCTURE ONLY. Only the test-suite, the smoke check and the CPU
baseline leg of the benchmark may import this module; the product path (the
HIP library and its binding) never does, and shares no code with it.

Every function evaluates the recurrence step by step, in plain fp64, in the
order and notation of the pages it follows:

* LSTM forward: popnn Lstm.cpp page, "basicLstmCellForwardPass" and
  "applyGateNonlinearities" (sigmoid on input/forget/output gates, tanh on the
  candidate; c = f*c_prev + i*g; h = o*tanh(c)).
* LSTM backward: popnn Lstm.cpp page, "backwardStepImpl" (one step of BPTT
  with the carried cell-state gradient), "basicLstmParamUpdate" (weight
  gradients dW += dG^T [x; h_prev]); cross-checked by the LSTM branch of the
  persistent backward kernel on the CUDA fragment page.
* GRU forward: popnn Gru.cpp page, "basicGruCellForwardPass" (reset, update,
  candidate; h = u*h_prev + (1-u)*c) and, for the reset-after variant,
  "gruCellForwardPassCalcUnitsResetAfter" (reset applied to the recurrent
  candidate term h_prev W_hc^T + b_hc).
* GRU backward: popnn Gru.cpp page, "backwardStepImpl" (basic) and
  "backwardStepImplResetAfter"; weight gradients "basicGruParamUpdate";
  cross-checked by the GRU (linear-before-reset) branch of the CUDA fragment.
* AUGRU: popnn Gru.cpp page, the attention-score branch of the GRU forward
  step ("UpdateScores": the update gate becomes u - a*u with a = att[t, b],
  one score per step and batch row) and of the backward step
  ("AttentionsGrad": the score gradient is minus the sum over hidden units
  of the update-gate gradient times the unscaled gate). Written here as the
  plain chain rule of h = ua*h_prev + (1-ua)*c with ua = (1-a)*u; the
  unscaled u is kept, so no division by 1-a is needed.

Conventions (readings where the pages leave a point open):
* Gate storage order: order[k] is the gate id stored in row block k of W_ih,
  W_hh, b_ih, b_hh (LSTM ids i=0, f=1, g=2, o=3; GRU r=0, u=1, c=2).
* Two bias vectors b_ih and b_hh; LSTM and basic GRU use their sum, the
  reset-after GRU keeps the recurrent candidate bias inside r*(.).
* reverse=True processes t = T-1 .. 0 but stores every per-step tensor at its
  own t; the final state is the one after t = 0.
* dh carry is seeded from dhT (and dcT for LSTM); None means zero.
* Weight gradients are sums over (t, b); db_ih and db_hh are reported
  separately (they differ only for the reset-after candidate row block).
* Variable sequence lengths (popnn's per-batch time-step limits: the gates of
  steps past a row's limit are masked to zero, the output sequence is
  zero-filled, and the state and the carried gradient state are latched,
  i.e. not updated, on those steps): row b has lengths[b] in [0, T] steps
  and step t is active for it iff t < lengths[b]. An inactive step outputs
  zero, saves zero gates, keeps the state and (backward) has zero gate
  gradients while the carries pass through unchanged. In the reverse
  direction a row therefore starts at its own step lengths[b]-1 from h0/c0.
  lengths=None means every row runs all T steps.
"""
from __future__ import annotations

import numpy as np

LSTM_I, LSTM_F, LSTM_G, LSTM_O = 0, 1, 2, 3
GRU_R, GRU_U, GRU_C = 0, 1, 2


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def _slot(order, gate, H):
    """Row range of gate `gate` in storage order `order`."""
    k = list(order).index(gate)
    return slice(k * H, (k + 1) * H)


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def _steps(T, reverse):
    return range(T - 1, -1, -1) if reverse else range(T)


def _lengths(lengths, T, B):
    if lengths is None:
        return np.full(B, T, dtype=np.int64)
    L = np.asarray(lengths, dtype=np.int64)
    assert L.shape == (B,) and np.all((L >= 0) & (L <= T)), "lengths must be B values in [0, T]"
    return L


def _first(t, L, T, reverse):
    """Per row: is t the first step processed for that row (its previous
    state is the initial one)?"""
    return (t == L - 1) if reverse else np.full(L.shape, t == 0)


def _prev(seq, t, first, init, reverse):
    """Per row: the state before step t (init on the row's first step)."""
    T = seq.shape[0]
    tp = (t + 1) if reverse else (t - 1)
    before = seq[tp] if 0 <= tp < T else np.zeros_like(init)
    return np.where(first[:, None], init, before)


# ---------------------------------------------------------------- LSTM ----

def lstm_forward(x, h0, c0, W_ih, W_hh, b_ih, b_hh, order=(0, 1, 2, 3), reverse=False, lengths=None):
    """LSTM layer forward over a sequence x [T, B, I].

    Returns a dict with y [T,B,H], hT, cT and the per-step activations the
    backward pass reads (i, f, g, o, c each [T,B,H]) plus the inputs."""
    x, W_ih, W_hh, b_ih, b_hh = map(_f64, (x, W_ih, W_hh, b_ih, b_hh))
    T, B, _ = x.shape
    H = W_hh.shape[1]
    L = _lengths(lengths, T, B)
    h = np.zeros((B, H)) if h0 is None else _f64(h0).copy()
    c = np.zeros((B, H)) if c0 is None else _f64(c0).copy()
    s = {k: _slot(order, k, H) for k in (LSTM_I, LSTM_F, LSTM_G, LSTM_O)}
    st = {k: np.zeros((T, B, H)) for k in ("i", "f", "g", "o", "c", "y")}
    for t in _steps(T, reverse):
        m = (t < L)[:, None]                                  # rows with a step at t
        z = x[t] @ W_ih.T + b_ih + h @ W_hh.T + b_hh        # [B, 4H], storage order
        i = np.where(m, sigmoid(z[:, s[LSTM_I]]), 0.0)      # gates masked past a row's limit
        f = np.where(m, sigmoid(z[:, s[LSTM_F]]), 0.0)
        g = np.where(m, np.tanh(z[:, s[LSTM_G]]), 0.0)
        o = np.where(m, sigmoid(z[:, s[LSTM_O]]), 0.0)
        c_new = f * c + i * g
        h_new = o * np.tanh(c_new)
        c = np.where(m, c_new, c)                             # state latched past the limit
        h = np.where(m, h_new, h)
        for k, v in (("i", i), ("f", f), ("g", g), ("o", o), ("c", c_new), ("y", h_new)):
            st[k][t] = v
    st.update(hT=h, cT=c, x=x, h0=h0, c0=c0, W_ih=W_ih, W_hh=W_hh,
              order=tuple(order), reverse=reverse, lengths=L)
    return st


def lstm_backward(fw, dy, dhT=None, dcT=None):
    """BPTT through an LSTM layer given the forward record `fw`.

    dy [T,B,H] is the gradient arriving at every output; dhT/dcT seed the
    carries at the last processed step. Returns dx, dh0, dc0, dW_ih, dW_hh,
    db_ih, db_hh and the per-step gate gradients dG [T,B,4H] (storage order,
    gradients with respect to the gate pre-activations)."""
    x, W_ih, W_hh, order, reverse = fw["x"], fw["W_ih"], fw["W_hh"], fw["order"], fw["reverse"]
    T, B, _ = x.shape
    H = W_hh.shape[1]
    dy = _f64(dy)
    s = {k: _slot(order, k, H) for k in (LSTM_I, LSTM_F, LSTM_G, LSTM_O)}
    h0 = np.zeros((B, H)) if fw["h0"] is None else _f64(fw["h0"])
    c0 = np.zeros((B, H)) if fw["c0"] is None else _f64(fw["c0"])
    dh_carry = np.zeros((B, H)) if dhT is None else _f64(dhT).copy()
    dc_carry = np.zeros((B, H)) if dcT is None else _f64(dcT).copy()
    dx = np.zeros_like(x)
    dW_ih = np.zeros_like(W_ih)
    dW_hh = np.zeros_like(W_hh)
    db = np.zeros(W_hh.shape[0])
    dG_all = np.zeros((T, B, 4 * H))
    L = fw["lengths"]
    for t in reversed(list(_steps(T, reverse))):
        m = (t < L)[:, None]
        first = _first(t, L, T, reverse)
        c_prev = _prev(fw["c"], t, first, c0, reverse)
        h_prev = _prev(fw["y"], t, first, h0, reverse)
        i, f, g, o, c = (fw[k][t] for k in ("i", "f", "g", "o", "c"))
        dh = dy[t] + dh_carry
        tc = np.tanh(c)
        d_o = dh * tc * o * (1 - o)
        dc = dh * o * (1 - tc * tc) + dc_carry
        d_i = dc * g * i * (1 - i)
        d_f = dc * c_prev * f * (1 - f)
        d_g = dc * i * (1 - g * g)
        dG = np.zeros((B, 4 * H))
        dG[:, s[LSTM_I]], dG[:, s[LSTM_F]] = d_i, d_f
        dG[:, s[LSTM_G]], dG[:, s[LSTM_O]] = d_g, d_o
        dG = np.where(m, dG, 0.0)                     # no gradient past a row's limit
        dG_all[t] = dG
        dh_carry = np.where(m, dG @ W_hh, dh_carry)   # carries latched past the limit
        dc_carry = np.where(m, dc * f, dc_carry)
        dx[t] = dG @ W_ih
        dW_ih += dG.T @ x[t]
        dW_hh += dG.T @ h_prev
        db += dG.sum(axis=0)
    return dict(dx=dx, dh0=dh_carry, dc0=dc_carry, dW_ih=dW_ih, dW_hh=dW_hh,
                db_ih=db.copy(), db_hh=db.copy(), dG=dG_all)


# ----------------------------------------------------------------- GRU ----

def gru_forward(x, h0, W_ih, W_hh, b_ih, b_hh, reset_after, order=(0, 1, 2), reverse=False, lengths=None,
                att=None):
    """GRU layer forward over x [T, B, I] (basic or reset-after variant).

    Returns y, hT and the per-step r, u, c (activated), n_h (reset-after:
    h_prev W_hc^T + b_hc, saved before the reset gate is applied) and
    rh = r*h_prev (basic: the activation the candidate weights see).
    att [T, B] (AUGRU) scales the update gate: ua = (1 - att[t, b]) * u."""
    x, W_ih, W_hh, b_ih, b_hh = map(_f64, (x, W_ih, W_hh, b_ih, b_hh))
    T, B, _ = x.shape
    H = W_hh.shape[1]
    L = _lengths(lengths, T, B)
    A = None if att is None else _f64(att)
    assert A is None or A.shape == (T, B), "att must be [T, B]"
    h = np.zeros((B, H)) if h0 is None else _f64(h0).copy()
    sr, su, sc = (_slot(order, k, H) for k in (GRU_R, GRU_U, GRU_C))
    st = {k: np.zeros((T, B, H)) for k in ("r", "u", "c", "nh", "rh", "y")}
    for t in _steps(T, reverse):
        m = (t < L)[:, None]
        xi = x[t] @ W_ih.T + b_ih                 # input parts, storage order
        hr = h @ W_hh.T + b_hh                    # recurrent parts, storage order
        r = sigmoid(xi[:, sr] + hr[:, sr])
        u = sigmoid(xi[:, su] + hr[:, su])
        if reset_after:
            nh = hr[:, sc]
            c = np.tanh(xi[:, sc] + r * nh)
            st["nh"][t] = np.where(m, nh, 0.0)
        else:
            rh = r * h
            c = np.tanh(xi[:, sc] + rh @ W_hh[sc].T + b_hh[sc])
            st["rh"][t] = np.where(m, rh, 0.0)
        ua = u if A is None else (1 - A[t][:, None]) * u   # attention-scaled update gate
        h_new = ua * h + (1 - ua) * c
        h = np.where(m, h_new, h)                 # state latched past a row's limit
        st["r"][t], st["u"][t], st["c"][t] = (np.where(m, v, 0.0) for v in (r, u, c))
        st["y"][t] = np.where(m, h_new, 0.0)
    st.update(hT=h, x=x, h0=h0, W_ih=W_ih, W_hh=W_hh, order=tuple(order),
              reverse=reverse, reset_after=reset_after, lengths=L, att=A)
    return st


def gru_backward(fw, dy, dhT=None):
    """BPTT through a GRU layer given the forward record `fw`.

    Returns dx, dh0, dW_ih, dW_hh, db_ih, db_hh and the per-step
    pre-activation gradients dGi (input side: [d_r, d_u, d_c]) and dGh
    (recurrent side), both [T,B,3H] in storage order; with attention scores
    also datt [T, B]."""
    x, W_ih, W_hh, order, reverse = fw["x"], fw["W_ih"], fw["W_hh"], fw["order"], fw["reverse"]
    ra = fw["reset_after"]
    T, B, _ = x.shape
    H = W_hh.shape[1]
    dy = _f64(dy)
    sr, su, sc = (_slot(order, k, H) for k in (GRU_R, GRU_U, GRU_C))
    h0 = np.zeros((B, H)) if fw["h0"] is None else _f64(fw["h0"])
    carry = np.zeros((B, H)) if dhT is None else _f64(dhT).copy()
    dx = np.zeros_like(x)
    dW_ih = np.zeros_like(W_ih)
    dW_hh = np.zeros_like(W_hh)
    db_ih = np.zeros(W_ih.shape[0])
    db_hh = np.zeros(W_hh.shape[0])
    dGi_all = np.zeros((T, B, 3 * H))
    dGh_all = np.zeros((T, B, 3 * H))
    L = fw["lengths"]
    A = fw.get("att")
    datt = None if A is None else np.zeros((T, B))
    for t in reversed(list(_steps(T, reverse))):
        m = (t < L)[:, None]
        first = _first(t, L, T, reverse)
        h_prev = _prev(fw["y"], t, first, h0, reverse)
        r, u, c = fw["r"][t], fw["u"][t], fw["c"][t]
        s = 1.0 if A is None else (1 - A[t][:, None])   # update-gate scale
        ua = s * u
        dh = dy[t] + carry
        d_c = dh * (1 - ua) * (1 - c * c)
        d_ua = dh * (h_prev - c)                  # gradient wrt the scaled gate
        d_u = d_ua * s * u * (1 - u)
        if A is not None:
            datt[t] = np.where(m[:, 0], -(d_ua * u).sum(axis=1), 0.0)
        dGi = np.zeros((B, 3 * H))
        dGh = np.zeros((B, 3 * H))
        if ra:
            d_r = d_c * fw["nh"][t] * r * (1 - r)
            dGi[:, sr], dGi[:, su], dGi[:, sc] = d_r, d_u, d_c
            dGh[:, sr], dGh[:, su], dGh[:, sc] = d_r, d_u, d_c * r
            dGi, dGh = np.where(m, dGi, 0.0), np.where(m, dGh, 0.0)
            carry = np.where(m, dGh @ W_hh + dh * ua, carry)
            dW_hh += dGh.T @ h_prev
        else:
            d_rh = d_c @ W_hh[sc]                 # gradient wrt r*h_prev
            d_r = d_rh * h_prev * r * (1 - r)
            dGi[:, sr], dGi[:, su], dGi[:, sc] = d_r, d_u, d_c
            dGi = np.where(m, dGi, 0.0)
            dGh[:] = dGi
            carry = np.where(m, d_rh * r + dh * ua + dGh[:, sr] @ W_hh[sr] + dGh[:, su] @ W_hh[su], carry)
            dW_hh[sr] += dGh[:, sr].T @ h_prev
            dW_hh[su] += dGh[:, su].T @ h_prev
            dW_hh[sc] += dGh[:, sc].T @ fw["rh"][t]
        dGi_all[t], dGh_all[t] = dGi, dGh
        dx[t] = dGi @ W_ih
        dW_ih += dGi.T @ x[t]
        db_ih += dGi.sum(axis=0)
        db_hh += dGh.sum(axis=0)
    out = dict(dx=dx, dh0=carry, dW_ih=dW_ih, dW_hh=dW_hh, db_ih=db_ih,
               db_hh=db_hh, dGi=dGi_all, dGh=dGh_all)
    if datt is not None:
        out["datt"] = datt
    return out


# ------------------------------------------------------ layer wrappers ----

def layer_forward(mode, x, h0, c0, p, order, reverse=False, reset_after=True, lengths=None, att=None):
    """One layer and direction; p has W_ih, W_hh, b_ih, b_hh; att (GRU
    only) the AUGRU attention scores [T, B]."""
    if mode == "lstm":
        assert att is None, "attention scores apply to the GRU only"
        return lstm_forward(x, h0, c0, p.W_ih, p.W_hh, p.b_ih, p.b_hh, order, reverse, lengths)
    return gru_forward(x, h0, p.W_ih, p.W_hh, p.b_ih, p.b_hh, reset_after, order, reverse, lengths, att)


def layer_backward(mode, fw, dy, dhT=None, dcT=None):
    if mode == "lstm":
        return lstm_backward(fw, dy, dhT, dcT)
    return gru_backward(fw, dy, dhT)


def stack_forward(mode, x, params, order, bidir, reset_after=True, h0=None, c0=None, lengths=None):
    """Stacked (optionally bidirectional) layers: layer l+1 reads the
    concatenation [y_fwd, y_rev] of layer l along the feature axis (the
    strided-output layout of the CUDA fragment's OUTPUT_STRIDE rows).
    h0/c0 apply to every layer and direction (None = zero)."""
    recs = []
    inp = _f64(x)
    for layer_params in params:
        fws = [layer_forward(mode, inp, h0, c0, p, order, reverse=(d == 1), reset_after=reset_after,
                             lengths=lengths) for d, p in enumerate(layer_params)]
        recs.append(fws)
        inp = np.concatenate([fw["y"] for fw in fws], axis=2)
        if not bidir:
            assert len(fws) == 1
    return recs, inp


def stack_backward(mode, recs, dy):
    """BPTT through the stack built by stack_forward; returns per layer and
    direction the gradient dicts, and dx of the first layer."""
    grads = [None] * len(recs)
    d_out = _f64(dy)
    for li in range(len(recs) - 1, -1, -1):
        fws = recs[li]
        H = fws[0]["W_hh"].shape[1]
        gl = [layer_backward(mode, fw, d_out[:, :, d * H:(d + 1) * H]) for d, fw in enumerate(fws)]
        grads[li] = gl
        d_out = sum(g["dx"] for g in gl)
    return grads, d_out


def rel_err(got, ref):
    """max_i |got_i - ref_i| / max_i |ref_i| over one tensor (0 when both are
    all-zero; the plain max|got - ref| when only the reference is).

    The tolerance metric of the parity tests (the pages give none; tanh
    outputs cross zero, so an element-wise relative error is not used).
    Shapes must match exactly (no broadcasting), and a NaN or infinity in
    either operand gives NaN, so that a comparison `err <= tol` fails."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise ValueError(f"rel_err: shape {got.shape} != reference shape {ref.shape}")
    if ref.size == 0:
        return 0.0
    if not (np.all(np.isfinite(got)) and np.all(np.isfinite(ref))):
        return float("nan")
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(got - ref)))
    if den == 0.0:
        return num
    return num / den


def rel_err_l2(got, ref):
    """Norm-wise companion of rel_err: ||got - ref||_2 / ||ref||_2 (same
    shape rule, NaN for non-finite input)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise ValueError(f"rel_err_l2: shape {got.shape} != reference shape {ref.shape}")
    if ref.size == 0:
        return 0.0
    if not (np.all(np.isfinite(got)) and np.all(np.isfinite(ref))):
        return float("nan")
    den = float(np.linalg.norm(ref.ravel()))
    num = float(np.linalg.norm((got - ref).ravel()))
    return num if den == 0.0 else num / den
