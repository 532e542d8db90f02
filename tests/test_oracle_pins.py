"""Pins of the CPU oracle against facts that do not come from the oracle.

* hand-worked single-step values (tests/golden/h1_cells.json);
* library special cases: torch's CPU nn.LSTM (gate order i,f,g,o, biases
  b_ih + b_hh) and nn.GRU (which is the reset-after GRU with order r,u,c),
  run in float64 with autograd for the gradients, including torch's
  bidirectional and two-layer stacking;
* central finite differences of a scalar loss for every gradient, which pins
  the backward recurrences to the forward ones (this is the main pin of the
  basic GRU, which torch does not implement);
* invariants named by the method: forget=1/input=0 keeps c, update=1 copies
  h, reverse direction = forward on the reversed sequence, storage order is a
  pure relabelling, the two GRU variants coincide when r is 1, gradients are
  linear in the upstream gradient, and the bias-gradient identities.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden", "h1_cells.json")


def _rng(seed=0):
    return np.random.Generator(np.random.PCG64(seed))


def _params(rng, G, H, I, k=0.5):
    return (rng.uniform(-k, k, (G * H, I)), rng.uniform(-k, k, (G * H, H)),
            rng.uniform(-k, k, G * H), rng.uniform(-k, k, G * H))


# ------------------------------------------------------------ H=1 values --

def _named(d, names):
    return np.array([[d[n]] for n in names])


@pytest.mark.parametrize("order", [(0, 1, 2, 3), (1, 0, 2, 3), (3, 2, 1, 0)])
def test_lstm_h1_worked_values(order):
    g = json.load(open(GOLD))["lstm"]
    names = "ifgo"
    sto = [names[k] for k in order]
    W_ih, W_hh = _named(g["W_ih"], sto), _named(g["W_hh"], sto)
    b_ih, b_hh = _named(g["b_ih"], sto)[:, 0], _named(g["b_hh"], sto)[:, 0]
    x, h0, c0 = np.ones((1, 1, 1)), np.array([[0.5]]), np.array([[0.25]])
    fw = O.lstm_forward(x, h0, c0, W_ih, W_hh, b_ih, b_hh, order)
    e = g["expect"]
    for k in "ifgo":
        assert fw[k][0, 0, 0] == pytest.approx(e[k], abs=1e-11)
    assert fw["cT"][0, 0] == pytest.approx(e["c1"], abs=1e-11)
    assert fw["hT"][0, 0] == pytest.approx(e["h1"], abs=1e-11)
    gr = O.lstm_backward(fw, np.ones((1, 1, 1)))
    for slot, k in enumerate(sto):
        assert gr["dG"][0, 0, slot] == pytest.approx(e["dG"][k], abs=1e-11)
        assert gr["dW_ih"][slot, 0] == pytest.approx(e["dG"][k], abs=1e-11)
        assert gr["dW_hh"][slot, 0] == pytest.approx(0.5 * e["dG"][k], abs=1e-11)
        assert gr["db_ih"][slot] == pytest.approx(e["dG"][k], abs=1e-11)
    for k in ("dx", "dh0", "dc0"):
        assert np.ravel(gr[k])[0] == pytest.approx(e[k], abs=1e-11)


@pytest.mark.parametrize("reset_after", [False, True])
@pytest.mark.parametrize("order", [(0, 1, 2), (2, 0, 1)])
def test_gru_h1_worked_values(reset_after, order):
    g = json.load(open(GOLD))["gru"]
    names = "ruc"
    sto = [names[k] for k in order]
    W_ih, W_hh = _named(g["W_ih"], sto), _named(g["W_hh"], sto)
    b_ih, b_hh = _named(g["b_ih"], sto)[:, 0], _named(g["b_hh"], sto)[:, 0]
    x, h0 = np.ones((1, 1, 1)), np.array([[0.5]])
    fw = O.gru_forward(x, h0, W_ih, W_hh, b_ih, b_hh, reset_after, order)
    e = g["reset_after" if reset_after else "basic"]
    assert fw["c"][0, 0, 0] == pytest.approx(e["c"], abs=1e-11)
    assert fw["hT"][0, 0] == pytest.approx(e["h1"], abs=1e-11)
    if reset_after:
        assert fw["nh"][0, 0, 0] == pytest.approx(e["n_h"], abs=1e-11)
    gr = O.gru_backward(fw, np.ones((1, 1, 1)))
    for slot, k in enumerate(sto):
        assert gr["dGi"][0, 0, slot] == pytest.approx(e["dG"][k], abs=1e-11)
    cs = sto.index("c")
    assert gr["db_hh"][cs] == pytest.approx(e["db_hh_c"], abs=1e-11)
    assert gr["dW_hh"][cs, 0] == pytest.approx(e["dW_hh_c"], abs=1e-11)
    assert np.ravel(gr["dx"])[0] == pytest.approx(e["dx"], abs=1e-11)
    assert np.ravel(gr["dh0"])[0] == pytest.approx(e["dh0"], abs=1e-11)


# ------------------------------------------------- torch library routines --

def _torch_run(module, x, h0, c0, gy, ghT, gcT):
    xt = torch.tensor(x, requires_grad=True)
    h0t = torch.tensor(h0, requires_grad=True)
    if c0 is not None:
        c0t = torch.tensor(c0, requires_grad=True)
        y, (hT, cT) = module(xt, (h0t, c0t))
        loss = (y * torch.tensor(gy)).sum() + (hT * torch.tensor(ghT)).sum() + (cT * torch.tensor(gcT)).sum()
    else:
        c0t = None
        y, hT = module(xt, h0t)
        cT = None
        loss = (y * torch.tensor(gy)).sum() + (hT * torch.tensor(ghT)).sum()
    loss.backward()
    return dict(y=y.detach().numpy(), hT=hT.detach().numpy(),
                cT=None if cT is None else cT.detach().numpy(),
                dx=xt.grad.numpy(), dh0=h0t.grad.numpy(),
                dc0=None if c0t is None else c0t.grad.numpy())


def _grads_of(module, name):
    return {n: p.grad.numpy() for n, p in module.named_parameters() if n.endswith(name)}


@pytest.mark.parametrize("bidir", [False, True])
def test_lstm_matches_torch_lstm(bidir):
    rng = _rng(1)
    T, B, I, H = 5, 3, 4, 6
    dirs = 2 if bidir else 1
    m = torch.nn.LSTM(I, H, bidirectional=bidir).double()
    x = rng.standard_normal((T, B, I))
    h0 = rng.standard_normal((dirs, B, H))
    c0 = rng.standard_normal((dirs, B, H))
    gy = rng.standard_normal((T, B, dirs * H))
    ghT = rng.standard_normal((dirs, B, H))
    gcT = rng.standard_normal((dirs, B, H))
    ref = _torch_run(m, x, h0, c0, gy, ghT, gcT)
    dx = np.zeros_like(x)
    for d in range(dirs):
        sfx = "_l0" + ("_reverse" if d else "")
        P = [getattr(m, n + sfx).detach().numpy() for n in ("weight_ih", "weight_hh", "bias_ih", "bias_hh")]
        fw = O.lstm_forward(x, h0[d], c0[d], *P, order=(0, 1, 2, 3), reverse=bool(d))
        np.testing.assert_allclose(fw["y"], ref["y"][:, :, d * H:(d + 1) * H], atol=1e-12)
        np.testing.assert_allclose(fw["hT"], ref["hT"][d], atol=1e-12)
        np.testing.assert_allclose(fw["cT"], ref["cT"][d], atol=1e-12)
        gr = O.lstm_backward(fw, gy[:, :, d * H:(d + 1) * H], ghT[d], gcT[d])
        np.testing.assert_allclose(gr["dh0"], ref["dh0"][d], atol=1e-11)
        np.testing.assert_allclose(gr["dc0"], ref["dc0"][d], atol=1e-11)
        for ours, theirs in (("dW_ih", "weight_ih"), ("dW_hh", "weight_hh"), ("db_ih", "bias_ih"), ("db_hh", "bias_hh")):
            np.testing.assert_allclose(gr[ours], getattr(m, theirs + sfx).grad.numpy(), atol=1e-11)
        dx += gr["dx"]
    np.testing.assert_allclose(dx, ref["dx"], atol=1e-11)


@pytest.mark.parametrize("bidir", [False, True])
def test_grura_matches_torch_gru(bidir):
    rng = _rng(2)
    T, B, I, H = 6, 2, 3, 5
    dirs = 2 if bidir else 1
    m = torch.nn.GRU(I, H, bidirectional=bidir).double()
    x = rng.standard_normal((T, B, I))
    h0 = rng.standard_normal((dirs, B, H))
    gy = rng.standard_normal((T, B, dirs * H))
    ghT = rng.standard_normal((dirs, B, H))
    ref = _torch_run(m, x, h0, None, gy, ghT, None)
    dx = np.zeros_like(x)
    for d in range(dirs):
        sfx = "_l0" + ("_reverse" if d else "")
        P = [getattr(m, n + sfx).detach().numpy() for n in ("weight_ih", "weight_hh", "bias_ih", "bias_hh")]
        fw = O.gru_forward(x, h0[d], *P, reset_after=True, order=(0, 1, 2), reverse=bool(d))
        np.testing.assert_allclose(fw["y"], ref["y"][:, :, d * H:(d + 1) * H], atol=1e-12)
        np.testing.assert_allclose(fw["hT"], ref["hT"][d], atol=1e-12)
        gr = O.gru_backward(fw, gy[:, :, d * H:(d + 1) * H], ghT[d])
        np.testing.assert_allclose(gr["dh0"], ref["dh0"][d], atol=1e-11)
        for ours, theirs in (("dW_ih", "weight_ih"), ("dW_hh", "weight_hh"), ("db_ih", "bias_ih"), ("db_hh", "bias_hh")):
            np.testing.assert_allclose(gr[ours], getattr(m, theirs + sfx).grad.numpy(), atol=1e-11)
        dx += gr["dx"]
    np.testing.assert_allclose(dx, ref["dx"], atol=1e-11)


def test_two_layer_bidir_stack_matches_torch():
    """Stacking: layer 2 reads [y_fwd, y_rev]; gradients split back."""
    rng = _rng(3)
    T, B, I, H = 4, 2, 3, 4
    m = torch.nn.LSTM(I, H, num_layers=2, bidirectional=True).double()
    x = rng.standard_normal((T, B, I))
    gy = rng.standard_normal((T, B, 2 * H))
    xt = torch.tensor(x, requires_grad=True)
    y, _ = m(xt)
    (y * torch.tensor(gy)).sum().backward()

    class P:
        pass

    params = []
    for layer in range(2):
        per = []
        for d in range(2):
            sfx = f"_l{layer}" + ("_reverse" if d else "")
            p = P()
            p.W_ih, p.W_hh, p.b_ih, p.b_hh = (getattr(m, n + sfx).detach().numpy()
                                              for n in ("weight_ih", "weight_hh", "bias_ih", "bias_hh"))
            per.append(p)
        params.append(per)
    recs, yo = O.stack_forward("lstm", x, params, (0, 1, 2, 3), bidir=True)
    np.testing.assert_allclose(yo, y.detach().numpy(), atol=1e-12)
    grads, dx = O.stack_backward("lstm", recs, gy)
    np.testing.assert_allclose(dx, xt.grad.numpy(), atol=1e-11)
    for layer in range(2):
        for d in range(2):
            sfx = f"_l{layer}" + ("_reverse" if d else "")
            np.testing.assert_allclose(grads[layer][d]["dW_hh"], getattr(m, "weight_hh" + sfx).grad.numpy(), atol=1e-11)
            np.testing.assert_allclose(grads[layer][d]["dW_ih"], getattr(m, "weight_ih" + sfx).grad.numpy(), atol=1e-11)


# --------------------------------------------------- finite differences --

def _loss(mode, ra, order, rev, x, h0, c0, P, gy, ghT, gcT):
    if mode == "lstm":
        fw = O.lstm_forward(x, h0, c0, *P, order=order, reverse=rev)
        return (fw["y"] * gy).sum() + (fw["hT"] * ghT).sum() + (fw["cT"] * gcT).sum()
    fw = O.gru_forward(x, h0, *P, reset_after=ra, order=order, reverse=rev)
    return (fw["y"] * gy).sum() + (fw["hT"] * ghT).sum()


@pytest.mark.parametrize("case", [
    ("lstm", None, (0, 1, 2, 3), False, 8, 2, 16, 32),
    ("lstm", None, (1, 0, 2, 3), True, 4, 2, 3, 5),
    ("gru", False, (0, 1, 2), False, 4, 2, 3, 5),
    ("gru", False, (1, 2, 0), True, 4, 2, 3, 5),
    ("gru", True, (0, 1, 2), False, 4, 2, 3, 5),
    ("gru", True, (2, 1, 0), True, 4, 2, 3, 5),
])
def test_finite_differences(case):
    mode, ra, order, rev, T, B, I, H = case
    rng = _rng(4)
    G = 4 if mode == "lstm" else 3
    P = list(_params(rng, G, H, I, k=1 / np.sqrt(H) if H > 8 else 0.5))
    x = rng.standard_normal((T, B, I))
    h0 = rng.standard_normal((B, H))
    c0 = rng.standard_normal((B, H)) if mode == "lstm" else None
    gy = rng.standard_normal((T, B, H))
    ghT = rng.standard_normal((B, H))
    gcT = rng.standard_normal((B, H)) if mode == "lstm" else None
    if mode == "lstm":
        fw = O.lstm_forward(x, h0, c0, *P, order=order, reverse=rev)
        gr = O.lstm_backward(fw, gy, ghT, gcT)
    else:
        fw = O.gru_forward(x, h0, *P, reset_after=ra, order=order, reverse=rev)
        gr = O.gru_backward(fw, gy, ghT)
    targets = {"dx": x, "dh0": h0, "dW_ih": P[0], "dW_hh": P[1], "db_ih": P[2], "db_hh": P[3]}
    if mode == "lstm":
        targets["dc0"] = c0
    eps = 1e-6
    pick = _rng(5)
    for name, arr in targets.items():
        flat = arr.reshape(-1)
        idx = pick.choice(flat.size, size=min(flat.size, 24), replace=False)
        for j in idx:
            old = flat[j]
            flat[j] = old + eps
            lp = _loss(mode, ra, order, rev, x, h0, c0, P, gy, ghT, gcT)
            flat[j] = old - eps
            lm = _loss(mode, ra, order, rev, x, h0, c0, P, gy, ghT, gcT)
            flat[j] = old
            fd = (lp - lm) / (2 * eps)
            an = gr[name].reshape(-1)[j]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, j, fd, an)


# ------------------------------------------------------------ invariants --

def test_lstm_forget_one_input_zero_keeps_cell():
    rng = _rng(6)
    T, B, I, H = 7, 3, 4, 5
    W_ih, W_hh, b_ih, b_hh = _params(rng, 4, H, I)
    for g in (0, 1):                       # input and forget rows (order i,f,g,o)
        W_ih[g * H:(g + 1) * H] = 0
        W_hh[g * H:(g + 1) * H] = 0
        b_hh[g * H:(g + 1) * H] = 0
    b_ih[0:H] = -30.0
    b_ih[H:2 * H] = 30.0
    c0 = rng.standard_normal((B, H))
    fw = O.lstm_forward(rng.standard_normal((T, B, I)), rng.standard_normal((B, H)), c0,
                        W_ih, W_hh, b_ih, b_hh)
    for t in range(T):
        np.testing.assert_allclose(fw["c"][t], c0, atol=1e-11)
    np.testing.assert_allclose(fw["y"], fw["o"] * np.tanh(c0)[None], atol=1e-11)


@pytest.mark.parametrize("reset_after", [False, True])
def test_gru_update_one_copies_h(reset_after):
    rng = _rng(7)
    T, B, I, H = 6, 2, 3, 4
    W_ih, W_hh, b_ih, b_hh = _params(rng, 3, H, I)
    W_ih[H:2 * H] = 0
    W_hh[H:2 * H] = 0
    b_ih[H:2 * H] = 30.0
    b_hh[H:2 * H] = 0
    h0 = rng.standard_normal((B, H))
    fw = O.gru_forward(rng.standard_normal((T, B, I)), h0, W_ih, W_hh, b_ih, b_hh, reset_after)
    for t in range(T):
        np.testing.assert_allclose(fw["y"][t], h0, atol=1e-11)


def test_gru_variants_coincide_when_reset_is_one():
    rng = _rng(8)
    T, B, I, H = 6, 2, 3, 4
    W_ih, W_hh, b_ih, b_hh = _params(rng, 3, H, I)
    W_ih[0:H] = 0
    W_hh[0:H] = 0
    b_ih[0:H] = 40.0
    b_hh[0:H] = 0
    b_hh[2 * H:] = 0
    x, h0 = rng.standard_normal((T, B, I)), rng.standard_normal((B, H))
    a = O.gru_forward(x, h0, W_ih, W_hh, b_ih, b_hh, False)
    b = O.gru_forward(x, h0, W_ih, W_hh, b_ih, b_hh, True)
    np.testing.assert_allclose(a["y"], b["y"], atol=1e-12)
    gy = rng.standard_normal((T, B, H))
    ga, gb = O.gru_backward(a, gy), O.gru_backward(b, gy)
    for k in ("dx", "dh0", "dW_ih", "dW_hh"):
        np.testing.assert_allclose(ga[k], gb[k], atol=1e-10)


def _rev_case(mode, ra, seed):
    rng = _rng(seed)
    T, B, I, H = 5, 2, 3, 4
    G = 4 if mode == "lstm" else 3
    P = _params(rng, G, H, I)
    x = rng.standard_normal((T, B, I))
    h0 = rng.standard_normal((B, H))
    c0 = rng.standard_normal((B, H))
    gy = rng.standard_normal((T, B, H))
    return P, x, h0, c0, gy


@pytest.mark.parametrize("mode,ra", [("lstm", None), ("gru", False), ("gru", True)])
def test_reverse_equals_forward_on_reversed_input(mode, ra):
    P, x, h0, c0, gy = _rev_case(mode, ra, 9)
    f = O.layer_forward(mode, x, h0, c0, _P(P), (0, 1, 2, 3) if mode == "lstm" else (0, 1, 2), False, ra)
    r = O.layer_forward(mode, x[::-1].copy(), h0, c0, _P(P), (0, 1, 2, 3) if mode == "lstm" else (0, 1, 2), True, ra)
    np.testing.assert_allclose(r["y"][::-1], f["y"], atol=1e-13)
    np.testing.assert_allclose(r["hT"], f["hT"], atol=1e-13)
    gf = O.layer_backward(mode, f, gy)
    gr = O.layer_backward(mode, r, gy[::-1].copy())
    np.testing.assert_allclose(gr["dx"][::-1], gf["dx"], atol=1e-12)
    for k in ("dh0", "dW_ih", "dW_hh", "db_ih", "db_hh"):
        np.testing.assert_allclose(gr[k], gf[k], atol=1e-12)


class _P:
    def __init__(self, P):
        self.W_ih, self.W_hh, self.b_ih, self.b_hh = P


@pytest.mark.parametrize("mode,ra,perm", [("lstm", None, (3, 1, 0, 2)), ("gru", False, (2, 0, 1)), ("gru", True, (1, 2, 0))])
def test_storage_order_is_a_relabelling(mode, ra, perm):
    """Same named gates stored in another row-block order give the same
    outputs, and gradients permuted the same way."""
    P, x, h0, c0, gy = _rev_case(mode, ra, 10)
    G = len(perm)
    H = P[1].shape[1]
    ident = tuple(range(G))

    def permute(a):                       # block k of the result = block perm[k] of a
        return np.concatenate([a[p * H:(p + 1) * H] for p in perm], axis=0)

    Pp = tuple(permute(a) for a in P)
    a = O.layer_forward(mode, x, h0, c0, _P(P), ident, False, ra)
    b = O.layer_forward(mode, x, h0, c0, _P(Pp), perm, False, ra)
    np.testing.assert_allclose(a["y"], b["y"], atol=1e-13)
    ga, gb = O.layer_backward(mode, a, gy), O.layer_backward(mode, b, gy)
    np.testing.assert_allclose(ga["dx"], gb["dx"], atol=1e-12)
    for k in ("dW_ih", "dW_hh", "db_ih", "db_hh"):
        np.testing.assert_allclose(permute(ga[k]), gb[k], atol=1e-12)


@pytest.mark.parametrize("mode,ra", [("lstm", None), ("gru", False), ("gru", True)])
def test_backward_is_linear_in_upstream_gradient(mode, ra):
    P, x, h0, c0, gy = _rev_case(mode, ra, 11)
    order = (0, 1, 2, 3) if mode == "lstm" else (0, 1, 2)
    f = O.layer_forward(mode, x, h0, c0, _P(P), order, False, ra)
    g1 = O.layer_backward(mode, f, gy)
    g2 = O.layer_backward(mode, f, -2.5 * gy)
    for k in ("dx", "dh0", "dW_ih", "dW_hh", "db_ih", "db_hh"):
        np.testing.assert_allclose(g2[k], -2.5 * g1[k], atol=1e-12, rtol=1e-12)


@pytest.mark.parametrize("mode,ra", [("lstm", None), ("gru", False), ("gru", True)])
def test_bias_gradient_identities(mode, ra):
    P, x, h0, c0, gy = _rev_case(mode, ra, 12)
    order = (0, 1, 2, 3) if mode == "lstm" else (0, 1, 2)
    H = P[1].shape[1]
    f = O.layer_forward(mode, x, h0, c0, _P(P), order, False, ra)
    g = O.layer_backward(mode, f, gy)
    if mode == "lstm" or not ra:
        np.testing.assert_array_equal(g["db_ih"], g["db_hh"])
    else:
        np.testing.assert_array_equal(g["db_ih"][:2 * H], g["db_hh"][:2 * H])
        # the recurrent candidate bias sees d_c * r
        assert not np.allclose(g["db_ih"][2 * H:], g["db_hh"][2 * H:])


def test_zero_recurrent_weights_reduce_to_independent_steps():
    """W_hh = 0 and h0 = 0: every step is the T=1 case on its own input."""
    rng = _rng(13)
    T, B, I, H = 4, 3, 5, 6
    W_ih, W_hh, b_ih, b_hh = _params(rng, 4, H, I)
    W_hh[:] = 0
    x = rng.standard_normal((T, B, I))
    f = O.lstm_forward(x, None, None, W_ih, W_hh, b_ih, b_hh)
    for t in range(T):
        z = x[t] @ W_ih.T + b_ih + b_hh
        i, fg, g, o = (z[:, k * H:(k + 1) * H] for k in range(4))
        i, fg, o = 1 / (1 + np.exp(-i)), 1 / (1 + np.exp(-fg)), 1 / (1 + np.exp(-o))
        c_prev = np.zeros((B, H)) if t == 0 else f["c"][t - 1]
        np.testing.assert_allclose(f["c"][t], fg * c_prev + i * np.tanh(g), atol=1e-13)


# ------------------------------------------------- variable sequence lengths --
# Reading (popnn's per-batch step limits): steps past a row's length output
# zero, keep the state and pass the carried gradients through; a reverse
# direction row starts at its own last step. torch's packed sequences define
# the same thing independently: outputs zero-padded, h_n/c_n the state at the
# row's last valid step, the reverse direction starting at each row's end.

def _torch_packed(module, x, lengths, h0, c0, gy, ghT, gcT):
    from torch.nn.utils.rnn import pack_padded_sequence, pad_packed_sequence
    xt = torch.tensor(x, requires_grad=True)
    h0t = torch.tensor(h0, requires_grad=True)
    packed = pack_padded_sequence(xt, torch.tensor(lengths), enforce_sorted=False)
    if c0 is not None:
        c0t = torch.tensor(c0, requires_grad=True)
        out, (hT, cT) = module(packed, (h0t, c0t))
    else:
        c0t, cT = None, None
        out, hT = module(packed, h0t)
    y, _ = pad_packed_sequence(out, total_length=x.shape[0])
    loss = (y * torch.tensor(gy)).sum() + (hT * torch.tensor(ghT)).sum()
    if cT is not None:
        loss = loss + (cT * torch.tensor(gcT)).sum()
    loss.backward()
    return dict(y=y.detach().numpy(), hT=hT.detach().numpy(), cT=None if cT is None else cT.detach().numpy(),
                dx=xt.grad.numpy(), dh0=h0t.grad.numpy(), dc0=None if c0t is None else c0t.grad.numpy())


@pytest.mark.parametrize("mode", ["lstm", "gru"])
@pytest.mark.parametrize("bidir", [False, True])
def test_variable_lengths_match_torch_packed_sequences(mode, bidir):
    rng = _rng(11)
    T, B, I, H = 7, 5, 3, 4
    lengths = [7, 3, 1, 5, 6]
    dirs = 2 if bidir else 1
    m = (torch.nn.LSTM if mode == "lstm" else torch.nn.GRU)(I, H, bidirectional=bidir).double()
    x = rng.standard_normal((T, B, I))
    h0 = rng.standard_normal((dirs, B, H))
    c0 = rng.standard_normal((dirs, B, H)) if mode == "lstm" else None
    gy = rng.standard_normal((T, B, dirs * H))
    ghT = rng.standard_normal((dirs, B, H))
    gcT = rng.standard_normal((dirs, B, H))
    ref = _torch_packed(m, x, lengths, h0, c0, gy, ghT, gcT)
    dx = np.zeros_like(x)
    for d in range(dirs):
        sfx = "_l0" + ("_reverse" if d else "")
        P = [getattr(m, n + sfx).detach().numpy() for n in ("weight_ih", "weight_hh", "bias_ih", "bias_hh")]
        if mode == "lstm":
            fw = O.lstm_forward(x, h0[d], c0[d], *P, order=(0, 1, 2, 3), reverse=bool(d), lengths=lengths)
            gr = O.lstm_backward(fw, gy[:, :, d * H:(d + 1) * H], ghT[d], gcT[d])
            np.testing.assert_allclose(fw["cT"], ref["cT"][d], atol=1e-12)
            np.testing.assert_allclose(gr["dc0"], ref["dc0"][d], atol=1e-11)
        else:
            fw = O.gru_forward(x, h0[d], *P, reset_after=True, order=(0, 1, 2), reverse=bool(d), lengths=lengths)
            gr = O.gru_backward(fw, gy[:, :, d * H:(d + 1) * H], ghT[d])
        np.testing.assert_allclose(fw["y"], ref["y"][:, :, d * H:(d + 1) * H], atol=1e-12)
        np.testing.assert_allclose(fw["hT"], ref["hT"][d], atol=1e-12)
        np.testing.assert_allclose(gr["dh0"], ref["dh0"][d], atol=1e-11)
        for ours, theirs in (("dW_ih", "weight_ih"), ("dW_hh", "weight_hh"), ("db_ih", "bias_ih"), ("db_hh", "bias_hh")):
            np.testing.assert_allclose(gr[ours], getattr(m, theirs + sfx).grad.numpy(), atol=1e-11)
        dx += gr["dx"]
    np.testing.assert_allclose(dx, ref["dx"], atol=1e-11)


@pytest.mark.parametrize("mode,ra", [("lstm", None), ("gru", False), ("gru", True)])
@pytest.mark.parametrize("reverse", [False, True])
def test_variable_lengths_equal_truncated_sequences(mode, ra, reverse):
    """Every row equals the fixed-length recurrence over its own first
    lengths[b] steps (zero steps: outputs zero, state and gradients pass
    through); the weight gradients are the sums of those runs."""
    rng = _rng(12)
    T, B, I, H = 6, 4, 3, 5
    G = 4 if mode == "lstm" else 3
    lengths = np.array([6, 2, 0, 4])
    W_ih, W_hh, b_ih, b_hh = _params(rng, G, H, I)

    class P:
        pass
    p = P()
    p.W_ih, p.W_hh, p.b_ih, p.b_hh = W_ih, W_hh, b_ih, b_hh
    order = (0, 1, 2, 3) if mode == "lstm" else (0, 1, 2)
    x = rng.standard_normal((T, B, I))
    h0 = rng.standard_normal((B, H))
    c0 = rng.standard_normal((B, H)) if mode == "lstm" else None
    dy = rng.standard_normal((T, B, H))
    dhT = rng.standard_normal((B, H))
    dcT = rng.standard_normal((B, H)) if mode == "lstm" else None
    fw = O.layer_forward(mode, x, h0, c0, p, order, reverse, bool(ra), lengths=lengths)
    gr = O.layer_backward(mode, fw, dy, dhT, dcT)
    acc = {k: np.zeros_like(gr[k]) for k in ("dW_ih", "dW_hh", "db_ih", "db_hh")}
    for b, L in enumerate(lengths):
        sub = lambda a: None if a is None else a[b:b + 1]  # noqa: E731
        if L == 0:
            np.testing.assert_array_equal(fw["y"][:, b], 0.0)
            np.testing.assert_array_equal(fw["hT"][b], h0[b])
            np.testing.assert_array_equal(gr["dh0"][b], dhT[b])
            np.testing.assert_array_equal(gr["dx"][:, b], 0.0)
            if mode == "lstm":
                np.testing.assert_array_equal(fw["cT"][b], c0[b])
                np.testing.assert_array_equal(gr["dc0"][b], dcT[b])
            continue
        fr = O.layer_forward(mode, x[:L, b:b + 1], sub(h0), sub(c0), p, order, reverse, bool(ra))
        rr = O.layer_backward(mode, fr, dy[:L, b:b + 1], sub(dhT), sub(dcT))
        np.testing.assert_allclose(fw["y"][:L, b], fr["y"][:, 0], atol=1e-13)
        np.testing.assert_array_equal(fw["y"][L:, b], 0.0)
        np.testing.assert_allclose(fw["hT"][b], fr["hT"][0], atol=1e-13)
        np.testing.assert_allclose(gr["dx"][:L, b], rr["dx"][:, 0], atol=1e-12)
        np.testing.assert_array_equal(gr["dx"][L:, b], 0.0)
        np.testing.assert_allclose(gr["dh0"][b], rr["dh0"][0], atol=1e-12)
        if mode == "lstm":
            np.testing.assert_allclose(fw["cT"][b], fr["cT"][0], atol=1e-13)
            np.testing.assert_allclose(gr["dc0"][b], rr["dc0"][0], atol=1e-12)
        for k in acc:
            acc[k] += rr[k]
    for k in acc:
        np.testing.assert_allclose(gr[k], acc[k], atol=1e-11)


def test_full_lengths_equal_no_lengths():
    rng = _rng(13)
    T, B, I, H = 5, 3, 2, 4
    W = _params(rng, 4, H, I)
    x = rng.standard_normal((T, B, I))
    a = O.lstm_forward(x, None, None, *W, reverse=True)
    b = O.lstm_forward(x, None, None, *W, reverse=True, lengths=[T] * B)
    for k in ("y", "hT", "cT", "c"):
        np.testing.assert_array_equal(a[k], b[k])


# ---------------------------------------------------------------- AUGRU --
# The attention-scaled update gate ua = (1 - a) u has no library routine to
# compare with; it is pinned by the two ends of the score range (a = 0 is the
# GRU, itself pinned above; a = 1 closes the update gate, which a GRU with
# the gate forced shut reproduces) and by finite differences of every
# gradient, the score gradient included.

def _augru_case(seed, T=5, B=3, I=4, H=6):
    rng = _rng(seed)
    P = list(_params(rng, 3, H, I))
    x = rng.standard_normal((T, B, I))
    h0 = rng.standard_normal((B, H))
    att = rng.uniform(0.0, 1.0, (T, B))
    gy = rng.standard_normal((T, B, H))
    ghT = rng.standard_normal((B, H))
    return P, x, h0, att, gy, ghT


@pytest.mark.parametrize("ra", [False, True])
@pytest.mark.parametrize("rev", [False, True])
def test_augru_zero_scores_are_the_gru(ra, rev):
    P, x, h0, att, gy, ghT = _augru_case(21)
    fa = O.gru_forward(x, h0, *P, reset_after=ra, reverse=rev, att=np.zeros_like(att))
    fg = O.gru_forward(x, h0, *P, reset_after=ra, reverse=rev)
    ga, gg = O.gru_backward(fa, gy, ghT), O.gru_backward(fg, gy, ghT)
    for k in ("y", "hT"):
        np.testing.assert_array_equal(fa[k], fg[k])
    for k in ("dx", "dh0", "dW_ih", "dW_hh", "db_ih", "db_hh"):
        np.testing.assert_array_equal(ga[k], gg[k])
    assert ga["datt"].shape == att.shape and "datt" not in gg


@pytest.mark.parametrize("ra", [False, True])
def test_augru_unit_scores_replace_the_state_by_the_candidate(ra):
    P, x, h0, att, gy, ghT = _augru_case(22)
    H = h0.shape[1]
    fa = O.gru_forward(x, h0, *P, reset_after=ra, att=np.ones_like(att))
    np.testing.assert_allclose(fa["y"], fa["c"], rtol=0, atol=1e-15)
    # the same layer with its update gate forced shut (order r,u,c)
    Q = [a.copy() for a in P]
    Q[0][H:2 * H] = 0
    Q[1][H:2 * H] = 0
    Q[2][H:2 * H] = -60.0
    Q[3][H:2 * H] = 0
    fq = O.gru_forward(x, h0, *Q, reset_after=ra)
    np.testing.assert_allclose(fa["y"], fq["y"], rtol=0, atol=1e-12)
    ga, gq = O.gru_backward(fa, gy, ghT), O.gru_backward(fq, gy, ghT)
    keep = np.r_[0:H, 2 * H:3 * H]          # rows of r and c (u rows hold other weights)
    for k in ("dx", "dh0"):
        np.testing.assert_allclose(ga[k], gq[k], rtol=0, atol=1e-12)
    for k in ("dW_ih", "dW_hh", "db_ih", "db_hh"):
        np.testing.assert_allclose(ga[k][keep], gq[k][keep], rtol=0, atol=1e-12)
        np.testing.assert_allclose(ga[k][H:2 * H], 0.0, atol=1e-15)


def _augru_loss(ra, rev, x, h0, P, att, gy, ghT, lengths=None):
    fw = O.gru_forward(x, h0, *P, reset_after=ra, reverse=rev, lengths=lengths, att=att)
    return (fw["y"] * gy).sum() + (fw["hT"] * ghT).sum()


@pytest.mark.parametrize("ra,rev,lengths", [(False, False, None), (True, True, None),
                                            (True, False, [5, 0, 3]), (False, True, [2, 5, 4])])
def test_augru_finite_differences(ra, rev, lengths):
    P, x, h0, att, gy, ghT = _augru_case(23)
    fw = O.gru_forward(x, h0, *P, reset_after=ra, reverse=rev, lengths=lengths, att=att)
    gr = O.gru_backward(fw, gy, ghT)
    targets = {"datt": att, "dx": x, "dh0": h0, "dW_ih": P[0], "dW_hh": P[1], "db_ih": P[2], "db_hh": P[3]}
    eps = 1e-6
    pick = _rng(24)
    for name, arr in targets.items():
        flat = arr.reshape(-1)
        idx = range(flat.size) if name == "datt" else pick.choice(flat.size, size=min(flat.size, 20),
                                                                    replace=False)
        for j in idx:
            old = flat[j]
            flat[j] = old + eps
            lp = _augru_loss(ra, rev, x, h0, P, att, gy, ghT, lengths)
            flat[j] = old - eps
            lm = _augru_loss(ra, rev, x, h0, P, att, gy, ghT, lengths)
            flat[j] = old
            fd = (lp - lm) / (2 * eps)
            an = gr[name].reshape(-1)[j]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, j, fd, an)
    if lengths is not None:
        T = x.shape[0]
        for b, Lb in enumerate(lengths):
            np.testing.assert_array_equal(gr["datt"][Lb:T, b], 0.0)


# ------------------------------------------------ the tolerance metric ----
# rel_err is max_i |got_i - ref_i| / max_i |ref_i| per tensor; every parity
# assertion rests on it, so it is pinned by values worked out by hand.

def test_rel_err_hand_values():
    # |got - ref| = (0.5, 0, 0.25), max = 0.5; max |ref| = 4 -> 0.125
    assert O.rel_err([1.5, -2.0, 4.25], [1.0, -2.0, 4.0]) == 0.125
    # the denominator takes the absolute value: max |ref| = |-8| = 8
    assert O.rel_err([0.0, -7.0], [1.0, -8.0]) == 1.0 / 8.0
    # a sign flip of the largest element counts twice its size: |-4 - 4| / 4
    assert O.rel_err([1.0, -4.0], [1.0, 4.0]) == 2.0
    # exact agreement
    assert O.rel_err(np.arange(6.0).reshape(2, 3), np.arange(6.0).reshape(2, 3)) == 0.0
    # a zero reference: the absolute difference (0.5), and 0 when both are zero
    assert O.rel_err([0.5, -0.25], [0.0, 0.0]) == 0.5
    assert O.rel_err(np.zeros(4), np.zeros(4)) == 0.0
    # norm-wise companion: ||(3, 4)|| / ||(6, 8)|| = 5 / 10
    assert O.rel_err_l2([3.0, 4.0], [0.0, 0.0]) == 5.0
    assert O.rel_err_l2([9.0, 12.0], [6.0, 8.0]) == 0.5


def test_rel_err_fails_on_nan_and_infinity():
    for bad in ([1.0, np.nan, 2.0], [np.inf, 0.0, 0.0], [1.0, 1.0, -np.inf]):
        e = O.rel_err(bad, [1.0, 1.0, 2.0])
        assert np.isnan(e) and not (e <= 1e-3)
        assert np.isnan(O.rel_err([1.0, 1.0, 2.0], bad))
        assert np.isnan(O.rel_err_l2(bad, [1.0, 1.0, 2.0]))


def test_rel_err_rejects_shape_mismatch():
    with pytest.raises(ValueError):
        O.rel_err(np.ones((3, 4)), np.ones(4))
    with pytest.raises(ValueError):
        O.rel_err(np.ones((2, 3)), np.ones((3, 2)))
    with pytest.raises(ValueError):
        O.rel_err_l2(np.ones(5), np.ones(4))
