"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small and medium cases (several MFMA tiles and ragged tails); every output
element is compared. The full-size workloads are in test_gpu_full_size.py.
"""
import numpy as np
import pytest
import torch

from gru_layer_fwd_amd import synth
from rnn_harness import Params, compare, gpu_layer, oracle_layer

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _case(name, **changes):
    wl = synth.small(W[name], **changes)
    inp = synth.make_inputs(wl)
    p = inp["params"][0][0]
    return wl, inp, Params(p.W_ih, p.W_hh, p.b_ih, p.b_hh)


def _run(wl, inp, P, direction=0, order=None, dhT=None, dcT=None, lengths=None, att=None, **kw):
    mode, dt = wl.mode, wl.dtype
    ra = wl.reset_after
    got = gpu_layer(mode, dt, P, inp["x"], inp["h0"], inp["c0"], inp["g"], dhT, dcT, direction, ra, order,
                    lengths=lengths, att=att, **kw)
    ref = oracle_layer(mode, P, inp["x"], inp["h0"], inp["c0"], inp["g"], dhT, dcT, direction, ra, order,
                       lengths=lengths, att=att)
    return got, ref


def _permute_params(P, order, H):
    """Store named gates (given in the identity order) in storage order `order`."""
    def perm(a):
        return np.concatenate([a[g * H:(g + 1) * H] for g in order], axis=0)
    return Params(perm(P.W_ih), perm(P.W_hh), perm(P.b_ih), perm(P.b_hh))


# ------------------------------------------------------------- small ----

@pytest.mark.parametrize("direction", [0, 1])
@pytest.mark.parametrize("order", [(0, 1, 2, 3), (1, 0, 2, 3)])
def test_lstm_f32_small(direction, order):
    wl, inp, P = _case("lstm_f32_t8_b2_i16_h32")
    P = _permute_params(P, order, wl.H)
    rng = np.random.default_rng(7)
    dhT, dcT = rng.standard_normal((wl.B, wl.H)), rng.standard_normal((wl.B, wl.H))
    got, ref = _run(wl, inp, P, direction, order, dhT, dcT)
    print(compare(got, ref, "f32", extra=f"dir={direction} order={order}"))


@pytest.mark.parametrize("ra", [False, True])
@pytest.mark.parametrize("direction", [0, 1])
def test_gru_f32_small_ragged(ra, direction):
    # B=3 (one partial 16-row group), I=24, H=32: ragged GEMM tiles
    wl, inp, P = _case("grura_f32_t64_b16_i256_h256", T=6, B=3, I=24, H=32, h0_std=1.0, reset_after=ra)
    order = (2, 0, 1)
    P = _permute_params(P, order, wl.H)
    rng = np.random.default_rng(8)
    dhT = rng.standard_normal((wl.B, wl.H))
    got, ref = _run(wl, inp, P, direction, order, dhT)
    print(compare(got, ref, "f32", extra=f"ra={ra} dir={direction}"))


def test_lstm_f32_ragged_strided():
    # B=19 (two batch groups, ragged), M=T*B=95 rows, padded row strides
    wl, inp, P = _case("lstm_f32_t8_b2_i16_h32", T=5, B=19, I=40, H=48)
    got, ref = _run(wl, inp, P, 1, None, xpad=8, ypad=16)
    print(compare(got, ref, "f32"))
    assert np.all(np.isnan(got["ypad"])), "y written outside its columns"
    assert np.all(got["dxpad"] == 0), "dx written outside its columns"


def test_edge_t1_b1_null_states():
    wl, inp, P = _case("lstm_f32_t8_b2_i16_h32", T=1, B=1, h0_std=0.0, c0_std=0.0)
    assert inp["h0"] is None and inp["c0"] is None
    got, ref = _run(wl, inp, P)
    print(compare(got, ref, "f32"))


def test_accumulate_and_skip_dx():
    wl, inp, P = _case("lstm_f32_t8_b2_i16_h32")
    once = gpu_layer("lstm", "f32", P, inp["x"], inp["h0"], inp["c0"], inp["g"])
    twice = gpu_layer("lstm", "f32", P, inp["x"], inp["h0"], inp["c0"], inp["g"], acc=True, repeat=2)[1]
    for k in ("dW_ih", "dW_hh", "db_ih", "db_hh", "dx"):
        np.testing.assert_allclose(twice[k], 2 * once[k], rtol=1e-5, atol=1e-6)
    nodx = gpu_layer("lstm", "f32", P, inp["x"], inp["h0"], inp["c0"], inp["g"], want_dx=False)
    for k in ("dW_ih", "dh0", "y"):
        np.testing.assert_array_equal(nodx[k], once[k])


@pytest.mark.parametrize("cell", ["lstm", "gru_ra", "gru_basic"])
def test_bf16_weight_gradients_without_dx(cell):
    # bf16 weight gradients run over transposed gate gradients, written by
    # the input-gradient product (and, for the reset-after GRU's
    # candidate-times-r lane, by a transpose) or, when dx is not requested,
    # by a transpose of their own: both give the same values
    if cell == "lstm":
        wl, inp, P = _case("lstm_bf16_t256_b64_i1024_h1024", T=16, B=32, I=256, H=256, h0_std=0.3, c0_std=0.3)
        mode, c0 = "lstm", inp["c0"]
    else:
        wl, inp, P = _case("grura_bf16_t128_b128_i2048_h2048", T=16, B=24, I=256, H=128, h0_std=0.3,
                           reset_after=cell == "gru_ra")
        mode, c0 = "gru", None
    ra = cell != "gru_basic"
    once = gpu_layer(mode, "bf16", P, inp["x"], inp["h0"], c0, inp["g"], reset_after=ra)
    nodx = gpu_layer(mode, "bf16", P, inp["x"], inp["h0"], c0, inp["g"], want_dx=False, reset_after=ra)
    for k in ("dW_ih", "dW_hh", "db_ih", "db_hh", "dh0", "dc0", "y"):
        if k in once:
            np.testing.assert_array_equal(nodx[k], once[k], err_msg=k)


@pytest.mark.parametrize("cell,H", [("lstm", 192), ("gru_ra", 272), ("gru_basic", 64)])
def test_f32_transposed_weight_gradients(cell, H):
    # fp32 layers with T*B >= 8192 and I a multiple of 256 (and no fused
    # dW_hh in the BPTT kernel) run the weight gradients over transposed
    # operands as bf16 layers do
    name = "lstm_f32_t8_b2_i16_h32" if cell == "lstm" else "grura_f32_t64_b16_i256_h256"
    changes = dict(T=128, B=64, I=256, H=H, h0_std=0.3)
    if cell == "lstm":
        changes["c0_std"] = 0.3
    else:
        changes["reset_after"] = cell == "gru_ra"
    wl, inp, P = _case(name, **changes)
    got, ref = _run(wl, inp, P, direction=1)
    print(compare(got, ref, "f32", extra=f"{cell} H{H} transposed dW"))


@pytest.mark.parametrize("cell", ["lstm", "gru_ra", "gru_basic"])
def test_f32_products_at_fp32_accuracy(cell):
    # fp32 recurrent products run on the bf16 matrix cores, each operand split
    # exactly into three bf16 pieces and the six leading piece products
    # summed: what they leave out is below 3*2^-24 of |a||b| per term, so two
    # steps at H = 512 (contractions of 512 to 2048 terms) match the fp64
    # oracle at fp32 rounding level (measured 1e-7 to 1e-6), far inside the
    # fp32 tolerance. A split that kept two pieces of one operand (terms left
    # out of size 2^-16 |a||b|) is off by ~1e-5 in the products and fails
    # these bounds. dx contracts 2048 terms (LSTM) through the fp32 GEMM.
    name = "lstm_f32_t8_b2_i16_h32" if cell == "lstm" else "grura_f32_t64_b16_i256_h256"
    changes = dict(T=2, B=8, I=64, H=512, h0_std=1.0)
    if cell == "lstm":
        changes["c0_std"] = 1.0
    else:
        changes["reset_after"] = cell == "gru_ra"
    wl, inp, P = _case(name, **changes)
    rng = np.random.default_rng(46)
    dhT = rng.standard_normal((wl.B, wl.H))
    got, ref = _run(wl, inp, P, dhT=dhT)
    errs = compare(got, ref, "f32", extra=f"{cell} fp32 accuracy")
    print(cell, {k: f"{e:.2e}" for k, e in errs.items()})
    for k, bound in (("y", 1.5e-6), ("hT", 1.5e-6), ("cT", 1.5e-6), ("dh0", 1.5e-6), ("dc0", 1.5e-6),
                     ("dx", 3e-6), ("dW_ih", 1.5e-6), ("dW_hh", 1.5e-6)):
        if k in errs:
            assert errs[k] <= bound, (k, errs[k])


def test_f32_direct_load_gemms_ragged():
    # fp32 products on the direct-to-LDS GEMM kernel (split bf16 pieces) with
    # ragged sizes: T*B = 8200 rows (the projection's last 256-row tile holds
    # 8), the transposed weight-gradient products split along K = 8200 into 8
    # slices of 1088 with a shorter last one, and the bias row sums from the
    # LDS tiles. The recurrence takes the per-step path at this batch.
    wl, inp, P = _case("bilstm2_f32_t512_b32_i512_h512", T=41, B=200, I=512, H=512, layers=1, bidir=False,
                       h0_std=0.3, c0_std=0.3)
    got, ref = _run(wl, inp, P, 0)
    errs = compare(got, ref, "f32", extra="f32 direct-load GEMMs, ragged")
    print(errs)
    # at fp32 rounding level (measured <= 1.5e-6), as the split products give
    for k, e in errs.items():
        assert e <= 5e-6, (k, e)


@pytest.mark.parametrize("ra", [True, False])
def test_augru_bf16_transposed_weight_gradients(ra):
    # AUGRU scores through the transposed weight-gradient products (the
    # scaled update gate changes every gate gradient they read)
    wl, inp, P = _case("grura_bf16_t128_b128_i2048_h2048", T=10, B=16, I=256, H=128, h0_std=0.3, reset_after=ra)
    att = _scores(wl.T, wl.B, 45, "bf16")
    got, ref = _run(wl, inp, P, att=att)
    print(compare(got, ref, "bf16", extra=f"augru ra={ra} transposed dW"))


@pytest.mark.parametrize("cell", ["lstm", "gru_ra", "gru_basic"])
def test_bf16_transposed_weight_gradients_accumulate(cell):
    # accumulate = 1 over the transposed weight-gradient products (both
    # output parts of the merged product, the candidate rows, the bias row
    # sums): a second call adds its gradients to the first call's stored ones
    if cell == "lstm":
        wl, inp, P = _case("lstm_bf16_t256_b64_i1024_h1024", T=8, B=16, I=256, H=128, h0_std=0.3, c0_std=0.3)
        mode, c0 = "lstm", inp["c0"]
    else:
        wl, inp, P = _case("grura_bf16_t128_b128_i2048_h2048", T=8, B=16, I=256, H=128, h0_std=0.3,
                           reset_after=cell == "gru_ra")
        mode, c0 = "gru", None
    ra = cell != "gru_basic"
    once = gpu_layer(mode, "bf16", P, inp["x"], inp["h0"], c0, inp["g"], reset_after=ra)
    twice = gpu_layer(mode, "bf16", P, inp["x"], inp["h0"], c0, inp["g"], reset_after=ra, acc=True, repeat=2)[1]
    for k in ("dW_ih", "dW_hh", "db_ih", "db_hh", "dx"):
        # the stored first gradient is rounded to bf16 before the second is
        # added in fp32 and the sum rounded again: within two bf16 roundings
        ref = 2.0 * once[k].astype(np.float64)
        err = np.max(np.abs(twice[k] - ref)) / max(np.max(np.abs(ref)), 1e-30)
        assert err < 2 ** -7, (k, err)


@pytest.mark.parametrize("ra", [True, False])
@pytest.mark.parametrize("direction,ragged", [(0, False), (1, True)])
def test_gru_bf16_transposed_weight_gradients(ra, direction, ragged):
    # GRU, bf16, I a multiple of 256: the r and u rows of both weight
    # gradients as one product over [x | h_{t-1}]; the candidate rows as two
    # products (reset-after: d_c against x, d_c * r against h_{t-1}) or as
    # one over [x | r * h_{t-1}] (basic), all over transposed operands;
    # direction 1 with ragged lengths adds the h0 terms of the rows that
    # start late
    wl, inp, P = _case("grura_bf16_t128_b128_i2048_h2048", T=14, B=24, I=256, H=128, h0_std=0.3, reset_after=ra)
    L = _ragged_lengths(wl.B, wl.T, 21 + direction) if ragged else None
    got, ref = _run(wl, inp, P, direction, lengths=L)
    print(compare(got, ref, "bf16", extra=f"gru ra={ra} nt dir{direction} ragged={ragged}"))


@pytest.mark.parametrize("order,direction", [((1, 0, 2, 3), 0), ((3, 2, 0, 1), 1)])
def test_bptt_transposed_recurrent_weights(order, direction):
    # bf16 LSTM, H = 1024 (8 MiB of W_hh), small batch: the BPTT kernel reads
    # W_hh from a copy transposed into its unit-major contraction order, gate
    # permutation included (fp32 has no forward plan with that much W_hh)
    wl, inp, P = _case("lstm_bf16_t256_b64_i1024_h1024", T=4, B=8, I=32, H=1024, h0_std=0.3, c0_std=0.3)
    P = _permute_params(P, order, wl.H)
    got, ref = _run(wl, inp, P, direction, order)
    print(compare(got, ref, "bf16", extra=f"order={order} dir={direction}"))


@pytest.mark.parametrize("name", ["gru_f32_t64_b16_i256_h256", "grura_f32_t64_b16_i256_h256"])
def test_gru_f32_full(name):
    wl, inp, P = _case(name)
    got, ref = _run(wl, inp, P)
    print(compare(got, ref, "f32", extra=name))


def test_deterministic_repeats():
    wl, inp, P = _case("grura_f32_t64_b16_i256_h256", T=16)
    a, b = gpu_layer("gru", "f32", P, inp["x"], inp["h0"], None, inp["g"], repeat=2)
    for k in a:
        np.testing.assert_array_equal(np.nan_to_num(a[k]), np.nan_to_num(b[k]), err_msg=k)


# ------------------------------------------------------------ bf16 -------

@pytest.mark.parametrize("name,changes", [
    ("lstm_bf16_t256_b64_i1024_h1024", dict(T=16, B=32, I=256, H=256)),
    ("grura_bf16_t128_b128_i2048_h2048", dict(T=16, B=20, I=128, H=128)),
    ("grura_bf16_t128_b128_i2048_h2048", dict(T=16, B=16, I=256, H=128)),
    ("grura_bf16_t128_b128_i2048_h2048", dict(T=12, B=16, I=64, H=64, reset_after=False)),
])
def test_bf16_medium(name, changes):
    wl, inp, P = _case(name, **changes)
    got, ref = _run(wl, inp, P)
    print(compare(got, ref, "bf16", extra=name))


# ------------------------------------------------- variable lengths -------

def _ragged_lengths(B, T, seed):
    """Per-row step counts with the special values 0, 1, T-1 and T present."""
    rng = np.random.default_rng(seed)
    L = rng.integers(0, T + 1, size=B)
    L[: min(B, 4)] = [0, 1, T - 1, T][: min(B, 4)]
    return rng.permutation(L).astype(np.int32)


@pytest.mark.parametrize("direction", [0, 1])
@pytest.mark.parametrize("cell", ["lstm", "gru_ra", "gru_basic"])
def test_variable_lengths_f32_small(cell, direction):
    # nonzero h0/c0, so that direction 1 checks each row starting from them
    # at its own last step
    name = "lstm_f32_t8_b2_i16_h32" if cell == "lstm" else "grura_f32_t64_b16_i256_h256"
    changes = dict(T=11, B=13, I=40, H=48, w_scale=0.15, h0_std=0.5, c0_std=0.5)
    if cell != "lstm":
        changes["reset_after"] = cell == "gru_ra"
    wl, inp, P = _case(name, **changes)
    L = _ragged_lengths(wl.B, wl.T, 7 + direction)
    got, ref = _run(wl, inp, P, direction, lengths=L)
    print(compare(got, ref, "f32", extra=f"{cell} dir{direction} lengths={L.tolist()}"))


@pytest.mark.parametrize("direction", [0, 1])
@pytest.mark.parametrize("cell,H", [("lstm", 48), ("lstm", 256), ("gru_ra", 48), ("gru_ra", 128)])
def test_variable_lengths_bf16_medium(cell, H, direction):
    # H=48 in bf16 runs without the exchange ring (y carries the state and a
    # later pass zeroes it past each row's length); the larger H use the ring
    name = "lstm_bf16_t256_b64_i1024_h1024" if cell == "lstm" else "grura_bf16_t128_b128_i2048_h2048"
    wl, inp, P = _case(name, T=14, B=24, I=64, H=H, h0_std=0.3, c0_std=0.3)
    L = _ragged_lengths(wl.B, wl.T, 11 + direction)
    got, ref = _run(wl, inp, P, direction, lengths=L)
    print(compare(got, ref, "bf16", extra=f"{cell} H{H} dir{direction}"))


def test_bidir_stack_on_a_side_stream():
    """A bidirectional stack run on a stream other than torch's current one
    (default priority): its stacked temporaries and gradient copy-backs are
    ordered with the library's kernels on that stream, so the results equal
    those of the current-stream run bit for bit; a raw handle is refused."""
    from gru_layer_fwd_amd.api import RnnStack
    from rnn_harness import dev
    T, B, I, H = 9, 5, 24, 32
    wl = synth.small(W["bilstm2_f32_t512_b32_i512_h512"], T=T, B=B, I=I, H=H, layers=2, bidir=True, w_scale=0.15)
    inp = synth.make_inputs(wl)
    params = [[tuple(dev(a, "f32") for a in (p.W_ih, p.W_hh, p.b_ih, p.b_hh)) for p in per] for per in inp["params"]]
    x, g = dev(inp["x"], "f32"), dev(inp["g"], "f32")

    def run(stream):
        st = RnnStack("lstm", T, B, I, H, "f32", 2, True)
        grads = [[tuple(torch.zeros_like(t) for t in pd) for pd in per] for per in params]
        dx = torch.empty_like(x)
        y = st.fwd(x, params, stream=stream)
        st.bwd(x, params, g, dx, grads, stream=stream)
        if stream is not None:
            torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()
        return y.clone(), dx, grads

    y0, dx0, g0 = run(None)
    side = torch.cuda.Stream()
    y1, dx1, g1 = run(side)
    assert torch.equal(y0, y1) and torch.equal(dx0, dx1)
    for li in range(2):
        for d in range(2):
            for a, b in zip(g0[li][d], g1[li][d]):
                assert torch.equal(a, b)
    with pytest.raises(TypeError):
        RnnStack("lstm", T, B, I, H, "f32", 2, True).fwd(x, params, stream=side.cuda_stream)


@pytest.mark.parametrize("mode", ["lstm", "gru"])
def test_bidir_stack_variable_lengths(mode):
    """Two bidirectional layers sharing one lengths array and nonzero h0/c0:
    the reverse halves start each row at its own last step in both layers."""
    import oracle as O
    from gru_layer_fwd_amd.api import RnnStack
    from rnn_harness import dev, host
    T, B, I, H = 10, 7, 32, 48
    base = "bilstm2_f32_t512_b32_i512_h512" if mode == "lstm" else "grura_f32_t64_b16_i256_h256"
    wl = synth.small(W[base], T=T, B=B, I=I, H=H, layers=2, bidir=True, w_scale=0.15)
    inp = synth.make_inputs(wl)
    rng = np.random.default_rng(5)
    h0 = rng.standard_normal((B, H)) * 0.5
    c0 = rng.standard_normal((B, H)) * 0.5 if mode == "lstm" else None
    L = _ragged_lengths(B, T, 9)
    order = (0, 1, 2, 3) if mode == "lstm" else (0, 1, 2)
    lens = torch.as_tensor(L, dtype=torch.int32).to("cuda")
    st = RnnStack(mode, T, B, I, H, "f32", 2, True, lengths=lens)
    params = [[tuple(dev(a, "f32") for a in (p.W_ih, p.W_hh, p.b_ih, p.b_hh)) for p in per] for per in inp["params"]]
    grads = [[tuple(torch.zeros_like(t) for t in pd) for pd in per] for per in params]
    x = dev(inp["x"], "f32")
    dx = torch.empty_like(x)
    h0d, c0d = dev(h0, "f32"), dev(c0, "f32")
    y = st.fwd(x, params, h0d, c0d)
    st.bwd(x, params, dev(inp["g"], "f32"), dx, grads, h0d, c0d)
    torch.cuda.synchronize()
    recs, y_ref = O.stack_forward(mode, inp["x"], inp["params"], order, True, True, h0, c0, lengths=L)
    gr_ref, dx_ref = O.stack_backward(mode, recs, inp["g"])
    errs = {"y": O.rel_err(host(y), y_ref), "dx": O.rel_err(host(dx), dx_ref)}
    for li in range(2):
        for d in range(2):
            for k, t in zip(("dW_ih", "dW_hh", "db_ih", "db_hh"), grads[li][d]):
                errs[f"L{li}d{d}.{k}"] = O.rel_err(host(t), gr_ref[li][d][k])
    print(errs)
    assert errs["y"] <= 1e-4, errs
    assert all(v <= 1e-3 for k, v in errs.items() if k != "y"), errs



# ------------------------------------------------------------ AUGRU -------

def _scores(T, B, seed, dtype):
    """Attention scores in [0, 1], rounded to the storage type as the GPU sees them."""
    from gru_layer_fwd_amd.synth import round_to
    a = np.random.default_rng(seed).uniform(0.0, 1.0, (T, B))
    a[0, 0], a[-1, -1] = 0.0, 1.0
    return round_to(a, dtype)


@pytest.mark.parametrize("direction", [0, 1])
@pytest.mark.parametrize("ra", [False, True])
@pytest.mark.parametrize("ragged", [False, True])
def test_augru_f32_small(ra, direction, ragged):
    wl, inp, P = _case("grura_f32_t64_b16_i256_h256", T=11, B=13, I=40, H=48, w_scale=0.15, h0_std=0.5,
                       reset_after=ra)
    att = _scores(wl.T, wl.B, 31 + direction, "f32")
    L = _ragged_lengths(wl.B, wl.T, 17) if ragged else None
    got, ref = _run(wl, inp, P, direction, lengths=L, att=att)
    print(compare(got, ref, "f32", extra=f"augru ra={ra} dir{direction} ragged={ragged}"))


@pytest.mark.parametrize("H", [48, 128])
@pytest.mark.parametrize("ra", [False, True])
def test_augru_bf16_medium(ra, H):
    wl, inp, P = _case("grura_bf16_t128_b128_i2048_h2048", T=14, B=24, I=64, H=H, h0_std=0.3, reset_after=ra)
    att = _scores(wl.T, wl.B, 41, "bf16")
    got, ref = _run(wl, inp, P, 1, lengths=_ragged_lengths(wl.B, wl.T, 19), att=att)
    print(compare(got, ref, "bf16", extra=f"augru ra={ra} H{H}"))


# ---------------------------------------- LSTM cell-state recomputation ----

@pytest.mark.parametrize("direction", [0, 1])
@pytest.mark.parametrize("ragged", [False, True])
def test_lstm_recompute_f32_small(direction, ragged):
    wl, inp, P = _case("lstm_f32_t8_b2_i16_h32", T=11, B=13, I=40, H=48, w_scale=0.15, h0_std=0.5, c0_std=0.5)
    L = _ragged_lengths(wl.B, wl.T, 29) if ragged else None
    got, ref = _run(wl, inp, P, direction, lengths=L, recompute=True)
    print(compare(got, ref, "f32", extra=f"recompute dir{direction} ragged={ragged}"))
    # fp32 gates rebuild the same cell states the forward kept: the two modes agree to rounding
    base = gpu_layer(wl.mode, wl.dtype, P, inp["x"], inp["h0"], inp["c0"], inp["g"], None, None, direction,
                     lengths=L)
    for k in base:
        np.testing.assert_allclose(got[k], base[k], rtol=1e-5, atol=1e-6, err_msg=k)


@pytest.mark.parametrize("H", [48, 256])
def test_lstm_recompute_bf16_medium(H):
    wl, inp, P = _case("lstm_bf16_t256_b64_i1024_h1024", T=14, B=24, I=64, H=H, h0_std=0.3, c0_std=0.3)
    got, ref = _run(wl, inp, P, 1, lengths=_ragged_lengths(wl.B, wl.T, 37), recompute=True)
    print(compare(got, ref, "bf16", extra=f"recompute H{H}"))


# ------------------------------------------- more ring configurations -----
# H = 512 bf16 (16 k-steps, two per packed tile) and H = 1024 with 5 rows
# (packed ring, 4-row groups) and 128 rows (the grid only fits 16-row groups:
# one k-step per tile).

@pytest.mark.parametrize("direction", [0, 1])
def test_lstm_bf16_h512_ragged(direction):
    wl, inp, P = _case("lstm_bf16_t256_b64_i1024_h1024", T=10, B=12, I=64, H=512, h0_std=0.3, c0_std=0.3)
    got, ref = _run(wl, inp, P, direction, lengths=_ragged_lengths(wl.B, wl.T, 43))
    print(compare(got, ref, "bf16", extra=f"lstm h512 dir{direction}"))


@pytest.mark.parametrize("rows", [5, 128])
def test_grura_bf16_h1024_augru(rows):
    # 5 rows: groups of <= 8 rows (two k-steps per ring tile); 128 rows: the
    # grid only fits with 16-row groups (one k-step per tile)
    wl, inp, P = _case("grura_bf16_t128_b128_i2048_h2048", T=4, B=rows, I=64, H=1024, w_scale=1 / 32,
                       h0_std=0.3)
    att = _scores(wl.T, wl.B, 61, "bf16")
    got, ref = _run(wl, inp, P, 0, att=att)
    print(compare(got, ref, "bf16", extra=f"grura h1024 B{rows}"))


def test_lstm_bf16_h2048_64_row_groups_ragged():
    # B = 72 at H = 2048: the forward runs two groups of 64 rows (the second
    # holding 8) on the 4-wave 64-row kernel, the BPTT 64-row groups as well
    wl, inp, P = _case("lstm_bf16_t128_b128_i2048_h2048", T=4, B=72, I=64, H=2048, h0_std=0.3, c0_std=0.3)
    got, ref = _run(wl, inp, P, 1, lengths=_ragged_lengths(wl.B, wl.T, 47))
    print(compare(got, ref, "bf16", extra="lstm h2048 B72"))


# --------------------------------------------- seeded shape sweep -------
# Cells, storage types, directions and sizes drawn once from a fixed seed:
# odd batches, T from 1, I a multiple of 8 and H of 16 that are mostly not
# multiples of 32 (ragged MFMA tiles and k-steps in the products), ragged
# lengths on some. Every element against the oracle.

def _sweep_cases(n=18, seed=2026):
    rng = np.random.default_rng(seed)
    cells = ["lstm", "gru_ra", "gru_basic"]
    out = []
    for i in range(n):
        cell = cells[i % 3]
        dtype = "f32" if (i // 3) % 2 == 0 else "bf16"
        T = int(rng.choice([1, 2, 3, 5, 7]))
        B = int(rng.choice([1, 3, 5, 9, 17, 20]))
        I = int(rng.choice([8, 24, 40, 72, 136]))
        H = int(rng.choice([16, 48, 80, 112, 144, 208]))  # H % 16 == 0 (the boundary's granularity)
        direction = int(rng.integers(0, 2))
        ragged = bool(rng.integers(0, 2)) and T > 1
        out.append((cell, dtype, T, B, I, H, direction, ragged))
    return out


@pytest.mark.parametrize("cell,dtype,T,B,I,H,direction,ragged", _sweep_cases())
def test_seeded_shape_sweep(cell, dtype, T, B, I, H, direction, ragged):
    name = "lstm_f32_t8_b2_i16_h32" if cell == "lstm" else "grura_f32_t64_b16_i256_h256"
    # weights ~ U(+-2/sqrt(H)): pre-activations of order one whatever H (the
    # workloads' own scale is 1/sqrt(H); far larger weights at large H put
    # bf16-rounded inputs' error alone near the bf16 tolerance)
    changes = dict(T=T, B=B, I=I, H=H, h0_std=0.5, w_scale=2.0 / np.sqrt(H), dtype=dtype)
    if cell == "lstm":
        changes["c0_std"] = 0.5
    else:
        changes["reset_after"] = cell == "gru_ra"
    wl, inp, P = _case(name, **changes)
    lengths = _ragged_lengths(B, T, 100 + T * B) if ragged else None
    rng = np.random.default_rng(H * 7 + I)
    dhT = rng.standard_normal((B, H))
    dcT = rng.standard_normal((B, H)) if cell == "lstm" else None
    got, ref = _run(wl, inp, P, direction, dhT=dhT, dcT=dcT, lengths=lengths)
    print(compare(got, ref, dtype, extra=f"{cell} {dtype} T{T} B{B} I{I} H{H} dir{direction} ragged={ragged}"))


def _sweep_cases_large(n=12, seed=2027):
    # larger hidden sizes and batches, which take the persistent plans' other
    # instantiations (8-wave kernels, several batch groups, multi-tile rows)
    rng = np.random.default_rng(seed)
    cells = ["lstm", "gru_ra", "gru_basic"]
    out = []
    for i in range(n):
        cell = cells[i % 3]
        dtype = "f32" if (i // 3) % 2 == 0 else "bf16"
        T = int(rng.choice([2, 3, 4]))
        B = int(rng.choice([12, 33, 64, 100]))
        I = int(rng.choice([64, 136, 256]))
        H = int(rng.choice([256, 384, 512] if dtype == "f32" else [256, 512, 768, 1024]))
        direction = int(rng.integers(0, 2))
        ragged = bool(rng.integers(0, 2))
        out.append((cell, dtype, T, B, I, H, direction, ragged))
    return out


@pytest.mark.parametrize("cell,dtype,T,B,I,H,direction,ragged", _sweep_cases_large())
def test_seeded_shape_sweep_large(cell, dtype, T, B, I, H, direction, ragged):
    test_seeded_shape_sweep(cell, dtype, T, B, I, H, direction, ragged)


# -------------------------------------------- lengths / scores: edges ----

def _edge_case(mode, ra, **sizes):
    name = "lstm_f32_t8_b2_i16_h32" if mode == "lstm" else "grura_f32_t64_b16_i256_h256"
    kw = dict(h0_std=0.7, c0_std=0.7, w_scale=0.3, **sizes)
    if mode == "gru":
        kw["reset_after"] = ra
    return _case(name, **kw)


def _final_grads(wl, seed):
    rng = np.random.default_rng(seed)
    dhT = rng.standard_normal((wl.B, wl.H))
    dcT = rng.standard_normal((wl.B, wl.H)) if wl.mode == "lstm" else None
    return dhT, dcT


@pytest.mark.parametrize("direction", [0, 1])
@pytest.mark.parametrize("mode,ra", [("lstm", None), ("gru", True), ("gru", False)])
def test_lengths_single_step_rows(mode, ra, direction):
    wl, inp, P = _edge_case(mode, ra, T=1, B=3, I=16, H=32)
    dhT, dcT = _final_grads(wl, 5)
    got, ref = _run(wl, inp, P, direction, None, dhT, dcT, lengths=np.array([0, 1, 0], np.int32))
    print(compare(got, ref, "f32", extra=f"{mode} ra={ra} dir{direction}"))


@pytest.mark.parametrize("direction", [0, 1])
@pytest.mark.parametrize("mode,ra", [("lstm", None), ("gru", True), ("gru", False)])
def test_lengths_all_rows_empty(mode, ra, direction):
    # nothing runs: zero output, the state and its gradients pass through,
    # zero input and weight gradients
    wl, inp, P = _edge_case(mode, ra, T=5, B=4, I=16, H=32)
    dhT, dcT = _final_grads(wl, 6)
    got, ref = _run(wl, inp, P, direction, None, dhT, dcT, lengths=np.zeros(wl.B, np.int32))
    print(compare(got, ref, "f32", extra=f"{mode} ra={ra} dir{direction}"))
    assert np.all(got["y"] == 0) and np.all(got["dx"] == 0)
    for k in ("dW_ih", "dW_hh", "db_ih", "db_hh"):
        assert np.all(got[k] == 0), k
    np.testing.assert_array_equal(got["hT"], inp["h0"].astype(np.float32))
    np.testing.assert_array_equal(got["dh0"], dhT.astype(np.float32))
    if mode == "lstm":
        np.testing.assert_array_equal(got["cT"], inp["c0"].astype(np.float32))
        np.testing.assert_array_equal(got["dc0"], dcT.astype(np.float32))


@pytest.mark.parametrize("direction", [0, 1])
def test_augru_final_state_gradient_and_accumulated_scores(direction):
    wl, inp, P = _edge_case("gru", True, T=7, B=5, I=24, H=32)
    att = _scores(wl.T, wl.B, 71, "f32")
    dhT, _ = _final_grads(wl, 7)
    got, ref = _run(wl, inp, P, direction, None, dhT, att=att, lengths=np.array([7, 0, 3, 6, 1], np.int32))
    print(compare(got, ref, "f32", extra=f"dir{direction}"))
    once = gpu_layer("gru", "f32", P, inp["x"], inp["h0"], None, inp["g"], dhT, None, direction, att=att)
    twice = gpu_layer("gru", "f32", P, inp["x"], inp["h0"], None, inp["g"], dhT, None, direction, att=att,
                      acc=True, repeat=2)[1]
    np.testing.assert_allclose(twice["datt"], 2 * once["datt"], rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("direction", [0, 1])
def test_lstm_recompute_with_final_state_gradients(direction):
    wl, inp, P = _edge_case("lstm", None, T=9, B=6, I=16, H=32)
    dhT, dcT = _final_grads(wl, 8)
    got, ref = _run(wl, inp, P, direction, None, dhT, dcT, lengths=np.array([9, 4, 0, 1, 8, 9], np.int32),
                    recompute=True)
    print(compare(got, ref, "f32", extra=f"dir{direction}"))


# ------------------------------------------------ bidirectional layer ----

@pytest.mark.parametrize("mode,ra,dtype,big,stepwise", [
    ("lstm", None, "f32", False, False), ("gru", True, "f32", False, False), ("gru", False, "f32", False, False),
    ("lstm", None, "bf16", False, False), ("lstm", None, "bf16", True, False),
    ("gru", True, "bf16", False, False), ("gru", False, "bf16", False, False),
    # the per-step path for both directions of a bidirectional layer
    ("lstm", None, "f32", False, True), ("gru", True, "bf16", False, True), ("gru", False, "f32", False, True)])
def test_bidirectional_layer_runs_both_directions(mode, ra, dtype, big, stepwise):
    """direction 2: [2, ...] stacked weights and states, y/dy halves in one
    [T, B, 2H] tensor, dx summed over the directions; each direction against
    the oracle with its own weights and initial and final states. `big`:
    H = 1024, so that each direction's BPTT reads its own transposed copy of
    its W_hh (8 MiB)."""
    import oracle as O
    from gru_layer_fwd_amd.api import RnnLayer
    from rnn_harness import dev, host
    T, B, I, H = 9, 12, 64, 64
    if dtype == "bf16":
        T, B, I, H = (6, 8, 32, 1024) if big else (12, 24, 256, 256)
    rng = np.random.default_rng(81)
    G = 4 if mode == "lstm" else 3
    from gru_layer_fwd_amd.synth import round_to
    rnd = lambda a: round_to(a, dtype)  # noqa: E731
    k = 1 / np.sqrt(H)
    W_ih, W_hh = rnd(rng.uniform(-k, k, (2, G * H, I))), rnd(rng.uniform(-k, k, (2, G * H, H)))
    b_ih, b_hh = rnd(rng.uniform(-k, k, (2, G * H))), rnd(rng.uniform(-k, k, (2, G * H)))
    x = rnd(rng.standard_normal((T, B, I)))
    h0 = rnd(0.5 * rng.standard_normal((2, B, H)))
    c0 = rnd(0.5 * rng.standard_normal((2, B, H))) if mode == "lstm" else None
    g = rnd(rng.standard_normal((T, B, 2 * H)))
    dhT = rnd(rng.standard_normal((2, B, H)))
    dcT = rnd(rng.standard_normal((2, B, H))) if mode == "lstm" else None
    L = _ragged_lengths(B, T, 83)
    lens = torch.as_tensor(L, dtype=torch.int32).to("cuda")
    lay = RnnLayer(mode, T, B, I, H, dtype, direction=2, reset_after=bool(ra), lengths=lens, stepwise=stepwise)
    d_ = lambda a: dev(a, dtype)  # noqa: E731
    tdt = lay.torch_dtype
    y = torch.full((T, B, 2 * H), float("nan"), dtype=tdt, device="cuda")
    hT = torch.empty(2, B, H, dtype=tdt, device="cuda")
    cT = torch.empty(2, B, H, dtype=tdt, device="cuda") if mode == "lstm" else None
    dx = torch.empty(T, B, I, dtype=tdt, device="cuda")
    dh0 = torch.empty(2, B, H, dtype=tdt, device="cuda")
    dc0 = torch.empty(2, B, H, dtype=tdt, device="cuda") if mode == "lstm" else None
    grads = [torch.empty(a.shape, dtype=tdt, device="cuda") for a in (W_ih, W_hh, b_ih, b_hh)]
    Wd = [d_(a) for a in (W_ih, W_hh, b_ih, b_hh)]
    lay.fwd(d_(x), d_(h0), d_(c0), *Wd, y, hT, cT)
    lay.bwd_data(Wd[0], Wd[1], d_(h0), d_(c0), y, d_(g), d_(dhT), d_(dcT), dx, dh0, dc0)
    lay.bwd_weights(d_(x), d_(h0), y, *grads)
    torch.cuda.synchronize()
    assert lay.device_status() == 0
    order = (0, 1, 2, 3) if mode == "lstm" else (0, 1, 2)
    tol_f, tol_g = (1e-4, 1e-3) if dtype == "f32" else (2e-2, 2e-2)
    dx_ref = 0
    for dd in range(2):
        P = Params(W_ih[dd], W_hh[dd], b_ih[dd], b_hh[dd])
        fw = O.layer_forward(mode, x, h0[dd], None if c0 is None else c0[dd], P, order, reverse=bool(dd),
                             reset_after=bool(ra), lengths=L)
        gr = O.layer_backward(mode, fw, g[:, :, dd * H:(dd + 1) * H], dhT[dd], None if dcT is None else dcT[dd])
        dx_ref = dx_ref + gr["dx"]
        errs = {"y": O.rel_err(host(y)[:, :, dd * H:(dd + 1) * H], fw["y"]), "hT": O.rel_err(host(hT)[dd], fw["hT"]),
                "dh0": O.rel_err(host(dh0)[dd], gr["dh0"])}
        for name, t in zip(("dW_ih", "dW_hh", "db_ih", "db_hh"), grads):
            errs[name] = O.rel_err(host(t)[dd], gr[name])
        if mode == "lstm":
            errs["cT"] = O.rel_err(host(cT)[dd], fw["cT"])
            errs["dc0"] = O.rel_err(host(dc0)[dd], gr["dc0"])
        print(dd, errs)
        assert all(v <= (tol_f if k in ("y", "hT", "cT") else tol_g) for k, v in errs.items()), (dd, errs)
    e = O.rel_err(host(dx), dx_ref)
    assert e <= tol_g, e


# ------------------------------------------------------ per-step path ----

@pytest.mark.parametrize("direction", [0, 1])
@pytest.mark.parametrize("cell", ["lstm", "gru_ra", "gru_basic"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_stepwise_path(cell, dtype, direction):
    """The per-step recurrence (forced on a shape the persistent kernels
    also take) against the oracle: ragged lengths with rows of length 0, 1,
    T-1 and T, nonzero initial states and final-state gradients; on
    direction 1 AUGRU scores (GRU) and cell-state recomputation (LSTM)."""
    name = "lstm_f32_t8_b2_i16_h32" if cell == "lstm" else "grura_f32_t64_b16_i256_h256"
    changes = dict(T=11, B=13, I=40, H=48, w_scale=0.15, h0_std=0.5, c0_std=0.5, dtype=dtype)
    if cell != "lstm":
        changes["reset_after"] = cell == "gru_ra"
    wl, inp, P = _case(name, **changes)
    rng = np.random.default_rng(5 + direction)
    from gru_layer_fwd_amd.synth import round_to
    dhT = round_to(rng.standard_normal((wl.B, wl.H)), dtype)
    dcT = round_to(rng.standard_normal((wl.B, wl.H)), dtype) if cell == "lstm" else None
    L = _ragged_lengths(wl.B, wl.T, 37 + direction)
    kw = {}
    if direction == 1 and cell != "lstm":
        kw["att"] = _scores(wl.T, wl.B, 43, dtype)
    if direction == 1 and cell == "lstm":
        kw["recompute"] = True
    got, ref = _run(wl, inp, P, direction, dhT=dhT, dcT=dcT, lengths=L, stepwise=True, **kw)
    print(compare(got, ref, dtype, extra=f"stepwise {cell} {dtype} dir{direction}"))


@pytest.mark.parametrize("cell,H", [("lstm", 1024), ("gru_ra", 1024), ("gru_basic", 1024), ("lstm", 2048)])
def test_shapes_beyond_the_plans_run_per_step(cell, H):
    """fp32 shapes with no persistent plan (W_hh 12-64 MiB): the layer takes
    the per-step path by itself and matches the oracle."""
    from gru_layer_fwd_amd import _lib as L
    name = "lstm_f32_t8_b2_i16_h32" if cell == "lstm" else "grura_f32_t64_b16_i256_h256"
    changes = dict(T=5, B=6, I=32, H=H, w_scale=1.0 / np.sqrt(H), h0_std=0.5, c0_std=0.5)
    if cell != "lstm":
        changes["reset_after"] = cell == "gru_ra"
    wl, inp, P = _case(name, **changes)
    d = L.make_desc(L.RNN_LSTM if cell == "lstm" else L.RNN_GRU, wl.T, wl.B, wl.I, H, L.RNN_F32, 0,
                    int(cell != "gru_basic"))
    for p in (0, 1):
        st, plan = L.rnn_plan_query(d, p)
        assert st == 0 and plan.stepwise == 1
    got, ref = _run(wl, inp, P, 1, lengths=_ragged_lengths(wl.B, wl.T, 47))
    print(compare(got, ref, "f32", extra=f"beyond plans {cell} H{H}"))


# ------------------------------------------------- failure detection ----

@pytest.mark.parametrize("bidir", [False, True])
def test_handshake_timeout_is_reported_and_recovers(bidir):
    """A time-out forced from the host (every bounded wait gives up at once):
    the kernels still run to the end and the workspace status word reports
    RNN_ERR_TIMEOUT; with the default restored the same layer is exact again."""
    from gru_layer_fwd_amd import _lib as Lb
    wl, inp, P = _case("lstm_f32_t8_b2_i16_h32", T=6, B=5, I=16, H=32)
    direction = 2 if bidir else 0
    try:
        Lb.rnn_set_handshake_timeout(-1.0)
        lay_args = dict(direction=direction)
        from gru_layer_fwd_amd.api import RnnLayer
        from rnn_harness import dev
        lay = RnnLayer("lstm", wl.T, wl.B, wl.I, wl.H, "f32", **lay_args)
        dirs = 2 if bidir else 1
        G = 4
        W = [torch.stack([dev(a, "f32")] * dirs) if bidir else dev(a, "f32") for a in (P.W_ih, P.W_hh, P.b_ih, P.b_hh)]
        x = dev(inp["x"], "f32")
        y = torch.empty(wl.T, wl.B, wl.H * dirs, device="cuda")
        g = torch.randn(wl.T, wl.B, wl.H * dirs, device="cuda")
        dx = torch.empty_like(x)
        lay.fwd(x, None, None, *W, y)
        torch.cuda.synchronize()
        assert lay.device_status() == Lb.RNN_ERR_TIMEOUT
        lay.bwd_data(W[0], W[1], None, None, y, g, None, None, dx)
        torch.cuda.synchronize()
        assert lay.device_status() == Lb.RNN_ERR_TIMEOUT
    finally:
        Lb.rnn_set_handshake_timeout(0.0)
    got, ref = _run(wl, inp, P)
    print(compare(got, ref, "f32"))


# ------------------------------------------- fused weight gradient -----

@pytest.mark.parametrize("direction", [0, 1])
@pytest.mark.parametrize("cell,B,H", [("lstm", 197, 128), ("lstm", 13, 64), ("gru_ra", 83, 256), ("gru_ra", 13, 96)])
def test_fused_recurrent_weight_gradient(cell, B, H, direction):
    """dW_hh accumulated inside the BPTT kernel (batch groups of 4 and of 8
    rows, a ragged last group, rows of length 0, 1, T-1 and T) and dW_hh
    from the separate product both match the oracle; the plan reports the
    fused path for these shapes."""
    from gru_layer_fwd_amd import _lib as L
    name = "lstm_f32_t8_b2_i16_h32" if cell == "lstm" else "grura_f32_t64_b16_i256_h256"
    wl, inp, P = _case(name, T=16, B=B, I=64, H=H, w_scale=0.1, h0_std=0.5, c0_std=0.5)
    d = L.make_desc(L.RNN_LSTM if cell == "lstm" else L.RNN_GRU, wl.T, B, wl.I, H, L.RNN_F32, direction, 1)
    st, plan = L.rnn_plan_query(d, 1)
    assert st == 0 and plan.fused_dw == 1 and plan.rows in (4, 8)
    lens = _ragged_lengths(B, wl.T, 11 + direction)
    print(f"[fused dW] {cell} B={B} H={H} dir={direction} rows={plan.rows} groups={plan.groups}", flush=True)
    got, ref = _run(wl, inp, P, direction, lengths=lens, acc=(direction == 1))
    e_fused = compare(got, ref, "f32", extra=f"fused {cell} B={B} H={H} dir{direction}")
    sep = gpu_layer(wl.mode, wl.dtype, P, inp["x"], inp["h0"], inp["c0"], inp["g"], None, None, direction,
                    wl.reset_after, None, lengths=lens, dw_hh_mode=1)
    e_sep = compare(sep, ref, "f32", extra=f"separate {cell} B={B} H={H} dir{direction}")
    print(f"dW_hh rel err fused {e_fused['dW_hh']:.2e} separate {e_sep['dW_hh']:.2e}")
    # the rest of the backward pass does not depend on where dW_hh is formed
    for k in ("dx", "dh0", "dW_ih", "db_ih"):
        np.testing.assert_array_equal(got[k], sep[k], err_msg=k)


@pytest.mark.parametrize("cell,order", [("lstm", (3, 1, 0, 2)), ("gru_ra", (2, 0, 1)), ("gru_basic", (1, 2, 0))])
@pytest.mark.parametrize("stepwise", [False, True])
def test_permuted_gate_order_paths(cell, order, stepwise):
    """A storage order other than the canonical one through the fused dW_hh
    (the fp32 LSTM and reset-after GRU plans of this shape) and through the
    per-step path: weights, biases and their gradients addressed through the
    permutation; then accumulation into the gradients (twice the one-call
    values)."""
    from gru_layer_fwd_amd import _lib as L
    name = "lstm_f32_t8_b2_i16_h32" if cell == "lstm" else "grura_f32_t64_b16_i256_h256"
    changes = dict(T=9, B=7, I=24, H=64, w_scale=0.2, h0_std=0.5, c0_std=0.5)
    if cell != "lstm":
        changes["reset_after"] = cell == "gru_ra"
    wl, inp, P = _case(name, **changes)
    if not stepwise and cell != "gru_basic":
        d = L.make_desc(L.RNN_LSTM if cell == "lstm" else L.RNN_GRU, wl.T, wl.B, wl.I, wl.H, L.RNN_F32, 1, 1,
                        order)
        st, plan = L.rnn_plan_query(d, 1)
        assert st == 0 and plan.fused_dw == 1
    P = _permute_params(P, order, wl.H)
    lens = _ragged_lengths(wl.B, wl.T, 53)
    got, ref = _run(wl, inp, P, 1, order, lengths=lens, stepwise=stepwise)
    print(compare(got, ref, "f32", extra=f"{cell} order={order} stepwise={stepwise}"))
    twice = gpu_layer(wl.mode, wl.dtype, P, inp["x"], inp["h0"], inp["c0"], inp["g"], None, None, 1,
                      wl.reset_after, order, acc=True, repeat=2, lengths=lens, stepwise=stepwise)[1]
    for k in ("dW_ih", "dW_hh", "db_ih", "db_hh", "dx"):
        np.testing.assert_allclose(twice[k], 2 * got[k], rtol=1e-5, atol=1e-6, err_msg=k)
