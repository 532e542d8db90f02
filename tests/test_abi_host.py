"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/rnn.h declares, sizes workspaces, and rejects bad
arguments with the documented status before touching the device."""
import ctypes
import os
import re

import pytest

import gru_layer_fwd_amd as g
from gru_layer_fwd_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "rnn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rnn_[a-z_]+)\s*\(", src)))


def test_header_declares_the_abi():
    assert _declared() == sorted(["rnn_workspace_bytes", "rnn_fwd", "rnn_bwd_data", "rnn_bwd_weights",
                                  "rnn_last_device_status", "rnn_status_string", "rnn_set_handshake_timeout", "rnn_plan_query",
                                  "rnn_fwd_noalloc", "rnn_handshake_probe",
                                  "rnn_profile_enable", "rnn_profile_read"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(L.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
        assert name in L._SIGS, name


def _desc(**kw):
    base = dict(mode=L.RNN_LSTM, T=8, B=2, I=16, H=32, dtype=L.RNN_F32)
    base.update(kw)
    return g.make_desc(base.pop("mode"), base.pop("T"), base.pop("B"), base.pop("I"), base.pop("H"),
                       base.pop("dtype"), **base)


def test_workspace_size_formula():
    d = _desc(T=7, B=3, I=16, H=32)
    n = g.rnn_workspace_bytes(d)
    # saved gates (4 lanes), cell states and gate gradients dominate: T*B*H*(4+1+4) elements
    assert n >= 7 * 3 * 32 * 9 * 4
    d2 = _desc(T=7, B=3, I=16, H=32, dtype=L.RNN_BF16)
    assert g.rnn_workspace_bytes(d2) < n
    dg = _desc(mode=L.RNN_GRU, T=7, B=3, I=16, H=32, reset_after=0, gate_order=(0, 1, 2))
    assert g.rnn_workspace_bytes(dg) > 0


@pytest.mark.parametrize("bad", [
    dict(mode=5), dict(dtype=3), dict(direction=3), dict(direction=-1), dict(T=0), dict(B=0), dict(I=0), dict(H=0),
    dict(gate_order=(0, 0, 2, 3)), dict(gate_order=(0, 1, 2, 4)),
    dict(mode=L.RNN_GRU, gate_order=(0, 1, 3)), dict(mode=L.RNN_GRU, reset_after=2, gate_order=(0, 1, 2)),
    dict(ldx=8), dict(ldy=16), dict(direction=2, ldy=48),
])
def test_invalid_descriptors(bad):
    d = _desc(**bad)
    assert g.rnn_workspace_bytes(d) == 0
    assert g.rnn_fwd(d, 16, 0, 0, 16, 16, 16, 16, 16, 0, 0, 256, 1 << 30, 0) == L.RNN_ERR_INVALID_ARG


def test_null_descriptor():
    lib = L.lib()
    assert lib.rnn_workspace_bytes(None) == 0
    assert lib.rnn_fwd(None, 16, 0, 0, 16, 16, 16, 16, 16, 0, 0, 256, 1 << 30, None) == L.RNN_ERR_INVALID_ARG


@pytest.mark.parametrize("shape", [dict(H=40), dict(I=12), dict(I=16, ldx=20)])
def test_unsupported_granularity(shape):
    d = _desc(**shape)
    assert g.rnn_workspace_bytes(d) > 0
    assert g.rnn_fwd(d, 16, 0, 0, 16, 16, 16, 16, 16, 0, 0, 256, 1 << 30, 0) == L.RNN_ERR_UNSUPPORTED


def test_workspace_too_small_and_missing_pointers():
    d = _desc()
    n = g.rnn_workspace_bytes(d)
    assert g.rnn_fwd(d, 16, 0, 0, 16, 16, 16, 16, 16, 0, 0, 256, n - 1, 0) == L.RNN_ERR_WORKSPACE_TOO_SMALL
    assert g.rnn_bwd_data(d, 16, 16, 0, 0, 16, 16, 0, 0, 0, 0, 0, 0, 0, 256, n - 1, 0) == L.RNN_ERR_WORKSPACE_TOO_SMALL
    assert g.rnn_bwd_weights(d, 16, 0, 16, 0, 0, 0, 0, 0, 256, n - 1, 0) == L.RNN_ERR_WORKSPACE_TOO_SMALL
    # required pointers
    assert g.rnn_fwd(d, 0, 0, 0, 16, 16, 16, 16, 16, 0, 0, 256, n, 0) == L.RNN_ERR_INVALID_ARG
    assert g.rnn_fwd(d, 16, 0, 0, 16, 16, 16, 16, 0, 0, 0, 256, n, 0) == L.RNN_ERR_INVALID_ARG
    assert g.rnn_bwd_data(d, 16, 16, 0, 0, 16, 0, 0, 0, 0, 0, 0, 0, 0, 256, n, 0) == L.RNN_ERR_INVALID_ARG
    assert g.rnn_bwd_weights(d, 0, 0, 16, 0, 0, 0, 0, 0, 256, n, 0) == L.RNN_ERR_INVALID_ARG
    assert g.rnn_fwd(d, 16, 0, 0, 16, 16, 16, 16, 16, 0, 0, 0, n, 0) == L.RNN_ERR_INVALID_ARG
    # misaligned tensor pointer
    assert g.rnn_fwd(d, 18, 0, 0, 16, 16, 16, 16, 16, 0, 0, 256, n, 0) == L.RNN_ERR_INVALID_ARG


def test_status_strings():
    for st in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(g.rnn_status_string(st), str) and g.rnn_status_string(st)


def test_profile_hook_without_device_work():
    assert g._lib.rnn_profile_enable(True) == 0
    assert g._lib.rnn_profile_read() == {}
    assert g._lib.rnn_profile_enable(False) == 0


def test_descriptor_layout_matches_the_header(tmp_path):
    """The ctypes descriptor has the C struct's size and field offsets
    (compiled from include/rnn.h with the host compiler)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    fields = [f[0] for f in L.RnnDesc._fields_]
    src = tmp_path / "off.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"rnn.h\"\nint main(void){\n"
                   "printf(\"size %zu\\n\", sizeof(rnn_desc_t));\n"
                   + "".join(f"printf(\"{f} %zu\\n\", offsetof(rnn_desc_t, {f}));\n" for f in fields)
                   + "return 0;}\n")
    exe = tmp_path / "off"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                        check=True).stdout.splitlines())
    assert int(out["size"]) == ctypes.sizeof(L.RnnDesc)
    for f in fields:
        assert int(out[f]) == getattr(L.RnnDesc, f).offset, f


def test_misaligned_lengths_rejected_before_device_work():
    d = _desc(lengths=20)
    n = g.rnn_workspace_bytes(d)
    assert n > 0
    assert g.rnn_fwd(d, 16, 0, 0, 16, 16, 16, 16, 16, 0, 0, 256, n, 0) == L.RNN_ERR_INVALID_ARG
    assert g.rnn_bwd_data(d, 16, 16, 0, 0, 16, 16, 0, 0, 0, 0, 0, 0, 0, 256, n, 0) == L.RNN_ERR_INVALID_ARG
    assert g.rnn_bwd_weights(d, 16, 0, 16, 0, 0, 0, 0, 0, 256, n, 0) == L.RNN_ERR_INVALID_ARG


def test_attention_scores_only_for_the_gru():
    assert g.rnn_workspace_bytes(_desc(att=256)) == 0           # LSTM with scores: invalid
    dg = _desc(mode=L.RNN_GRU, gate_order=(0, 1, 2), att=256)
    n = g.rnn_workspace_bytes(dg)
    assert n > g.rnn_workspace_bytes(_desc(mode=L.RNN_GRU, gate_order=(0, 1, 2)))  # score partials
    # misaligned scores or score gradient: rejected before device work
    assert g.rnn_fwd(_desc(mode=L.RNN_GRU, gate_order=(0, 1, 2), att=260), 16, 0, 0, 16, 16, 16, 16, 16, 0, 0,
                     256, n, 0) == L.RNN_ERR_INVALID_ARG
    assert g.rnn_bwd_data(dg, 16, 16, 0, 0, 16, 16, 0, 0, 0, 0, 0, 20, 0, 256, n, 0) == L.RNN_ERR_INVALID_ARG


def test_recompute_mode_is_lstm_only_and_drops_the_cell_sequence():
    T, B, H = 7, 3, 32
    n0 = g.rnn_workspace_bytes(_desc(T=T, B=B, H=H))
    n1 = g.rnn_workspace_bytes(_desc(T=T, B=B, H=H, recompute=1))
    assert n1 > 0 and n0 - n1 >= T * B * H * 4
    assert g.rnn_workspace_bytes(_desc(recompute=2)) == 0
    assert g.rnn_workspace_bytes(_desc(mode=L.RNN_GRU, gate_order=(0, 1, 2), recompute=1)) == 0


def test_bidirectional_layer_workspace_is_two_halves():
    single = g.rnn_workspace_bytes(_desc(direction=1, ldy=64))
    both = g.rnn_workspace_bytes(_desc(direction=2))       # ldy 0 means 2H for both directions
    assert single > 0 and both == 2 * single
    assert g.rnn_workspace_bytes(_desc(direction=2, ldy=64)) == both


# ------------------------------------------- plans and co-residency ----
# rnn_plan_query with an injected CU count and occupancy is the same host
# decision rnn_fwd / rnn_bwd_data take before a persistent launch, made
# without a device.

def _plan(desc, pass_, cu=256, occ=1):
    return L.rnn_plan_query(desc, pass_, cu, occ)


def test_headline_plan_one_batch_group_per_xcd():
    d = g.make_desc(L.RNN_LSTM, 256, 64, 1024, 1024, L.RNN_BF16)
    for p in (0, 1):
        st, pl = _plan(d, p)
        assert st == L.RNN_OK
        # 8 groups of 8 rows, each over the 32 CUs of one XCD (32 slices of 32 units)
        assert (pl.groups, pl.rows, pl.slices, pl.units, pl.waves) == (8, 8, 32, 32, 8)
        assert pl.workgroups == 256 and pl.xcd_span == 1 and pl.ring == 2 and pl.dual == 0
        assert 0 < pl.model_us_per_step < 10


def test_large_lstm_forward_plan_two_64_row_groups():
    # B = 128, H = 2048 bf16: two groups of 64 rows over 128 slices of 16
    # units (4 waves), half the per-step vector reads of one 128-row group
    d = g.make_desc(L.RNN_LSTM, 128, 128, 2048, 2048, L.RNN_BF16)
    st, pl = _plan(d, 0)
    assert st == L.RNN_OK
    assert (pl.groups, pl.rows, pl.slices, pl.units, pl.waves) == (2, 64, 128, 16, 4)
    assert pl.workgroups == 256 and pl.stepwise == 0


def test_large_gru_bptt_plan_eight_waves():
    # reset-after GRU B = 128, H = 2048 bf16 BPTT: 64-row groups on the
    # 8-wave kernel (two waves per SIMD issue its MFMAs at the full rate)
    d = g.make_desc(L.RNN_GRU, 128, 128, 2048, 2048, L.RNN_BF16, reset_after=1)
    st, pl = _plan(d, 1)
    assert st == L.RNN_OK
    assert (pl.groups, pl.rows, pl.slices, pl.units, pl.waves) == (2, 64, 128, 16, 8)


def test_coresidency_refusal_with_injected_cu_count():
    d = g.make_desc(L.RNN_LSTM, 256, 64, 1024, 1024, L.RNN_BF16)
    # half the chip: the planner still finds a grid that fits (16-row groups)
    st, pl = _plan(d, 0, cu=128)
    assert st == L.RNN_OK and pl.workgroups <= 128 and pl.stepwise == 0
    # 16 CUs cannot hold W_hh (8 MiB) in the registers of a co-resident grid:
    # no persistent grid, the layer takes the per-step path
    for cu in (16, 31):
        for p in (0, 1):
            st, pl = _plan(d, p, cu=cu)
            assert st == L.RNN_OK and pl.stepwise == 1, (cu, p)
            assert pl.workgroups == 0 and pl.blocks == 0 and pl.fused_dw == 0


def test_stepwise_descriptor_field():
    """`stepwise` = 1 asks for the per-step path on any shape; values other
    than 0 and 1 are refused; the plan query reports the path taken."""
    for mode, ra, H, dt in ((L.RNN_LSTM, 1, 1024, L.RNN_BF16), (L.RNN_GRU, 1, 256, L.RNN_F32),
                            (L.RNN_GRU, 0, 256, L.RNN_F32)):
        d = g.make_desc(mode, 64, 16, 256, H, dt, reset_after=ra, stepwise=1)
        assert g.rnn_workspace_bytes(d) > 0
        for p in (0, 1):
            st, pl = _plan(d, p)
            assert st == L.RNN_OK and pl.stepwise == 1 and pl.groups == 0 and pl.fused_dw == 0
        d0 = g.make_desc(mode, 64, 16, 256, H, dt, reset_after=ra)
        st, pl = _plan(d0, 1)
        assert st == L.RNN_OK and pl.stepwise == 0 and pl.groups > 0
    bad = g.make_desc(L.RNN_LSTM, 8, 2, 16, 32, L.RNN_F32, stepwise=2)
    assert g.rnn_workspace_bytes(bad) == 0


def test_shapes_beyond_the_plan_table_take_the_per_step_path():
    """fp32 H = 1024 and 2048 (W_hh 16 / 64 MiB), the basic GRU at H = 1024
    fp32, bf16 H = 4096: no persistent plan, per-step path."""
    for mode, ra, H, dt in ((L.RNN_LSTM, 1, 1024, L.RNN_F32), (L.RNN_GRU, 1, 2048, L.RNN_F32),
                            (L.RNN_GRU, 0, 1024, L.RNN_F32), (L.RNN_LSTM, 1, 4096, L.RNN_BF16)):
        d = g.make_desc(mode, 16, 64, 256, H, dt, reset_after=ra)
        assert g.rnn_workspace_bytes(d) > 0
        for p in (0, 1):
            st, pl = _plan(d, p)
            assert st == L.RNN_OK and pl.stepwise == 1, (mode, ra, H, dt, p)


def test_bidirectional_layer_shares_one_launch():
    d = g.make_desc(L.RNN_LSTM, 512, 32, 512, 512, L.RNN_F32, direction=2)
    for p in (0, 1):
        st, pl = _plan(d, p)
        assert st == L.RNN_OK and pl.dual == 1
        assert pl.workgroups == 2 * pl.groups * pl.slices <= 256


def test_plan_query_argument_errors():
    d = g.make_desc(L.RNN_LSTM, 8, 2, 16, 32, L.RNN_F32)
    assert L.rnn_plan_query(d, 2, 256, 1)[0] == L.RNN_ERR_INVALID_ARG
    assert L.rnn_plan_query(d, 0, -1, 1)[0] == L.RNN_ERR_INVALID_ARG
    assert L.rnn_plan_query(d, 0, 256, -1)[0] == L.RNN_ERR_INVALID_ARG
    assert L.lib().rnn_plan_query(ctypes.byref(d), 0, 256, 1, None) == L.RNN_ERR_INVALID_ARG
    assert L.rnn_plan_query(_desc(H=40), 0, 256, 1)[0] == L.RNN_ERR_UNSUPPORTED


def test_fused_weight_gradient_plans():
    """The BPTT kernel accumulates dW_hh for the small fp32 layers (both
    reset-after GRU and LSTM shapes), not for bf16, the basic GRU or when
    the descriptor asks for the separate product; the workspace holds the
    per-group partials only where the fusion can apply."""
    cases = [
        # (mode, reset_after, T, B, I, H, dtype, fused)
        (L.RNN_LSTM, 1, 8, 2, 16, 32, L.RNN_F32, 1),
        (L.RNN_GRU, 1, 64, 16, 256, 256, L.RNN_F32, 1),
        (L.RNN_GRU, 0, 64, 16, 256, 256, L.RNN_F32, 0),
        (L.RNN_LSTM, 1, 256, 64, 1024, 1024, L.RNN_BF16, 0),
        (L.RNN_LSTM, 1, 512, 32, 512, 512, L.RNN_F32, 0),
    ]
    for mode, ra, T, B, I, H, dt, fused in cases:
        d = g.make_desc(mode, T, B, I, H, dt, reset_after=ra)
        st, pl = _plan(d, 1)
        assert st == L.RNN_OK
        assert pl.fused_dw == fused, (mode, ra, H, dt)
        st, pl = _plan(d, 0)
        assert st == L.RNN_OK and pl.fused_dw == 0
        sep = g.make_desc(mode, T, B, I, H, dt, reset_after=ra, dw_hh_mode=1)
        st, pl = _plan(sep, 1)
        assert st == L.RNN_OK and pl.fused_dw == 0
        n_auto, n_sep = g.rnn_workspace_bytes(d), g.rnn_workspace_bytes(sep)
        if fused:
            # ceil(B / 4) groups of K x (H + 1) fp32 partials (dW_hh and db_hh) at most
            K = (4 if mode == L.RNN_LSTM else 3) * H
            assert n_sep < n_auto <= n_sep + ((B + 3) // 4) * K * (H + 1) * 4 + 4096
        bad = g.make_desc(mode, T, B, I, H, dt, reset_after=ra, dw_hh_mode=2)
        assert g.rnn_workspace_bytes(bad) == 0
