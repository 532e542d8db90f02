"""Host logic of the profile summariser: every dispatch of a layer step gets
the step it performs from its place in the dispatch order."""
from gru_layer_fwd_amd.prof_summary import step_labels


def test_step_labels_follow_dispatch_order():
    step = ["fill_i32", "gemm_kernel<proj>", "rec_fwd<...>",
            "fill_i32", "weight_transpose<W_hh>", "rec_bwd<...>",
            "weight_transpose<W_ih>", "gemm_kernel<dx>", "gather_transpose<x>", "gather_transpose<h>",
            "gemm_kernel<dW>", "splitk_finish", "rowsum_finish"]
    want = ["fill", "proj_gemm", "rec_fwd",
            "fill", "rec_bwd (W_hh transpose)", "rec_bwd",
            "dx_gemm (W_ih transpose)", "dx_gemm", "dw_gemm (transposes)", "dw_gemm (transposes)",
            "dw_gemm", "dw_gemm (finish)", "dw_gemm (finish)"]
    # two steps in a row: the second starts over at its fill
    assert step_labels(step + step) == want + want
    # bidirectional layer: one input-gradient product per direction
    bi = ["rec_bwd<...>", "gemm_kernel<dx dir 0>", "gemm_kernel<dx dir 1>", "gather_transpose<x>", "gemm_kernel<dW>"]
    assert step_labels(bi, dx_gemms=2)[1:] == ["dx_gemm", "dx_gemm", "dw_gemm (transposes)", "dw_gemm"]
    # the combined split-K / row-sum finishing pass
    assert step_labels(["rec_bwd<...>", "gemm_kernel<dx>", "gemm_kernel<dW>", "gemm_finish<bf16>"])[-1] \
        == "dw_gemm (finish)"
    # fused recurrent-weight gradient: the partial sums' finishing pass
    assert step_labels(["rec_bwd<...>", "gemm_kernel<dx>", "gemm_kernel<dW_ih>", "dw_partials_finish<float>"])[-1] \
        == "dw_gemm (finish)"


def test_counter_tables_from_a_multi_counter_pass(tmp_path):
    """Several counters per dispatch: grouped per kernel and step, with the
    MFMA busy share and the issued-over-algorithmic FLOP ratio derived."""
    from gru_layer_fwd_amd.prof_summary import counter_lines, read_counter_set
    rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
    disp = [(1, "gemm_kernel<proj>"), (2, "rec_fwd<x>")]
    vals = {"gemm_kernel<proj>": {"SQ_VALU_MFMA_BUSY_CYCLES": 512.0e3, "GRBM_GUI_ACTIVE": 8.0e3,
                                  "SQ_INSTS_VALU_MFMA_MOPS_BF16": 2.0 * 16 * 128 * 16 / 512},
            "rec_fwd<x>": {"SQ_VALU_MFMA_BUSY_CYCLES": 256.0e3, "GRBM_GUI_ACTIVE": 16.0e3,
                           "SQ_INSTS_VALU_MFMA_MOPS_BF16": 2.0 * 16 * 128 * 32 / 512}}
    for i, n in disp:
        for c, v in vals[n].items():
            rows.append(f"{i},{n},{c},{v}")
    p = tmp_path / "c.csv"
    p.write_text("\n".join(rows) + "\n")
    cs = read_counter_set(str(p))
    assert cs[("gemm_kernel<proj>", "proj_gemm")]["GRBM_GUI_ACTIVE"] == 8.0e3
    assert cs[("rec_fwd<x>", "rec_fwd")]["SQ_VALU_MFMA_BUSY_CYCLES"] == 256.0e3
    # the tiny LSTM workload (T=8, B=2, I=16, H=32): proj = 2*16*128*16 FLOPs
    text = "\n".join(counter_lines([str(p)], "lstm_f32_t8_b2_i16_h32", cus=256, simds=4, xcds=8))
    proj = next(line for line in text.splitlines() if "proj_gemm" in line).split(" | ")
    rec = next(line for line in text.splitlines() if "rec_fwd" in line).split(" | ")
    assert proj[-4] == "50.0"          # 512e3 / (8e3 / 8 * 1024)
    assert proj[-1].rstrip(" |") == "1.00"  # issued 65536 = algorithmic 2*16*128*16
    assert rec[-4] == "12.5"           # 256e3 / (16e3 / 8 * 1024)
    assert rec[-1].rstrip(" |") == "1.00"   # 2*16*128*32
