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
