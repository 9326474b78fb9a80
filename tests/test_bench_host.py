"""Host logic of bench.py (no GPU): the byte models, the grouping of counter
dispatches into calls, and the refusal of more than one GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from stream_residual_mixing_amd.binding import Config  # noqa: E402


def test_layer_byte_models():
    cfg = Config(N=16, k=4, m=2, C=4096, B=2, S=8192, n_convs=3, dtype="bf16")
    C2 = 4096 * 2
    assert bench.bytes_per_token("xhc", cfg) == (17 * C2, 9 * C2)          # 26C per layer
    assert bench.bytes_per_token("xhcb", cfg) == (23 * C2, 45 * C2)        # backward: (N + k + 3)C, (3N - k + 1)C
    assert sum(bench.flash_bytes_per_token(cfg)) == 54 * C2                # Flash: 54C per block
    assert sum(bench.flash4_bytes_per_token(cfg)) == 90 * C2               # 4sub: 90C per group


def test_backward_dispatches_group_into_calls():
    k = "xhc::"
    rows = [(f"void {k}xhc_prep_kernel<Bf16>", 1.0), (f"void {k}xhc_pre_fused_kernel<Bf16, 16, 4, 4>", 1.0),
            (f"void {k}xhc_pre_fused_kernel<Bf16, 16, 4, 1>", 1.0), ("normal_kernel", 5.0)]
    # a large set-up xhc_pre: the routing pass, then the last-sublayer pre pass
    rows += [(f"void {k}{n}", 1.0) for n in ("xhc_prep_kernel<Bf16>", "xhc_proj_s_kernel<Bf16, 16, RouteDims<16>>",
                                             "xhc_route_fin_kernel<16, 4>", "xhc_prep_kernel<Bf16>",
                                             "xhc_pre_chained_s_kernel<Bf16, 16, 4, 4, 2, false>",
                                             "xhc_act_fin_kernel<4, 4>")]
    post_m = [f"void {k}(anonymous namespace)::bwd_apply_kernel<Bf16, 16, 4, 4>(Args)",
              f"void {k}(anonymous namespace)::bwd_conv_kernel<Bf16>(Args)", f"{k}(anonymous namespace)::bwd_reduce_kernel"]
    pre = [f"void {k}pack_b_kernel<Bf16>", f"void {k}pack_b_kernel<Bf16>", f"void {k}proj_gen_kernel<Bf16, 2>",
           f"void {k}(anonymous namespace)::bwd_token_kernel<16, 4, 4>", f"void {k}(anonymous namespace)::bwd_rows_mfma_kernel<4>"]
    post_a = [f"void {k}(anonymous namespace)::bwd_apply_kernel<Bf16, 16, 4, 1>(Args)"]
    for group in (post_m, pre, post_a, pre):
        rows += [(n, 2.0) for n in group]
    calls = bench._split_backward_calls(rows)
    assert [len(c) for c in calls] == [3, 5, 1, 5]
    assert all("bwd_apply_kernel" in c[0][0] for c in (calls[0], calls[2]))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_counter_rows_split_into_calls():
    """The traffic summary groups one step's dispatches into the calls the
    bench times: route, then per layer pre and post (the attention-type post
    is the persistent pass alone, the MLP-type one starts at its Gram pass);
    for mHC, pre then post."""
    k = lambda n: (f"void xhc::{n}(xhc::Args)", 1.0)   # noqa: E731
    chain = [k("xhc_prep_kernel<xhc::Bf16>"), k("xhc_proj_p_kernel<xhc::Bf16, 16>"), k("xhc_route_fin_kernel<16, 4>"),
             k("xhc_prep_kernel<xhc::Bf16>"), k("xhc_pre_chained_p_kernel<xhc::Bf16, 16, 4, 1, 2>"),
             k("xhc_act_fin_kernel<4, 1>"),
             k("xhc_post_p_kernel<xhc::Bf16, 16, 4, 2, 1>"), k("xhc_route_fin_kernel<16, 4>"),
             k("xhc_prep_kernel<xhc::Bf16>"), k("xhc_pre_chained_kernel<xhc::Bf16, 16, 4, 4, false, 1>"),
             k("xhc_act_fin_kernel<4, 4>"),
             k("xhc_gram_kernel<xhc::Bf16>"), k("xhc_wcoef_kernel<4>"),
             k("xhc_post_p_kernel<xhc::Bf16, 16, 4, 2, 4>"), k("xhc_route_fin_kernel<16, 4>"),
             k("xhc_prep_kernel<xhc::Bf16>"), k("xhc_pre_chained_kernel<xhc::Bf16, 16, 4, 1, false, 1>"),
             k("xhc_act_fin_kernel<4, 1>"),
             k("xhc_apply_kernel<xhc::Bf16, 4, 1, 8, 0>")]
    calls = bench._split_calls(chain)
    assert [len(c) for c in calls] == [3, 3, 2, 3, 4, 3, 1]
    mhc = [k("pack_b_kernel<xhc::Bf16>"), k("mhc_proj_kernel<18>"), k("mhc_read_kernel<xhc::Bf16, 16>"),
           k("mhc_post_kernel<xhc::Bf16, 16>")]
    assert [len(c) for c in bench._split_calls(mhc)] == [3, 1]
    # the staged attention-type post pass starts its call too
    staged = [k("xhc_post_s_kernel<xhc::Bf16, 16, 4, 2, 1>"), k("xhc_route_fin_kernel<16, 4>"),
              k("xhc_prep_kernel<xhc::Bf16>"), k("xhc_pre_chained_s_kernel<xhc::Bf16, 16, 4, 4, 2, true>"),
              k("xhc_act_fin_kernel<4, 4>")]
    assert [len(c) for c in bench._split_calls(staged)] == [2, 3]
    # per-sublayer calls: a large xhc_pre is the routing pass and then the
    # pre pass, one call; the MLP-type xhc_post starts at its Gram pass
    single = [k("xhc_prep_kernel<xhc::Bf16>"), k("xhc_proj_s_kernel<xhc::Bf16, 16>"), k("xhc_route_fin_kernel<16, 4>"),
              k("xhc_prep_kernel<xhc::Bf16>"), k("xhc_pre_chained_s_kernel<xhc::Bf16, 16, 4, 4, 2, false>"),
              k("xhc_act_fin_kernel<4, 4>"), k("xhc_gram_kernel<xhc::Bf16>"),
              k("xhc_apply_kernel<xhc::Bf16, 4, 4, 6, 0>")]
    assert [len(c) for c in bench._split_calls(single, single=True)] == [6, 2]
    assert [len(c) for c in bench._split_calls(single)] == [3, 3, 2]
