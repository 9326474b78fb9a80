"""The draws of test_gpu_maps.py move the maps enough to tell a right
Sinkhorn from a wrong one (CPU, oracle only).

For each draw the GPU cases use, the oracle's H_res under the right
procedure (columns then rows, the round count asked for, the row clamp for
xHC) is compared with the same oracle under a plausible mistake: another
round count, rows normalised first (at 1 and 3 rounds: after 20 both orders
are near the same limit), no clamp.  Every mistake must move H_res
by at least ten times the fp32 bar in the metric the GPU cases use, so that
a GPU doing it fails them.  At the workloads' own draw (alpha = 0.01,
biases 0) some of these differences fall under the bar, which is why those
cases exist.  Also checked: the lag-0 kernels really make each branch
nearly parallel to the output, and Gram-Schmidt then changes the write by
far more than the bar; the zero kernels make the write the output alone.

Explainer "xHC: sixteen residual streams, four written at a time",
sections "mHC: keep the mixing doubly stochastic" and "Which constraint
survives".
"""
import numpy as np
import pytest

import cases as K
import test_gpu_maps as M
from oracle import hc_oracle as O
from stream_residual_mixing_amd import synth
from stream_residual_mixing_amd.binding import Config

BAR = 10 * K.TOL["f32"]


def xhc_res_logits(cfg, seed, alpha_res, affine=False):
    """The k x k residual logits of an xHC draw (oracle steps: routing, the
    active rows, their RMSNorm and projection)."""
    wd = synth.xhc_stress_weights(seed, 0, cfg.N, cfg.k, cfg.C, cfg.K_r, cfg.dtype, alpha_res=alpha_res)
    ow = K.oracle_weights(wd)
    X = K.f64(synth.state(seed, cfg.T, cfg.N, cfg.C, cfg.dtype, affine=affine))
    pre = O.xhc_pre(X, ow["w_full"], ow["w_act"], cfg.m, cfg.k, cfg.K_r, (1.0, alpha_res, 1.0), ow["b_pre"],
                    ow["b_res"], ow["b_post"], iters=cfg.iters)
    Xa = np.take_along_axis(X, pre["I"][:, :, None], axis=1)
    la = O.rms_normalize(Xa.reshape(cfg.T, -1)) @ ow["w_act"][:, : cfg.k * cfg.k]
    return alpha_res * la.reshape(cfg.T, cfg.k, cfg.k) + ow["b_res"].reshape(cfg.k, cfg.k), pre


def mhc_res_logits(N, C, seed, alpha_res, dtype, affine=False):
    wd = synth.mhc_stress_weights(seed, 0, N, C, dtype, alpha_res=alpha_res)
    ow = K.oracle_weights(wd)
    X = K.f64(synth.state(seed, 74, N, C, dtype, affine=affine))
    xn = O.rms_normalize(X.reshape(74, -1))
    lr = xn @ ow["w_full"][:, 2 * N:]
    return alpha_res * lr.reshape(74, N, N) + ow["b_res"].reshape(N, N)


def rows_first(L, iters):
    """Sinkhorn with rows normalised before columns in every round."""
    return np.swapaxes(O.sinkhorn(np.swapaxes(L, -1, -2), iters), -1, -2)


def check_separation(L, clamp):
    fix = O.row_clamp if clamp else (lambda H: H)
    right = {it: fix(O.sinkhorn(L, it)) for it in (0, 1, 3, 20)}
    for a in right:
        for b in right:
            if a < b:
                d = K.rel_err(right[a], right[b])
                assert d >= BAR, f"{a} and {b} rounds differ by {d:.2e} only"
    # after twenty rounds both orders are close to the same doubly
    # stochastic limit; the order is pinned by the 1- and 3-round cases
    for it in (1, 3):
        d = K.rel_err(fix(rows_first(L, it)), right[it])
        assert d >= BAR, f"rows first at {it} rounds differs by {d:.2e} only"
    if clamp:
        d = K.rel_err(O.sinkhorn(L, 0), right[0])
        assert d >= BAR, f"the clamp changes the 0-round map by {d:.2e} only"


@pytest.mark.parametrize("alpha_res", [1.0, 4.0])
@pytest.mark.parametrize("mlp", [False, True])
def test_xhc_draws_separate_the_alternatives(alpha_res, mlp):
    """Every per-sublayer draw of the round-count cases, and the scaled and
    offset state rows."""
    for iters in (0, 1, 3, 20):
        cfg = Config(N=16, k=4, m=2, C=256, B=2, S=37, n_convs=3 if mlp else 0, iters=iters, dtype="f32")
        L, _ = xhc_res_logits(cfg, M.seed_rounds(iters, alpha_res, mlp), alpha_res)
        check_separation(L, clamp=True)
    cfg = Config(N=16, k=4, m=2, C=256, B=2, S=37, n_convs=3 if mlp else 0, dtype="f32")
    L, _ = xhc_res_logits(cfg, M.seed_affine(mlp), 4.0, affine=True)
    check_separation(L, clamp=True)


@pytest.mark.parametrize("N,k,m", [(16, 2, 1), (8, 4, 2), (4, 4, 4), (16, 4, 0)])
def test_xhc_draws_separate_other_shapes(N, k, m):
    cfg = Config(N=N, k=k, m=m, C=192, B=2, S=29, n_convs=3, iters=3, dtype="f32")
    L, _ = xhc_res_logits(cfg, M.seed_shape(N, k, m), 4.0)
    check_separation(L, clamp=True)


@pytest.mark.parametrize("alpha_res", [1.0, 4.0])
@pytest.mark.parametrize("N", [4, 16])
def test_mhc_draws_separate_the_alternatives(N, alpha_res):
    for iters in (0, 1, 3, 20):
        L = mhc_res_logits(N, 256, M.seed_mhc(N, iters, alpha_res), alpha_res, "f32")
        check_separation(L, clamp=False)
    L = mhc_res_logits(N, 256, M.seed_mhc_affine(N), 4.0, "f32", affine=True)
    check_separation(L, clamp=False)


def test_c4096_draws_separate_the_alternatives():
    """The benchmark-width draws: the per-sublayer case (residual scale 4,
    20 rounds, scaled and offset rows) and the first layer of the chain
    (residual scale 1, 3 rounds)."""
    cfg = Config(N=16, k=4, m=2, C=4096, B=1, S=48, n_convs=3, dtype="bf16")
    L, _ = xhc_res_logits(cfg, 260, 4.0, affine=True)
    check_separation(L, clamp=True)
    cfg = Config(N=16, k=4, m=2, C=4096, B=1, S=96, n_convs=3, iters=3, dtype="bf16")
    L, _ = xhc_res_logits(cfg, 280, 1.0)
    check_separation(L, clamp=True)


def test_workload_draw_hides_the_round_count():
    """At alpha = 0.01 and zero biases one round and twenty differ by less
    than the fp32 bar: the reason the draws above exist."""
    cfg = Config(N=16, k=4, m=2, C=512, B=2, S=37, n_convs=3, dtype="f32")
    wd = synth.xhc_layer_weights(83, 0, cfg.N, cfg.k, cfg.C, cfg.K_r, cfg.dtype)
    ow = K.oracle_weights(wd)
    X = K.f64(synth.state(83, cfg.T, cfg.N, cfg.C, cfg.dtype))
    h = [O.xhc_pre(X, ow["w_full"], ow["w_act"], 2, 4, 4, (0.01, 0.01, 0.01), ow["b_pre"], ow["b_res"],
                   ow["b_post"], iters=it)["h_res"] for it in (1, 20)]
    assert K.rel_err(h[0], h[1]) < K.TOL["f32"]


def test_lag0_kernels_make_branches_parallel_and_gram_schmidt_matter():
    C, S = 256, 37
    ks = synth.conv_kernels_lag0(231, 0, C)    # the lag-0 case of test_gpu_maps
    out = K.f64(synth.sublayer_out(231, 0, 2, S, C, "f32"))
    comps = [O.causal_dwconv(out, K.f64(w)) for w in ks]
    for g in comps:
        cos = np.sum(g * out, -1) / (np.linalg.norm(g, axis=-1) * np.linalg.norm(out, axis=-1))
        assert cos.min() >= 0.95, cos.min()
    with_mgs = O.xhc_write_basis(out, [K.f64(w) for w in ks], use_mgs=True)
    without = O.xhc_write_basis(out, [K.f64(w) for w in ks], use_mgs=False)
    assert K.rel_err(np.stack(with_mgs), np.stack(without)) >= BAR


def test_zero_kernels_write_only_the_output():
    """With every kernel zero the branches vanish and so do their Gram-Schmidt
    residuals: the write of position j is p_j H_post[j][0] out."""
    cfg = Config(N=16, k=4, m=2, C=256, B=2, S=37, n_convs=3, dtype="f32")
    wd = synth.xhc_stress_weights(230, 0, cfg.N, cfg.k, cfg.C, cfg.K_r, cfg.dtype, conv="zero")
    ow = K.oracle_weights(wd)
    X = K.f64(synth.state(230, cfg.T, cfg.N, cfg.C, cfg.dtype))
    out = K.f64(synth.sublayer_out(230, 0, cfg.B, cfg.S, cfg.C, cfg.dtype))
    r = K.oracle_xhc(cfg, X, out, ow, dtype="f64")
    Xa = np.take_along_axis(X, r["I"][:, :, None], axis=1)
    mix = np.einsum("tji,tic->tjc", r["h_res"], Xa)
    write = (r["p"] * r["h_post"][:, :, 0])[:, :, None] * out.reshape(cfg.T, 1, cfg.C)
    got = np.take_along_axis(r["X"], r["I"][:, :, None], axis=1)
    np.testing.assert_allclose(got, mix + write, rtol=1e-12, atol=1e-12)
