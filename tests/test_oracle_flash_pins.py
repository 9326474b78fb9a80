"""Pins of the oracle's xHC-Flash block against what the pages and
mathematics fix (xHC paper, "xHC-Flash" section, Eqs. 17-19 and Appendix
E.1; explainer "xHC: sixteen residual streams, four written at a time",
section "What it costs").

None of these retypes the oracle's formulas: the Eq. 19 correction is
checked against the dense read of the rewritten state it replaces, the
attention write and the MLP maps against the separately pinned full-xHC
functions, the whole block against the scalar-loop derivation of
``brute_force.py`` and against the plain residual it reduces to.
"""
import numpy as np
import pytest

import brute_force as BF
from oracle import hc_oracle as O


def rng(*k):
    return np.random.default_rng(list(k))


def flash_inputs(r, T, N, k, C, K_r, B=1, wstd=0.3):
    S = T // B
    return dict(
        X=r.standard_normal((T, N, C)),
        out_a=r.standard_normal((B, S, C)),
        out_m=r.standard_normal((B, S, C)),
        W_full=r.standard_normal((N * C, 3 * N)) * wstd,
        W_pa=r.standard_normal((k * C, k)) * wstd,
        W_am=r.standard_normal((k * C, k * k + k * K_r)) * wstd,
        convs=[r.standard_normal((kap, C)) / kap for kap in (4, 8, 12)][: K_r - 1],
        b_pa=r.standard_normal(N) * 0.1, b_pm=r.standard_normal(N) * 0.1, b_po=r.standard_normal(k) * 0.1,
        b_res=r.standard_normal(k * k) * 0.1, b_pm2=r.standard_normal(k * K_r) * 0.1,
        alpha=(0.7, 0.9, 0.8, 1.1, 0.6),
    )


def run_block(d, m, k, dtype="f64", iters=20):
    return O.xhcf_block(d["X"], d["out_a"], d["out_m"], d["W_full"], d["W_pa"], d["W_am"], m, k, d["convs"],
                        d["alpha"], d["b_pa"], d["b_pm"], d["b_po"], d["b_res"], d["b_pm2"], iters=iters,
                        dtype=dtype)


def test_corrected_mlp_input_is_the_dense_read_of_the_rewritten_state():
    """Appendix E.1: with routing and the MLP pre-map fixed at the block
    entry, the base readout plus the Eq. 19 scalar times out_A equals the
    MLP pre-map applied to the state after the attention write.  Exact in
    real arithmetic; a dropped router weight, a pre-map read at position j
    instead of stream I_j, or a missing post-map factor all break it."""
    r = rng(11)
    T, N, k, m, C = 40, 16, 4, 2, 24
    d = flash_inputs(r, T, N, k, C, 1, wstd=0.5)
    pre = O.xhcf_pre(d["X"], d["W_full"], d["W_pa"], m, k, d["alpha"][:3], d["b_pa"], d["b_pm"], d["b_po"])
    out_a = d["out_a"].reshape(T, C)
    X1 = O.xhcf_attn_write(d["X"], out_a, pre["I"], pre["p"], pre["h_post_attn"])
    direct = np.einsum("tn,tnc->tc", pre["h_pre_mlp"], X1)
    corr, a = O.xhcf_mlp_input(pre["inp_mlp"], out_a, pre["I"], pre["p"], pre["h_pre_mlp"], pre["h_post_attn"])
    np.testing.assert_allclose(corr, direct, rtol=0, atol=1e-12 * np.abs(direct).max())
    # routed gates are genuinely below one, so the test sees p
    assert np.all(pre["p"][:, m:] < 1.0) and np.all(pre["p"][:, :m] == 1.0)
    assert np.all(a > 0)


def test_attention_write_is_the_unmixed_sparse_write():
    """Eq. 18: the attention sublayer of xHC-Flash is full xHC's write with
    the residual map replaced by the identity, K_r = 1 (checked against the
    separately pinned full-xHC post), and touches only the active rows."""
    r = rng(12)
    T, N, k, m, C = 12, 8, 4, 2, 16
    X = r.standard_normal((T, N, C))
    out = r.standard_normal((1, T, C))
    I = np.stack([np.concatenate([[0, 1], r.choice(np.arange(2, N), 2, replace=False)]) for _ in range(T)])
    p = np.concatenate([np.ones((T, 2)), r.uniform(0.1, 0.9, (T, 2))], axis=1)
    hpo = r.uniform(0.2, 1.8, (T, k))
    got = O.xhcf_attn_write(X, out.reshape(T, C), I, p, hpo)
    ref = O.xhc_post(X, out, I, p, np.tile(np.eye(k), (T, 1, 1)), hpo[:, :, None])
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-14)
    # one token by hand: stream I_2 gains p_2 * h_2 * out, the rest of the token is untouched
    t = 3
    hand = X[t].copy()
    for j in range(k):
        hand[I[t, j]] = X[t, I[t, j]] + p[t, j] * hpo[t, j] * out[0, t]
    np.testing.assert_array_equal(got[t], hand)


def test_mlp_maps_equal_full_xhc_active_maps():
    """The MLP's active maps are full xHC's active-map generation: with every
    stream active (k = m = N, so both sides use the same rows in the same
    order) they equal the H_res and H_post of the full-xHC pre stage."""
    r = rng(13)
    T, N, C, K_r = 9, 4, 32, 4
    X1 = r.standard_normal((T, N, C))
    W_act = r.standard_normal((N * C, N * N + N * K_r)) * 0.3
    W_full = r.standard_normal((N * C, 2 * N)) * 0.3
    b_res, b_post = r.standard_normal(N * N) * 0.1, r.standard_normal(N * K_r) * 0.1
    I = np.tile(np.arange(N), (T, 1))
    h_res, h_post = O.xhcf_mlp_maps(X1, I, W_act, K_r, 1.3, 0.7, b_res, b_post, iters=20)
    ref = O.xhc_pre(X1, W_full, W_act, N, N, K_r, (0.5, 1.3, 0.7), np.zeros(N), b_res, b_post, iters=20)
    np.testing.assert_allclose(h_res, ref["h_res"], rtol=1e-13, atol=0)
    np.testing.assert_allclose(h_post, ref["h_post"], rtol=1e-13, atol=0)


def test_one_stream_block_is_two_plain_residual_steps():
    """With one stream, unit maps and zero conv kernels a Flash block is the
    plain residual twice: inp_A = x, the MLP input = x + out_A and the new
    state x + out_A + out_M (the single-stream special case of the pages'
    hyper-connections; sigmoid(40) is 1 in float64, 2 sigmoid(0) = 1, a 1 x 1
    Sinkhorn map is 1)."""
    r = rng(14)
    T, C = 20, 32
    d = flash_inputs(r, T, 1, 1, C, 4)
    d.update(b_pa=np.full(1, 40.0), b_pm=np.full(1, 40.0), b_po=np.zeros(1), b_res=np.zeros(1),
             b_pm2=np.zeros(4), alpha=(0.0, 0.0, 0.0, 0.0, 0.0),
             convs=[np.zeros((kap, C)) for kap in (4, 8, 12)])
    res = run_block(d, 1, 1)
    x = d["X"][:, 0, :]
    oa, om = d["out_a"].reshape(T, C), d["out_m"].reshape(T, C)
    np.testing.assert_array_equal(res["inp_attn"], x)
    np.testing.assert_allclose(res["inp_mlp"], x + oa, rtol=0, atol=4e-16 * 8)
    np.testing.assert_allclose(res["X"][:, 0, :], x + oa + om, rtol=0, atol=4e-16 * 16)


def test_block_changes_exactly_the_active_rows():
    """Both writes of a block touch only the k streams of the shared active
    list; every other stream passes through bit for bit."""
    r = rng(15)
    T, N, k, m, C = 30, 16, 4, 2, 16
    d = flash_inputs(r, T, N, k, C, 4, B=2)
    X0 = O.round_state(d["X"], "bf16")
    d["X"] = X0
    res = run_block(d, m, k, dtype="bf16")
    for t in range(T):
        act = set(res["I"][t].tolist())
        for i in range(N):
            same = np.array_equal(res["X"][t, i], X0[t, i])
            assert same == (i not in act), (t, i)


def test_swapping_the_pre_map_columns_swaps_the_readouts():
    """The two pre-maps are separate column blocks of one projection: trading
    the blocks (and their biases and scales) trades the two readouts."""
    r = rng(16)
    T, N, k, m, C = 10, 8, 4, 2, 16
    d = flash_inputs(r, T, N, k, C, 1)
    a = d["alpha"]
    p1 = O.xhcf_pre(d["X"], d["W_full"], d["W_pa"], m, k, (a[0], a[1], a[2]), d["b_pa"], d["b_pm"], d["b_po"])
    W2 = np.concatenate([d["W_full"][:, :N], d["W_full"][:, 2 * N:], d["W_full"][:, N:2 * N]], axis=1)
    p2 = O.xhcf_pre(d["X"], W2, d["W_pa"], m, k, (a[1], a[0], a[2]), d["b_pm"], d["b_pa"], d["b_po"])
    np.testing.assert_array_equal(p1["inp_attn"], p2["inp_mlp"])
    np.testing.assert_array_equal(p1["inp_mlp"], p2["inp_attn"])
    np.testing.assert_array_equal(p1["I"], p2["I"])


@pytest.mark.parametrize("mlp_convs", [3, 0])
def test_flash_block_matches_scalar_brute_force(mlp_convs):
    """The vectorised block against the scalar-loop derivation (top-k by
    subset enumeration, the MLP input as the dense read of the rewritten
    state, explicit convolution lags and Gram-Schmidt dot products) on tiny
    shapes with two batch items."""
    r = rng(17, mlp_convs)
    B, S, N, k, m, C = 2, 14, 6, 3, 1, 8
    T = B * S
    K_r = 1 + mlp_convs
    d = flash_inputs(r, T, N, k, C, K_r, B=B, wstd=0.4)
    res = run_block(d, m, k)
    bf = BF.xhcf_block(d["X"].tolist(), d["out_a"].tolist(), d["out_m"].tolist(), d["W_full"].tolist(),
                       d["W_pa"].tolist(), d["W_am"].tolist(), m, k, [w.tolist() for w in d["convs"]],
                       d["alpha"], d["b_pa"].tolist(), d["b_pm"].tolist(), d["b_po"].tolist(),
                       d["b_res"].tolist(), d["b_pm2"].tolist(), 20)
    np.testing.assert_array_equal(res["I"], np.array(bf["I"]))
    for key, ref in (("p", bf["p"]), ("inp_attn", bf["inp_attn"]), ("inp_mlp", bf["inp_mlp"]),
                     ("X1", bf["X1"]), ("X", bf["X"]), ("alpha", bf["alpha_corr"])):
        ref = np.array(ref)
        np.testing.assert_allclose(res[key], ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max(), err_msg=key)


# ---------------------------------------------------------------- xHC-Flash-4sub

def flash4_inputs(r, T, N, k, C, B=1, wstd=0.3):
    S = T // B
    return dict(
        X=r.standard_normal((T, N, C)),
        outs=[r.standard_normal((B, S, C)) for _ in range(4)],
        W_full=r.standard_normal((N * C, 5 * N)) * wstd,
        W_posts=[r.standard_normal((k * C, k)) * wstd, r.standard_normal((k * C, 4 * k)) * wstd,
                 r.standard_normal((k * C, k)) * wstd],
        W_act_last=r.standard_normal((k * C, k * k + 4 * k)) * wstd,
        convs=[[r.standard_normal((kap, C)) / kap for kap in (4, 8, 12)] for _ in range(2)],
        alpha=dict(pre=(0.7, 0.9, 0.6, 1.2), post=(0.8, 0.5, 1.1, 0.6), res=1.1),
        b=dict(pre=[r.standard_normal(N) * 0.1 for _ in range(4)],
               post=[r.standard_normal(k) * 0.1, r.standard_normal(4 * k) * 0.1, r.standard_normal(k) * 0.1,
                     r.standard_normal(4 * k) * 0.1], res=r.standard_normal(k * k) * 0.1),
    )


def run_group(d, m, k, dtype="f64"):
    return O.xhcf4_group(d["X"], d["outs"], d["W_full"], d["W_posts"], d["W_act_last"], m, k, d["convs"],
                         d["alpha"], d["b"], dtype=dtype)


def test_4sub_inputs_are_dense_reads_of_the_current_state():
    """Appendix E.2: with routing and the four pre-maps fixed at the group
    entry and no residual mixing before the last sublayer, each sublayer's
    input (non-active base + pre-map on the current active rows) equals that
    pre-map applied to the whole state as it stands before the sublayer."""
    r = rng(21)
    T, N, k, m, C = 24, 16, 4, 2, 16
    d = flash4_inputs(r, T, N, k, C, B=2)
    g = run_group(d, m, k)
    prev = [d["X"]] + g["states"][:3]
    for q in range(4):
        direct = np.einsum("tn,tnc->tc", g["h_pre"][q], prev[q])
        np.testing.assert_allclose(g["inputs"][q], direct, rtol=0, atol=1e-12 * np.abs(direct).max(), err_msg=str(q))


def test_4sub_first_two_sublayers_are_an_xhc_flash_block():
    """Up to the second sublayer's input, a 4-sublayer group is an xHC-Flash
    block with the same router, first two pre-maps and attention post-map:
    same routing, same attention input and write, and the MLP input of the
    Eq. 19 correction equals the active-state form."""
    r = rng(22)
    T, N, k, m, C = 20, 8, 4, 2, 16
    d = flash4_inputs(r, T, N, k, C)
    g = run_group(d, m, k)
    a = d["alpha"]
    fl = O.xhcf_block(d["X"], d["outs"][0], d["outs"][1], d["W_full"][:, :3 * N], d["W_posts"][0],
                      d["W_act_last"], m, k, d["convs"][0], (a["pre"][0], a["pre"][1], a["post"][0], a["res"],
                                                             a["post"][3]),
                      d["b"]["pre"][0], d["b"]["pre"][1], d["b"]["post"][0], d["b"]["res"], d["b"]["post"][3])
    np.testing.assert_array_equal(g["I"], fl["I"])
    np.testing.assert_allclose(g["inputs"][0], fl["inp_attn"], rtol=1e-13)
    np.testing.assert_allclose(g["maps"][0]["h_post"][:, :, 0], fl["h_post_attn"], rtol=1e-13)
    np.testing.assert_allclose(g["states"][0], fl["X1"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(g["inputs"][1], fl["inp_mlp"], rtol=1e-12, atol=1e-12)


def test_4sub_unmixed_mlp_post_map_addresses_position_and_component():
    """The unmixed MLP post-map reads column j*K_r + r for position j and
    component r: a weight with one non-zero column moves only that entry."""
    r = rng(23)
    T, k, C, K_r = 5, 4, 8, 4
    Xa = r.standard_normal((T, k, C))
    for j, rr in ((0, 0), (2, 3), (3, 1)):
        W = np.zeros((k * C, k * K_r))
        W[:, j * K_r + rr] = r.standard_normal(k * C)
        h = O.xhcf4_post_map(Xa, W, K_r, 0.9, np.zeros(k * K_r))
        moved = np.abs(h - 1.0) > 1e-12
        assert moved[:, j, rr].all() and moved.sum() == T


def test_4sub_one_stream_is_four_plain_residual_steps():
    r = rng(24)
    T, C = 12, 16
    d = flash4_inputs(r, T, 1, 1, C)
    d.update(alpha=dict(pre=(0.0,) * 4, post=(0.0,) * 4, res=0.0),
             b=dict(pre=[np.full(1, 40.0)] * 4, post=[np.zeros(1), np.zeros(4), np.zeros(1), np.zeros(4)],
                    res=np.zeros(1)),
             convs=[[np.zeros((kap, C)) for kap in (4, 8, 12)] for _ in range(2)])
    g = run_group(d, 1, 1)
    x = d["X"][:, 0, :]
    o = [v.reshape(T, C) for v in d["outs"]]
    run = x.copy()
    for q in range(4):
        np.testing.assert_allclose(g["inputs"][q], run, rtol=0, atol=1e-14)
        run = run + o[q]
        np.testing.assert_allclose(g["states"][q][:, 0, :], run, rtol=0, atol=1e-14)


def test_4sub_changes_only_the_shared_active_rows():
    r = rng(25)
    T, N, k, m, C = 16, 16, 4, 2, 16
    d = flash4_inputs(r, T, N, k, C)
    d["X"] = O.round_state(d["X"], "bf16")
    g = run_group(d, m, k, dtype="bf16")
    for t in range(T):
        act = set(g["I"][t].tolist())
        for i in range(N):
            assert np.array_equal(g["states"][3][t, i], d["X"][t, i]) == (i not in act), (t, i)
