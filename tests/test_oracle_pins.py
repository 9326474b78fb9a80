"""Pins of the float64 oracle against what the pages and mathematics fix.

Each test states the fact it checks and where it comes from.  None of them
retypes the oracle's formula: they use closed forms, invariants, special
cases that reduce to a known result, library routines, and the independent
scalar-loop derivation in ``brute_force.py``.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import brute_force as BF
from oracle import hc_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(*k):
    return np.random.default_rng(list(k))


# ---------------------------------------------------------------- rounding

def test_bf16_rounding_matches_torch_including_ties():
    """The oracle's direct float64 -> bfloat16 rounding agrees with
    PyTorch's float32 -> bfloat16 conversion (round to nearest even) on
    float32 inputs, including exact halfway cases."""
    r = rng(1)
    x32 = (r.standard_normal(20000) * np.exp(r.uniform(-8, 8, 20000))).astype(np.float32)
    b = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    nxt = np.nextafter(b.astype(np.float32), np.float32(np.inf))
    bn = torch.from_numpy(nxt).to(torch.bfloat16).to(torch.float32).numpy()
    bn = np.where(bn == b, torch.from_numpy((b * (1 + 2 ** -7)).astype(np.float32)).to(torch.bfloat16).float().numpy(), bn)
    ties = ((b + bn) / 2).astype(np.float32)          # exactly representable midpoints
    allx = np.concatenate([x32, ties])
    ref = torch.from_numpy(allx).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_to_bf16(allx.astype(np.float64)), ref)


# ---------------------------------------------------------------- normalisation

def test_normalisations_have_their_defining_moments():
    r = rng(2)
    v = r.standard_normal((7, 300)) * 3 + 0.5
    ln = O.ln_normalize(v)
    sd = v.std(axis=1)
    np.testing.assert_allclose(ln.mean(axis=1), 0, atol=1e-13)
    np.testing.assert_allclose(ln.std(axis=1), sd / (sd + 1e-6), rtol=1e-13)
    rm = O.rms_normalize(v)
    ms = (v * v).mean(axis=1)
    np.testing.assert_allclose((rm * rm).mean(axis=1), ms / (ms + 1e-6), rtol=1e-13)


def test_sigmoid_symmetry_and_range():
    z = np.linspace(-800, 800, 4001)
    s = O.sigmoid(z)
    assert np.all(np.isfinite(s)) and s.min() >= 0 and s.max() <= 1
    np.testing.assert_allclose(O.sigmoid(-z), 1 - s, atol=1e-15)
    assert O.sigmoid(np.array([0.0]))[0] == 0.5


# ---------------------------------------------------------------- Sinkhorn

@pytest.mark.parametrize("n", [2, 4, 16])
@pytest.mark.parametrize("iters", [1, 3, 20])
def test_sinkhorn_rows_sum_to_one_exactly(n, iters):
    """Rows are normalised last, so every row sums to 1 up to rounding
    (explainer, "mHC: keep the mixing doubly stochastic")."""
    L = rng(3, n, iters).standard_normal((50, n, n)) * 3
    H = O.sinkhorn(L, iters)
    assert np.all(H > 0)
    np.testing.assert_allclose(H.sum(-1), 1, atol=4e-16 * n)


def test_sinkhorn_2x2_limit_closed_form():
    """A positive 2x2 matrix scales to [[a, 1-a], [1-a, a]] with
    a = sqrt(m11 m22) / (sqrt(m11 m22) + sqrt(m12 m21)), because row and
    column scaling leaves the cross ratio m11 m22 / (m12 m21) unchanged."""
    L = rng(4).standard_normal((40, 2, 2)) * 2
    M = np.exp(L)
    s1 = np.sqrt(M[:, 0, 0] * M[:, 1, 1])
    s2 = np.sqrt(M[:, 0, 1] * M[:, 1, 0])
    a = s1 / (s1 + s2)
    H = O.sinkhorn(L, 1000)
    np.testing.assert_allclose(H[:, 0, 0], a, atol=1e-12)
    np.testing.assert_allclose(H[:, 1, 1], a, atol=1e-12)
    np.testing.assert_allclose(H[:, 0, 1], 1 - a, atol=1e-12)


@pytest.mark.parametrize("iters", [1, 2, 20])
def test_sinkhorn_preserves_cross_ratios(iters):
    """Any sequence of row and column scalings keeps every cross ratio
    H_ij H_kl / (H_il H_kj) of exp(L); so Sinkhorn's output is
    diag(u) exp(L) diag(v), whatever the iteration count."""
    L = rng(5, iters).standard_normal((6, 5, 5)) * 2
    H = O.sinkhorn(L, iters)
    M = np.exp(L)
    for (i, j, k, l) in [(0, 0, 1, 1), (0, 2, 3, 4), (4, 1, 2, 3), (1, 0, 4, 2)]:
        ch = H[:, i, j] * H[:, k, l] / (H[:, i, l] * H[:, k, j])
        cm = M[:, i, j] * M[:, k, l] / (M[:, i, l] * M[:, k, j])
        np.testing.assert_allclose(ch, cm, rtol=1e-12)


def test_sinkhorn_converges_to_doubly_stochastic():
    """Column error shrinks with iterations and vanishes in the limit."""
    L = rng(6).standard_normal((30, 16, 16)) * 2
    devs = [np.abs(O.sinkhorn(L, it).sum(-2) - 1).max() for it in (1, 2, 5, 20, 200)]
    assert all(a >= b for a, b in zip(devs, devs[1:])), devs
    assert devs[-1] < 1e-12
    assert devs[0] > 1e-2


def test_sinkhorn_shift_invariance():
    L = rng(7).standard_normal((5, 4, 4))
    np.testing.assert_allclose(O.sinkhorn(L, 20), O.sinkhorn(L + 37.5, 20), rtol=1e-13)


def test_row_clamp_only_shrinks_rows_above_one():
    H = np.abs(rng(8).standard_normal((20, 4, 4)))
    Hc = O.row_clamp(H)
    rs = H.sum(-1)
    assert np.all(Hc.sum(-1) <= 1 + 1e-15)
    keep = rs <= 1
    np.testing.assert_array_equal(Hc[keep], H[keep])
    np.testing.assert_allclose(Hc[~keep].sum(-1), 1, atol=1e-15)


# ---------------------------------------------------------------- closure

@pytest.mark.parametrize("n", [4, 16])
def test_products_of_sinkhorn_maps_stay_doubly_stochastic(n):
    """Doubly stochastic matrices are closed under products, so the
    composite mixing over depth has forward gain (largest absolute row sum)
    exactly 1 and column sums within the per-layer tolerance (explainer,
    "mHC: keep the mixing doubly stochastic")."""
    Ls = rng(9, n).standard_normal((64, n, n)) * 2
    Hs = O.sinkhorn(Ls, 20)
    P = np.eye(n)
    for H in Hs:
        P = H @ P
    np.testing.assert_allclose(np.abs(P).sum(1).max(), 1.0, atol=1e-12)
    dev = np.abs(Hs.sum(-2) - 1).max()
    assert np.abs(P.sum(0) - 1).max() <= 64 * dev + 1e-12


def test_xhc_effective_16x16_maps_are_doubly_stochastic_and_close_under_products():
    """One xHC sublayer's full map is the k x k Sinkhorn block on the active
    streams and the identity elsewhere (explainer, "Which constraint
    survives"): row sums are 1 and columns within the Sinkhorn tolerance,
    also for products over an 8-layer chain."""
    N, k, m, C, T = 16, 4, 2, 8, 12
    r = rng(10)
    X = r.standard_normal((T, N, C))
    P = np.tile(np.eye(N), (T, 1, 1))
    for layer in range(8):
        W_full = r.standard_normal((N * C, 2 * N)) * 0.3
        W_act = r.standard_normal((k * C, k * k + k)) * 0.3
        pre = O.xhc_pre(X, W_full, W_act, m, k, 1, (1.0, 1.0, 1.0),
                        np.zeros(N), np.zeros(k * k), np.zeros(k))
        E = O.effective_mixing(pre["I"], pre["h_res"], N)
        np.testing.assert_allclose(E.sum(-1), 1, atol=1e-14)
        dev = np.abs(pre["h_res"].sum(-2) - 1).max()
        assert np.abs(E.sum(-2) - 1).max() <= dev + 1e-15
        P = E @ P
        out = r.standard_normal((1, T, C))
        X = O.xhc_post(X, out, pre["I"], pre["p"], pre["h_res"], pre["h_post"])
    np.testing.assert_allclose(np.abs(P).sum(-1).max(), 1.0, atol=1e-12)


# ---------------------------------------------------------------- special cases

def test_mhc_with_one_stream_and_unit_maps_is_the_plain_residual():
    """N = 1 with every map fixed at 1 is x + F(x) (explainer, "Hyper-
    connections: N streams, three small maps").  alpha = 0 and b_pre = 40
    make sigmoid exactly 1.0 in float64; 2 sigmoid(0) = 1; a 1x1 Sinkhorn is 1."""
    r = rng(11)
    T, C = 9, 32
    X = r.standard_normal((T, 1, C)).astype(np.float32).astype(np.float64)
    out = r.standard_normal((T, C)).astype(np.float32).astype(np.float64)
    W = r.standard_normal((C, 3))
    res = O.mhc_sublayer(X, out, W, (0.0, 0.0, 0.0), [40.0], [0.0], [0.0])
    np.testing.assert_array_equal(res["X"][:, 0], X[:, 0] + out)
    np.testing.assert_array_equal(res["inp"], X[:, 0])


def test_xhc_with_one_stream_is_the_plain_residual():
    r = rng(12)
    B, S, C = 2, 5, 32
    X = r.standard_normal((B * S, 1, C)).astype(np.float32).astype(np.float64)
    out = r.standard_normal((B, S, C)).astype(np.float32).astype(np.float64)
    res = O.xhc_sublayer(X, out, r.standard_normal((C, 2)), r.standard_normal((C, 2)), 1, 1, [],
                         (0.0, 0.0, 0.0), [40.0], [0.0], [0.0])
    np.testing.assert_array_equal(res["X"][:, 0], X[:, 0] + out.reshape(-1, C))
    np.testing.assert_array_equal(res["inp"], X[:, 0])
    assert np.all(res["I"] == 0) and np.all(res["p"] == 1)


def test_xhc_with_all_streams_active_equals_mhc():
    """With k = m = N, no router choice, K_r = 1 and the same residual and
    post columns, xHC's active maps come from the same normalised state as
    mHC's, so the two sublayers agree (xHC paper, Appendix C: mHC is the
    case k = N with no router, K_r = 1 and no convolution).  This ties the
    dense and the sparse code paths of the oracle together."""
    r = rng(13)
    N, C, B, S = 4, 16, 2, 4
    T = B * S
    X = r.standard_normal((T, N, C))
    out = r.standard_normal((B, S, C))
    Wm = r.standard_normal((N * C, 2 * N + N * N)) * 0.2
    bp, bo, br = r.standard_normal(N), r.standard_normal(N), r.standard_normal(N * N)
    alpha = (0.7, 1.3, 0.9)                         # pre, post, res for mHC
    m = O.mhc_sublayer(X, out, Wm, alpha, bp, bo, br)
    W_full = np.concatenate([r.standard_normal((N * C, N)), Wm[:, :N]], axis=1)
    W_act = np.concatenate([Wm[:, 2 * N:], Wm[:, N:2 * N]], axis=1)
    x = O.xhc_sublayer(X, out, W_full, W_act, N, N, [], (0.7, 0.9, 1.3), bp, br, bo)
    np.testing.assert_allclose(x["inp"], m["inp"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(x["X"], m["X"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(x["h_res"], m["h_res"], rtol=1e-13)


def test_mix_of_identical_streams_returns_that_stream():
    """The rows of H_res sum to one, so a new stream is a weighted average of
    the old ones and a state whose streams are all the same vector is mixed
    back into that vector; after a single Sinkhorn round the column sums
    are far from one, so applying the transposed map would not give it
    back (explainer, "mHC: keep the mixing doubly stochastic")."""
    r = rng(14)
    N, C, T = 5, 12, 6
    c = r.standard_normal((T, 1, C))
    X = np.repeat(c, N, axis=1)
    W = r.standard_normal((N * C, 2 * N + N * N))
    res = O.mhc_sublayer(X, np.zeros((T, C)), W, (1, 1, 4.0), np.zeros(N), np.zeros(N),
                         np.zeros(N * N), iters=1)
    assert np.abs(res["h_res"].sum(-2) - 1).max() > 0.1
    np.testing.assert_allclose(res["X"], X, rtol=1e-13, atol=1e-14)
    # xHC: the active rows mix among themselves
    k, m = 3, 1
    Wf = r.standard_normal((N * C, 2 * N))
    Wa = r.standard_normal((k * C, k * k + k)) * 3
    x = O.xhc_sublayer(X, np.zeros((1, T, C)), Wf, Wa, m, k, [], (1, 4.0, 1), np.zeros(N),
                       np.zeros(k * k), np.zeros(k), iters=1)
    assert np.abs(x["h_res"].sum(-2) - 1).max() > 0.1
    np.testing.assert_allclose(x["X"], X, rtol=1e-13, atol=1e-14)


def test_pre_and_post_maps_address_the_right_streams():
    """Saturated biases make H_pre and H_post one-hot (alpha = 0): the
    sublayer input is then stream 1 alone and only stream 2 receives out."""
    r = rng(15)
    N, C, T = 3, 10, 4
    X = r.standard_normal((T, N, C))
    out = r.standard_normal((T, C))
    W = r.standard_normal((N * C, 2 * N + N * N))
    b_res = np.array([[60, 0, 0], [0, 60, 0], [0, 0, 60]], float).ravel()  # ~identity mix
    res = O.mhc_sublayer(X, out, W, (0, 0, 0), [-40, 40, -40], [-40, -40, 40], b_res)
    np.testing.assert_allclose(res["inp"], X[:, 1], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(res["X"][:, 0], X[:, 0], atol=1e-15)
    np.testing.assert_allclose(res["X"][:, 1], X[:, 1], atol=1e-15)
    np.testing.assert_allclose(res["X"][:, 2], X[:, 2] + 2 * out, rtol=1e-15, atol=1e-15)


# ---------------------------------------------------------------- routing

@pytest.mark.parametrize("N,k,m", [(6, 3, 1), (16, 4, 2), (8, 4, 0), (5, 5, 2)])
def test_router_selection_matches_subset_enumeration(N, k, m):
    r = rng(16, N, k, m)
    C = 6
    for _ in range(20):
        Xt = r.standard_normal((N, C))
        W = r.standard_normal((N * C, 2 * N))
        I_bf, p_bf, _ = BF.xhc_route_token(Xt.tolist(), W.tolist(), m, k)
        z = O.xhc_router_logits(Xt[None], W[:, :N])
        I, p = O.xhc_select(z, m, k)
        assert I[0].tolist() == I_bf
        np.testing.assert_allclose(p[0], p_bf, rtol=1e-14)


def test_router_ties_go_to_the_lower_index_and_margin_sees_them():
    z = np.array([[0.0, 0.0, 3.0, 1.0, 3.0, 1.0]])
    I, p = O.xhc_select(z, 1, 3)
    assert I[0].tolist() == [0, 2, 4]
    assert O.xhc_topk_margin(z, 1, 3)[0] == 0.0
    z2 = np.array([[0.0, 0.0, 3.0, 1.0, 2.5, 1.2]])
    assert O.xhc_topk_margin(z2, 1, 3)[0] == pytest.approx(0.5)   # 3 vs 2.5 (order), 2.5 vs 1.2 (set)


# ---------------------------------------------------------------- temporal augmentation

def test_conv_impulse_response_is_the_kernel():
    """A unit impulse at t0 comes out as w[i] at t0 + i: kernel entry i
    multiplies lag i, and nothing leaks before t0 or across batch items."""
    C, S = 7, 20
    w = rng(17).standard_normal((8, C))
    out = np.zeros((2, S, C))
    out[0, 5] = 1.0
    g = O.causal_dwconv(out, w)
    np.testing.assert_array_equal(g[0, 5:13], w)
    assert np.all(g[0, :5] == 0) and np.all(g[0, 13:] == 0) and np.all(g[1] == 0)


def test_post_is_causal_and_stays_within_a_batch_item():
    """Changing the sublayer output at (b, t0) changes no state row at an
    earlier position of b and nothing in the other batch item (explainer,
    "What xHC changes": causal convolutions along the sequence)."""
    r = rng(18)
    N, k, m, C, B, S = 6, 3, 1, 8, 2, 16
    T = B * S
    X = r.standard_normal((T, N, C))
    out = r.standard_normal((B, S, C))
    convs = [r.standard_normal((kap, C)) / kap for kap in (4, 8, 12)]
    W_full = r.standard_normal((N * C, 2 * N))
    W_act = r.standard_normal((k * C, k * k + 4 * k))
    args = (W_full, W_act, m, k, convs, (0.3, 0.3, 0.3), np.zeros(N), np.zeros(k * k), np.zeros(4 * k))
    a = O.xhc_sublayer(X, out, *args)
    out2 = out.copy()
    out2[1, 7] += 1.0
    b = O.xhc_sublayer(X, out2, *args)
    diff = np.any(a["X"] != b["X"], axis=(1, 2)).reshape(B, S)
    assert not diff[0].any()
    assert not diff[1, :7].any()
    assert diff[1, 7:].any()


def test_gram_schmidt_orthogonality_bound():
    """With eps added to <v, v>, the step that removes v_j leaves
    <u, v_j> = <u, v_j>_before * eps / (|v_j|^2 + eps), and later steps only
    add O(eps) terms; so cos(v_i, v_j) <= 2 eps |g_i| / (|v_j|^2 |v_i|) with
    g_i the branch v_i came from, and MGS is orthogonal to rounding as
    eps -> 0."""
    r = rng(19)
    C = 256
    out = r.standard_normal((5, C))
    gs = [0.7 * out + r.standard_normal((5, C)) * s for s in (0.3, 1.0, 2.0)]
    comps = [out] + gs
    for eps in (1e-6, 0.0):
        vs = O.gram_schmidt(comps, eps)
        for i in range(4):
            for j in range(i):
                ni, nj = np.linalg.norm(vs[i], axis=-1), np.linalg.norm(vs[j], axis=-1)
                cos = np.abs((vs[i] * vs[j]).sum(-1)) / (ni * nj)
                lim = 2 * eps * np.linalg.norm(comps[i], axis=-1) / (nj ** 2 * ni) + 1e-13
                assert np.all(cos <= lim), (i, j, eps, cos, lim)


def test_gram_schmidt_spans_the_same_space_and_keeps_out_first():
    r = rng(20)
    C = 64
    comps = [r.standard_normal((3, C)) for _ in range(4)]
    vs = O.gram_schmidt(comps, 0.0)
    np.testing.assert_array_equal(vs[0], comps[0])
    for t in range(3):
        A = np.stack([c[t] for c in comps], 1)
        V = np.stack([v[t] for v in vs], 1)
        coef, *_ = np.linalg.lstsq(A, V, rcond=None)
        np.testing.assert_allclose(A @ coef, V, atol=1e-12)
        assert np.allclose(np.triu(coef), coef, atol=1e-12)   # v_j uses comps up to j only
        np.testing.assert_allclose(np.diag(coef), 1, atol=1e-12)


def test_zero_kernels_give_the_single_write():
    """Zero-initialised kernels make v_2..v_4 exactly 0 (eps guards 0/0), so
    the write is p_j H_post[j, 0] out, mHC's single write (explainer, "What
    xHC changes" and "What I could not check")."""
    r = rng(21)
    N, k, m, C, B, S = 6, 3, 1, 8, 1, 14
    X = r.standard_normal((B * S, N, C))
    out = r.standard_normal((B, S, C))
    V = O.xhc_write_basis(out, [np.zeros((kap, C)) for kap in (4, 8, 12)])
    assert np.all(V[:, :, 1:] == 0)
    np.testing.assert_array_equal(V[:, :, 0], out)


def test_write_is_homogeneous_in_the_sublayer_output():
    """Gram-Schmidt without normalisation is degree-1 homogeneous in out
    (exactly so at eps = 0), so the write term scales linearly with out; a
    normalised basis would not scale at all."""
    r = rng(22)
    N, k, m, C, B, S = 6, 3, 1, 64, 1, 14
    T = B * S
    X = r.standard_normal((T, N, C))
    out = r.standard_normal((B, S, C))
    convs = [r.standard_normal((kap, C)) / kap for kap in (4, 8, 12)]
    pre = O.xhc_pre(X, r.standard_normal((N * C, 2 * N)), r.standard_normal((k * C, k * k + 4 * k)),
                    m, k, 4, (0.1, 0.1, 0.1), np.zeros(N), np.zeros(k * k), np.zeros(4 * k))
    f = lambda o, eps=0.0: O.xhc_post(X, o, pre["I"], pre["p"], pre["h_res"], pre["h_post"], convs, eps=eps)
    base = f(np.zeros_like(out), 1e-6)          # the mix alone (eps keeps 0/0 away)
    assert np.all(np.isfinite(base))
    d1 = f(out) - base
    d3 = f(3.0 * out) - base
    assert np.all(np.isfinite(d1)) and np.abs(d1).max() > 0.1
    np.testing.assert_allclose(d3, 3.0 * d1, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- sparsity and conservation

def test_exactly_k_streams_change_and_the_rest_pass_through():
    """Per token only the k active rows are written; the N - k others are
    returned bit for bit (explainer, "What xHC changes")."""
    r = rng(23)
    N, k, m, C, B, S = 16, 4, 2, 32, 2, 12
    T = B * S
    X = r.standard_normal((T, N, C))
    out = r.standard_normal((B, S, C))
    convs = [r.standard_normal((kap, C)) / kap for kap in (4, 8, 12)]
    res = O.xhc_sublayer(X, out, r.standard_normal((N * C, 2 * N)) * 0.02,
                         r.standard_normal((k * C, k * k + 4 * k)) * 0.02, m, k, convs,
                         (0.01, 0.01, 0.01), np.zeros(N), np.zeros(k * k), np.zeros(4 * k))
    changed = np.any(res["X"] != X, axis=2)
    assert np.all(changed.sum(1) == k)
    for t in range(T):
        assert sorted(np.nonzero(changed[t])[0].tolist()) == sorted(res["I"][t].tolist())


def test_sum_over_streams_is_conserved_when_the_write_is_zero():
    """With out = 0, the stream sum changes only by the Sinkhorn column
    error; at the workloads' small logits that is at rounding level (the
    explainer's numpy check reports 3.6e-15)."""
    r = rng(24)
    N, k, m, C, B, S = 16, 4, 2, 64, 1, 32
    T = B * S
    X = r.standard_normal((T, N, C))
    res = O.xhc_sublayer(X, np.zeros((B, S, C)), r.standard_normal((N * C, 2 * N)) * 0.02,
                         r.standard_normal((k * C, k * k + 4 * k)) * 0.02, m, k,
                         [r.standard_normal((kap, C)) / kap for kap in (4, 8, 12)],
                         (0.01, 0.01, 0.01), np.zeros(N), np.zeros(k * k), np.zeros(4 * k))
    drift = np.abs(res["X"].sum(1) - X.sum(1)).max()
    assert drift < 1e-13
    # and with strongly non-uniform maps the drift is bounded by the column error
    res2 = O.xhc_sublayer(X, np.zeros((B, S, C)), r.standard_normal((N * C, 2 * N)),
                          r.standard_normal((k * C, k * k + k)) * 3, m, k, [],
                          (1.0, 3.0, 1.0), np.zeros(N), np.zeros(k * k), np.zeros(k), iters=3)
    dev = np.abs(res2["h_res"].sum(-2) - 1).max()
    drift2 = np.abs(res2["X"].sum(1) - X.sum(1)).max()
    assert drift2 <= dev * np.abs(X).sum(1).max() + 1e-12


# ---------------------------------------------------------------- brute force

def _tolist(a):
    return np.asarray(a).tolist()


@pytest.mark.parametrize("mlp", [False, True])
def test_xhc_sublayer_matches_scalar_brute_force(mlp):
    r = rng(25, mlp)
    N, k, m, C, B, S = 6, 3, 1, 8, 2, 16
    T = B * S
    X = r.standard_normal((T, N, C))
    out = r.standard_normal((B, S, C))
    convs = [r.standard_normal((kap, C)) / kap for kap in (4, 8, 12)] if mlp else []
    K_r = 1 + len(convs)
    Wf = r.standard_normal((N * C, 2 * N)) * 0.3
    Wa = r.standard_normal((k * C, k * k + k * K_r)) * 0.3
    alpha = (0.8, 1.1, 0.6)
    bp, br, bo = r.standard_normal(N) * 0.1, r.standard_normal(k * k) * 0.1, r.standard_normal(k * K_r) * 0.1
    o = O.xhc_sublayer(X, out, Wf, Wa, m, k, convs, alpha, bp, br, bo)
    b = BF.xhc_sublayer(_tolist(X), _tolist(out), _tolist(Wf), _tolist(Wa), m, k,
                        [_tolist(w) for w in convs], alpha, _tolist(bp), _tolist(br), _tolist(bo), 20)
    assert o["I"].tolist() == b["I"]
    for key in ("inp", "X", "p", "h_pre", "h_res", "h_post"):
        np.testing.assert_allclose(o[key], np.array(b[key]), rtol=1e-11, atol=1e-12, err_msg=key)


def test_mhc_sublayer_matches_scalar_brute_force():
    r = rng(26)
    N, C, T = 3, 8, 7
    X = r.standard_normal((T, N, C))
    out = r.standard_normal((T, C))
    W = r.standard_normal((N * C, 2 * N + N * N)) * 0.3
    alpha = (0.8, 1.1, 0.6)
    bp, bo, br = r.standard_normal(N), r.standard_normal(N), r.standard_normal(N * N)
    o = O.mhc_sublayer(X, out, W, alpha, bp, bo, br)
    for t in range(T):
        inp, new = BF.mhc_token(_tolist(X[t]), _tolist(out[t]), _tolist(W), alpha,
                                _tolist(bp), _tolist(bo), _tolist(br), 20)
        np.testing.assert_allclose(o["inp"][t], inp, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(o["X"][t], new, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- printed figures

def test_parameter_counts_reproduce_the_printed_figures():
    """The weight shapes used by the oracle and the library give the
    per-layer parameter counts printed in the xHC paper's Appendix C."""
    with open(os.path.join(GOLDEN, "param_counts.json")) as f:
        g = json.load(f)
    C = 1
    for case in g["cases"]:
        if case["method"] == "mHC":
            assert O.mhc_param_count(case["N"], C) == case["params_per_C"]
        else:
            assert O.xhc_param_count(case["N"], case["k"], C, case["conv_kernels"]) == case["params_per_C"]
    ratio = O.mhc_param_count(16, 1) / O.xhc_param_count(16, 4, 1)
    assert round(ratio, 1) == g["ratio_mhc16_over_xhc"]


# ---------------------------------------------------------------- decode

@pytest.mark.parametrize("use_mgs", [True, False])
def test_decode_token_by_token_equals_the_prefill(use_mgs):
    """Decoding a sequence one token at a time, with the conv history kept in
    the ring, writes the same state as the prefill post over the whole
    sequence (which convolves along the sequence directly), for sequences
    shorter and longer than the ring and two sequences decoded side by side."""
    r = rng(31, int(use_mgs))
    B, S, N, k, C = 2, 29, 6, 3, 16
    X = r.standard_normal((B * S, N, C))
    out = r.standard_normal((B, S, C))
    convs = [r.standard_normal((kap, C)) / kap for kap in (4, 8, 12)]
    I = np.stack([np.concatenate([[0], r.choice(np.arange(1, N), k - 1, replace=False)]) for _ in range(B * S)])
    p = np.concatenate([np.ones((B * S, 1)), r.uniform(0.1, 0.9, (B * S, k - 1))], axis=1)
    h_res = O.row_clamp(O.sinkhorn(r.standard_normal((B * S, k, k)), 20))
    h_post = r.uniform(0.1, 1.9, (B * S, k, 4))
    ref = O.xhc_post(X, out, I, p, h_res, h_post, convs, use_mgs)
    ring = r.standard_normal((B, O.RING, C))   # stale contents must not leak into a new sequence
    for s in range(S):
        rows = np.arange(B) * S + s
        Xn, ring = O.xhc_decode_post(X[rows], out[:, s], ring, np.full(B, s), I[rows], p[rows], h_res[rows],
                                     h_post[rows], convs, use_mgs)
        np.testing.assert_allclose(Xn, ref[rows], rtol=0, atol=1e-12 * np.abs(ref).max())
    for b in range(B):
        for s in range(S - O.RING, S):
            np.testing.assert_array_equal(ring[b, s % O.RING], out[b, s])
