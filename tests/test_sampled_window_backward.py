"""The sampled-token method of the full-size backward test, checked on the
CPU with the gradient oracle: for a token t, the oracle on the 23 tokens
t - 11 .. t + 11 of its sequence (clipped at its ends) gives the same state
gradient, map gradients and d_out at t as the oracle on the whole batch."""
import numpy as np
import pytest

from oracle import hc_grad as G
from oracle import hc_oracle as O


def _grads(X, out, d_inp, d_X, w, m, k, K_r):
    alpha = (0.7, 0.9, 0.8)
    pre = O.xhc_pre(X, w["W_full"], w["W_act"], m, k, K_r, alpha, w["b_pre"], w["b_res"], w["b_post"], iters=20)
    ga = G.xhc_apply_grads(X, out, pre["I"], pre["p"], pre["h_pre"], pre["h_res"], pre["h_post"], w["convs"], d_inp,
                           d_X)
    gg = G.xhc_gen_grads(X, w["W_full"], w["W_act"], m, k, K_r, alpha, w["b_pre"], w["b_res"], w["b_post"], pre["I"],
                         ga["h_pre"], ga["h_res"], ga["h_post"], ga["p"])
    return pre, ga, gg


@pytest.mark.parametrize("mlp", [True, False])
def test_window_oracle_equals_whole_sequence(mlp):
    r = np.random.default_rng([57, int(mlp)])
    B, S, N, k, m, C = 2, 40, 6, 3, 1, 8
    T = B * S
    K_r = 4 if mlp else 1
    w = dict(W_full=r.standard_normal((N * C, 2 * N)) * 0.4, W_act=r.standard_normal((k * C, k * k + k * K_r)) * 0.4,
             convs=[r.standard_normal((kap, C)) / kap for kap in (4, 8, 12)] if mlp else [],
             b_pre=r.standard_normal(N) * 0.1, b_res=r.standard_normal(k * k) * 0.1,
             b_post=r.standard_normal(k * K_r) * 0.1)
    X = r.standard_normal((T, N, C))
    out = r.standard_normal((B, S, C))
    d_inp, d_X = r.standard_normal((T, C)), r.standard_normal((T, N, C))
    pre, ga, gg = _grads(X, out, d_inp, d_X, w, m, k, K_r)
    for t in (0, 5, 11, 12, 20, 28, 39, 40, 52, 79):
        b, s = divmod(t, S)
        lo, hi = b * S + max(0, s - 11), b * S + min(S - 1, s + 11)
        sl = slice(lo, hi + 1)
        W = hi - lo + 1
        p2, a2, g2 = _grads(X[sl], out.reshape(T, C)[sl].reshape(1, W, C), d_inp[sl], d_X[sl], w, m, k, K_r)
        j = t - lo
        np.testing.assert_array_equal(p2["I"][j], pre["I"][t])
        np.testing.assert_allclose(a2["X"][j] + g2["X"][j], ga["X"][t] + gg["X"][t], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(a2["out"].reshape(W, C)[j], ga["out"].reshape(T, C)[t], rtol=1e-10, atol=1e-12)
        for key in ("h_pre", "h_res", "h_post", "p"):
            np.testing.assert_allclose(a2[key][j], ga[key][t], rtol=1e-10, atol=1e-12)
