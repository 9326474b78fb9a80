"""Pins of the float64 gradient oracle of one xHC sublayer
(``oracle/hc_grad.py``): its forward against the NumPy oracle, every gradient
against central finite differences of the NumPy oracle, and the one-stream
plain residual, whose gradients are known in closed form."""
import numpy as np
import pytest

from oracle import hc_grad as G
from oracle import hc_oracle as O


def rng(*k):
    return np.random.default_rng(list(k))


def case(r, B, S, N, k, m, C, mlp, wstd=0.4):
    T = B * S
    K_r = 4 if mlp else 1
    d = dict(
        X=r.standard_normal((T, N, C)), out=r.standard_normal((B, S, C)),
        W_full=r.standard_normal((N * C, 2 * N)) * wstd, W_act=r.standard_normal((k * C, k * k + k * K_r)) * wstd,
        convs=[r.standard_normal((kap, C)) / kap for kap in (4, 8, 12)] if mlp else [],
        alpha=np.array([0.7, 0.9, 0.8]), b_pre=r.standard_normal(N) * 0.1, b_res=r.standard_normal(k * k) * 0.1,
        b_post=r.standard_normal(k * K_r) * 0.1,
    )
    # redraw tokens whose routing is near a tie, so small perturbations keep the active set
    for _ in range(50):
        z = O.xhc_router_logits(d["X"], d["W_full"][:, :N])
        bad = np.nonzero(O.xhc_topk_margin(z, m, k) < 1e-2)[0]
        if bad.size == 0:
            break
        d["X"][bad] = r.standard_normal((bad.size, N, C))
    return d


def loss_np(d, m, k, d_inp, d_X, use_mgs=True):
    res = O.xhc_sublayer(d["X"], d["out"], d["W_full"], d["W_act"], m, k, d["convs"], tuple(d["alpha"]), d["b_pre"],
                         d["b_res"], d["b_post"], iters=20, use_mgs=use_mgs, dtype="f64")
    return float(np.sum(res["inp"] * d_inp) + np.sum(res["X"] * d_X)), res


def grads(d, m, k, d_inp, d_X, use_mgs=True):
    return G.xhc_sublayer_grads(d["X"], d["out"], d["W_full"], d["W_act"], m, k, d["convs"], tuple(d["alpha"]),
                                d["b_pre"], d["b_res"], d["b_post"], d_inp, d_X, iters=20, use_mgs=use_mgs)


@pytest.mark.parametrize("mlp", [True, False])
def test_gradient_oracle_forward_is_the_numpy_oracle(mlp):
    r = rng(51, int(mlp))
    B, S, N, k, m, C = 2, 9, 6, 3, 1, 8
    d = case(r, B, S, N, k, m, C, mlp)
    import torch
    t = {n: torch.as_tensor(v) for n, v in d.items() if n not in ("convs", "alpha")}
    inp, Xn, I, p = G.xhc_sublayer_forward(t["X"], t["out"], t["W_full"], t["W_act"], m, k,
                                           [torch.as_tensor(w) for w in d["convs"]],
                                           [torch.tensor(a) for a in d["alpha"]], t["b_pre"], t["b_res"], t["b_post"])
    ref = O.xhc_sublayer(d["X"], d["out"], d["W_full"], d["W_act"], m, k, d["convs"], tuple(d["alpha"]), d["b_pre"],
                         d["b_res"], d["b_post"], iters=20, dtype="f64")
    np.testing.assert_array_equal(I, ref["I"])
    np.testing.assert_allclose(p.detach().numpy(), ref["p"], rtol=1e-13)
    np.testing.assert_allclose(inp.detach().numpy(), ref["inp"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Xn.detach().numpy(), ref["X"], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("mlp,use_mgs", [(True, True), (True, False), (False, True)])
def test_gradients_match_central_differences_of_the_numpy_oracle(mlp, use_mgs):
    """Directional derivatives along random directions in every input agree
    with central differences of the NumPy oracle's loss <inp, d_inp> +
    <X', d_X> (step 1e-5; truncation and rounding stay below 1e-7
    relative)."""
    r = rng(52, int(mlp), int(use_mgs))
    B, S, N, k, m, C = 2, 14, 6, 3, 1, 8
    d = case(r, B, S, N, k, m, C, mlp)
    T = B * S
    d_inp = r.standard_normal((T, C))
    d_X = r.standard_normal((T, N, C))
    g = grads(d, m, k, d_inp, d_X, use_mgs)
    h = 1e-5
    names = ["X", "out", "W_full", "W_act", "b_pre", "b_res", "b_post", "alpha"] + (["convs"] if mlp else [])
    for name in names:
        if name == "convs":
            dirs = [r.standard_normal(w.shape) for w in d["convs"]]
            lin = sum(float(np.sum(gw * dw)) for gw, dw in zip(g["convs"], dirs))
            plus = dict(d, convs=[w + h * dw for w, dw in zip(d["convs"], dirs)])
            minus = dict(d, convs=[w - h * dw for w, dw in zip(d["convs"], dirs)])
        else:
            dv = r.standard_normal(np.shape(d[name]))
            lin = float(np.sum(g[name] * dv))
            plus, minus = dict(d), dict(d)
            plus[name] = d[name] + h * dv
            minus[name] = d[name] - h * dv
        lp, rp = loss_np(plus, m, k, d_inp, d_X, use_mgs)
        lm, rm = loss_np(minus, m, k, d_inp, d_X, use_mgs)
        assert np.array_equal(rp["I"], rm["I"]), f"{name}: the active set moved under the perturbation"
        fd = (lp - lm) / (2 * h)
        assert abs(fd - lin) <= 1e-7 * max(1.0, abs(fd)), (name, fd, lin)


def test_one_stream_gradients_are_the_plain_residual():
    """One stream, unit maps (alpha = 0, sigmoid(40) = 1, 2 sigmoid(0) = 1, a
    1 x 1 Sinkhorn map is 1), attention-type: inp = x and x' = x + out, so
    dx = d_inp + d_X and dout = d_X exactly."""
    r = rng(53)
    B, S, C = 2, 5, 8
    T = B * S
    d = dict(X=r.standard_normal((T, 1, C)), out=r.standard_normal((B, S, C)),
             W_full=r.standard_normal((C, 2)), W_act=r.standard_normal((C, 2)), convs=[],
             alpha=np.zeros(3), b_pre=np.full(1, 40.0), b_res=np.zeros(1), b_post=np.zeros(1))
    d_inp = r.standard_normal((T, C))
    d_X = r.standard_normal((T, 1, C))
    g = grads(d, 1, 1, d_inp, d_X)
    np.testing.assert_allclose(g["X"][:, 0], d_inp + d_X[:, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(g["out"].reshape(T, C), d_X[:, 0], rtol=0, atol=1e-15)


def _maps(d, m, k, K_r, iters=20):
    pre = O.xhc_pre(d["X"], d["W_full"], d["W_act"], m, k, K_r, tuple(d["alpha"]), d["b_pre"], d["b_res"],
                    d["b_post"], iters=iters)
    return pre


@pytest.mark.parametrize("mlp,use_mgs", [(True, True), (True, False), (False, True)])
def test_application_half_matches_central_differences(mlp, use_mgs):
    """Maps held fixed: the loss <sum_n h_pre[n] X_n, d_inp> + <xhc_post(...),
    d_X> of the NumPy oracle, differentiated numerically along random
    directions in the state, the output, the conv kernels and every map."""
    r = rng(54, int(mlp), int(use_mgs))
    B, S, N, k, m, C = 2, 13, 6, 3, 1, 8
    d = case(r, B, S, N, k, m, C, mlp)
    K_r = 4 if mlp else 1
    T = B * S
    pre = _maps(d, m, k, K_r)
    maps = dict(h_pre=pre["h_pre"], h_res=pre["h_res"], h_post=pre["h_post"], p=pre["p"])
    d_inp, d_X = r.standard_normal((T, C)), r.standard_normal((T, N, C))
    g = G.xhc_apply_grads(d["X"], d["out"], pre["I"], maps["p"], maps["h_pre"], maps["h_res"], maps["h_post"],
                          d["convs"], d_inp, d_X, use_mgs)

    def loss(v):
        inp = np.einsum("tn,tnc->tc", v["h_pre"], v["X"])
        Xn = O.xhc_post(v["X"], v["out"], pre["I"], v["p"], v["h_res"], v["h_post"], v["convs"], use_mgs)
        return float(np.sum(inp * d_inp) + np.sum(Xn * d_X))

    base = dict(maps, X=d["X"], out=d["out"], convs=d["convs"])
    h = 1e-5
    for name in ["X", "out", "h_pre", "h_res", "h_post", "p"] + (["convs"] if mlp else []):
        if name == "convs":
            dirs = [r.standard_normal(w.shape) for w in d["convs"]]
            lin = sum(float(np.sum(gw * dw)) for gw, dw in zip(g["convs"], dirs))
            plus = dict(base, convs=[w + h * dw for w, dw in zip(d["convs"], dirs)])
            minus = dict(base, convs=[w - h * dw for w, dw in zip(d["convs"], dirs)])
        else:
            dv = r.standard_normal(np.shape(base[name]))
            lin = float(np.sum(g[name] * dv))
            plus, minus = dict(base), dict(base)
            plus[name] = base[name] + h * dv
            minus[name] = base[name] - h * dv
        fd = (loss(plus) - loss(minus)) / (2 * h)
        assert abs(fd - lin) <= 1e-7 * max(1.0, abs(fd)), (name, fd, lin)


@pytest.mark.parametrize("mlp,iters", [(True, 20), (False, 20), (True, 0), (False, 2)])
def test_generation_half_matches_central_differences(mlp, iters):
    """Given map gradients, the loss sum(map * d_map) over the maps of the
    NumPy oracle's xhc_pre, differentiated numerically along random
    directions in the state, the weights, the biases and the scales.  With
    no Sinkhorn round the row clamp acts (the row holding the largest logit
    sums to more than one) and its divide is differentiated."""
    r = rng(55, int(mlp), iters)
    B, S, N, k, m, C = 2, 11, 6, 3, 1, 8
    d = case(r, B, S, N, k, m, C, mlp)
    K_r = 4 if mlp else 1
    T = B * S
    pre = _maps(d, m, k, K_r, iters)
    dm = dict(h_pre=r.standard_normal((T, N)), h_res=r.standard_normal((T, k, k)),
              h_post=r.standard_normal((T, k, K_r)), p=r.standard_normal((T, k)))
    g = G.xhc_gen_grads(d["X"], d["W_full"], d["W_act"], m, k, K_r, tuple(d["alpha"]), d["b_pre"], d["b_res"],
                        d["b_post"], pre["I"], dm["h_pre"], dm["h_res"], dm["h_post"], dm["p"], iters=iters)
    if iters == 0:   # the row clamp acts on some rows: that derivative is what this case pins
        Xa = np.take_along_axis(d["X"], pre["I"][:, :, None], axis=1).reshape(T, -1)
        la = O.rms_normalize(Xa) @ d["W_act"]
        L = d["alpha"][1] * la[:, : k * k].reshape(T, k, k) + np.asarray(d["b_res"]).reshape(k, k)
        assert (O.sinkhorn(L, 0).sum(-1) > 1.0 + 1e-3).any()

    def loss(v):
        q = _maps(v, m, k, K_r, iters)
        assert np.array_equal(q["I"], pre["I"]), "the active set moved under the perturbation"
        return sum(float(np.sum(q[n] * dm[n])) for n in dm)

    h = 1e-5
    for name in ["X", "W_full", "W_act", "b_pre", "b_res", "b_post", "alpha"]:
        dv = r.standard_normal(np.shape(d[name]))
        lin = float(np.sum(g[name] * dv))
        plus, minus = dict(d), dict(d)
        plus[name] = d[name] + h * dv
        minus[name] = d[name] - h * dv
        fd = (loss(plus) - loss(minus)) / (2 * h)
        assert abs(fd - lin) <= 1e-7 * max(1.0, abs(fd)), (name, fd, lin)


@pytest.mark.parametrize("mlp", [True, False])
def test_halves_add_up_to_the_whole_sublayer(mlp):
    """Application half, then the generation half fed with its map
    gradients: the state gradients add, and every other gradient is the whole
    sublayer's."""
    r = rng(56, int(mlp))
    B, S, N, k, m, C = 2, 9, 6, 3, 1, 8
    d = case(r, B, S, N, k, m, C, mlp)
    K_r = 4 if mlp else 1
    T = B * S
    d_inp, d_X = r.standard_normal((T, C)), r.standard_normal((T, N, C))
    whole = grads(d, m, k, d_inp, d_X)
    pre = _maps(d, m, k, K_r)
    ga = G.xhc_apply_grads(d["X"], d["out"], pre["I"], pre["p"], pre["h_pre"], pre["h_res"], pre["h_post"],
                           d["convs"], d_inp, d_X)
    gg = G.xhc_gen_grads(d["X"], d["W_full"], d["W_act"], m, k, K_r, tuple(d["alpha"]), d["b_pre"], d["b_res"],
                         d["b_post"], pre["I"], ga["h_pre"], ga["h_res"], ga["h_post"], ga["p"])
    np.testing.assert_allclose(ga["X"] + gg["X"], whole["X"], rtol=1e-10, atol=1e-12)
    # the active-row path touches only the active rows
    inactive = np.ones((T, N), dtype=bool)
    np.put_along_axis(inactive, pre["I"], False, axis=1)
    assert np.all(gg["X_act"][inactive] == 0.0)
    np.testing.assert_allclose(ga["out"], whole["out"], rtol=1e-10, atol=1e-12)
    for a, b in zip(ga["convs"], whole["convs"]):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)
    for name in ["W_full", "W_act", "b_pre", "b_res", "b_post", "alpha"]:
        np.testing.assert_allclose(gg[name], whole[name], rtol=1e-10, atol=1e-12)
