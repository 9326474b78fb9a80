"""Gradients of one xHC sublayer in float64: the reference for a backward pass.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the product path
never imports it.

The forward is the one of ``hc_oracle.xhc_sublayer`` (same readings, same
order of operations), written with PyTorch CPU tensors so that reverse-mode
differentiation, a library primitive, gives every gradient.  The active set is
a selection: it is computed without gradient, and the router receives
gradient only through the router weights p of the selected routed streams
(xHC paper "xHC: Expanded Hyper-Connections", paragraph "Mapping generation":
the backward propagates routing gradients only through the selected logits).
The Sinkhorn iterations are differentiated through, which is what a backward
that recomputes them computes (same paragraph).

The backward splits in two halves, the application (``xhc_apply_grads``:
the maps held fixed) and the generation (``xhc_gen_grads``: given the maps'
gradients), whose sum is the whole sublayer's gradient.

Pinned in ``tests/test_oracle_grad_pins.py``: the forward against the NumPy
oracle, every gradient of the whole sublayer and of each half against central
finite differences of the NumPy oracle, and the sum of the halves against the
whole.
"""
from __future__ import annotations

import numpy as np
import torch

EPS_NORM = 1e-6
EPS_MGS = 1e-6


def _t(a, grad=False):
    t = torch.as_tensor(np.asarray(a, dtype=np.float64)).clone()
    t.requires_grad_(grad)
    return t


def _rms(v):
    return v / torch.sqrt((v * v).mean(-1, keepdim=True) + EPS_NORM)


def _ln(v):
    mu = v.mean(-1, keepdim=True)
    sd = torch.sqrt(((v - mu) ** 2).mean(-1, keepdim=True))
    return (v - mu) / (sd + EPS_NORM)


def _sinkhorn(L, iters):
    M = torch.exp(L - L.amax(dim=(-2, -1), keepdim=True))
    for _ in range(iters):
        M = M / M.sum(-2, keepdim=True)
        M = M / M.sum(-1, keepdim=True)
    return M


def _conv(out, w):
    """Causal depthwise convolution along the sequence: out [B, S, C], w [kappa, C]."""
    B, S, C = out.shape
    g = torch.zeros_like(out)
    for i in range(w.shape[0]):
        if i >= S:
            break
        g = g + torch.nn.functional.pad(w[i] * out[:, : S - i, :], (0, 0, i, 0))
    return g


def _mgs(comps):
    vs = [comps[0]]
    for g in comps[1:]:
        u = g
        for v in vs:
            u = u - (u * v).sum(-1, keepdim=True) / ((v * v).sum(-1, keepdim=True) + EPS_MGS) * v
        vs.append(u)
    return vs


def _select(z, m, k):
    """Active set: the fixed streams, then routed streams by descending z,
    ties to the lower index (the same rule as hc_oracle.xhc_select)."""
    T, N = z.shape
    zr = z.detach().numpy()
    I = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        cand = sorted(range(m, N), key=lambda i: (-zr[t, i], i))
        I[t] = list(range(m)) + cand[: k - m]
    return I


def xhc_generation(X, W_full, W_act, m, k, K_r, alpha, b_pre, b_res, b_post, iters=20, I=None, X_act_src=None):
    """Mapping generation (the steps of hc_oracle.xhc_pre without the dense
    read): torch tensors in, (I, p, h_pre, h_res, h_post) out.  The active
    set is a selection made without gradient; pass I to hold it fixed.
    X_act_src (same values as X) feeds the active-row maps instead of X, so
    that the two paths' state gradients can be told apart."""
    T, N, C = X.shape
    a_pre, a_res, a_post = alpha
    x = X.reshape(T, N * C)
    z = _ln(x) @ W_full[:, :N]
    if I is None:
        with torch.no_grad():
            I = _select(z, m, k)
    It = torch.as_tensor(I)
    s = torch.sigmoid(z)
    p = torch.cat([torch.ones(T, m, dtype=X.dtype), torch.gather(s, 1, It[:, m:])], dim=1)
    h_pre = torch.sigmoid(a_pre * (_rms(x) @ W_full[:, N:2 * N]) + b_pre)
    Xa = torch.gather(X if X_act_src is None else X_act_src, 1, It[:, :, None].expand(T, k, C))
    la = _rms(Xa.reshape(T, k * C)) @ W_act
    L = a_res * la[:, : k * k].reshape(T, k, k) + b_res.reshape(k, k)
    H = _sinkhorn(L, iters)
    H = H / torch.clamp(H.sum(-1, keepdim=True), min=1.0)
    h_post = 2.0 * torch.sigmoid(a_post * la[:, k * k:].reshape(T, k, K_r) + b_post.reshape(k, K_r))
    return I, p, h_pre, H, h_post


def xhc_application(X, out, I, p, h_pre, H, h_post, convs, use_mgs=True):
    """Dense read and mapping application with the maps given (the read of
    hc_oracle.xhc_pre, then hc_oracle.xhc_post): torch tensors in,
    (inp, new state) out."""
    T, N, C = X.shape
    k = I.shape[1]
    It = torch.as_tensor(I)
    inp = torch.einsum("tn,tnc->tc", h_pre, X)
    Xa = torch.gather(X, 1, It[:, :, None].expand(T, k, C))
    K_r = 1 + len(convs)
    comps = [out] + [_conv(out, w) for w in convs]
    if use_mgs and len(comps) > 1:
        comps = _mgs(comps)
    V = torch.stack(comps, dim=2).reshape(T, K_r, C)
    new_a = torch.einsum("tij,tjc->tic", H, Xa) + p[:, :, None] * torch.einsum("tjr,trc->tjc", h_post, V)
    Xn = X.scatter(1, It[:, :, None].expand(T, k, C), new_a)
    return inp, Xn


def xhc_sublayer_forward(X, out, W_full, W_act, m, k, convs, alpha, b_pre, b_res, b_post, iters=20, use_mgs=True):
    """Torch tensors in, (inp, new state, I, p) out; the steps of
    ``hc_oracle.xhc_pre`` then ``hc_oracle.xhc_post``."""
    I, p, h_pre, H, h_post = xhc_generation(X, W_full, W_act, m, k, 1 + len(convs), alpha, b_pre, b_res, b_post, iters)
    inp, Xn = xhc_application(X, out, I, p, h_pre, H, h_post, convs, use_mgs)
    return inp, Xn, I, p


def xhc_sublayer_grads(X, out, W_full, W_act, m, k, convs, alpha, b_pre, b_res, b_post, d_inp, d_X, iters=20,
                       use_mgs=True):
    """Gradients of <inp, d_inp> + <X', d_X> (the upstream gradients d_inp of
    the sublayer input and d_X of the new state) with respect to every input
    of the sublayer: the state, the sublayer output, the projection weights,
    the conv kernels, the biases and the scales.  NumPy float64 arrays in and
    out (a dict keyed by the argument names; conv kernels as a list)."""
    args = dict(X=_t(X, True), out=_t(out, True), W_full=_t(W_full, True), W_act=_t(W_act, True),
                b_pre=_t(b_pre, True), b_res=_t(b_res, True), b_post=_t(b_post, True))
    cw = [_t(w, True) for w in convs]
    al = [_t(a, True) for a in alpha]
    inp, Xn, I, p = xhc_sublayer_forward(args["X"], args["out"], args["W_full"], args["W_act"], m, k, cw, al,
                                         args["b_pre"], args["b_res"], args["b_post"], iters, use_mgs)
    loss = (inp * _t(d_inp)).sum() + (Xn * _t(d_X)).sum()
    loss.backward()
    g = {name: t.grad.numpy().copy() for name, t in args.items()}
    g["convs"] = [w.grad.numpy().copy() for w in cw]
    g["alpha"] = np.array([a.grad.item() for a in al])
    g["I"] = I
    return g


def xhc_apply_grads(X, out, I, p, h_pre, h_res, h_post, convs, d_inp, d_X, use_mgs=True):
    """The application half of the backward: gradients of <inp, d_inp> +
    <X', d_X> with the maps held fixed, with respect to the state (through the
    dense read and the mix only), the sublayer output, the conv kernels and
    the maps h_pre [T, N], h_res [T, k, k], h_post [T, k, K_r], p [T, k]."""
    args = dict(X=_t(X, True), out=_t(out, True), h_pre=_t(h_pre, True), h_res=_t(h_res, True),
                h_post=_t(h_post, True), p=_t(p, True))
    cw = [_t(w, True) for w in convs]
    inp, Xn = xhc_application(args["X"], args["out"], np.asarray(I), args["p"], args["h_pre"], args["h_res"],
                              args["h_post"], cw, use_mgs)
    loss = (inp * _t(d_inp)).sum() + (Xn * _t(d_X)).sum()
    loss.backward()
    g = {name: t.grad.numpy().copy() for name, t in args.items()}
    g["convs"] = [w.grad.numpy().copy() for w in cw]
    return g


def xhc_gen_grads(X, W_full, W_act, m, k, K_r, alpha, b_pre, b_res, b_post, I, d_h_pre, d_h_res, d_h_post, d_p,
                  iters=20):
    """The generation half of the backward: given the gradients of the maps
    (d_h_pre [T, N], d_h_res [T, k, k], d_h_post [T, k, K_r], d_p [T, k]),
    the gradients of sum(map * d_map) with respect to the state (through the
    norms and projections), the projection weights, the biases and the
    scales, with the active set I held fixed.  The state gradient is also
    returned split by path: "X_full" through the full-state router and
    pre-map, "X_act" through the active-row maps ("X" is their sum)."""
    args = dict(X=_t(X, True), W_full=_t(W_full, True), W_act=_t(W_act, True), b_pre=_t(b_pre, True),
                b_res=_t(b_res, True), b_post=_t(b_post, True))
    X_act = _t(X, True)
    al = [_t(a, True) for a in alpha]
    _, p, h_pre, H, h_post = xhc_generation(args["X"], args["W_full"], args["W_act"], m, k, K_r, al, args["b_pre"],
                                            args["b_res"], args["b_post"], iters, I=np.asarray(I), X_act_src=X_act)
    loss = (h_pre * _t(d_h_pre)).sum() + (H * _t(d_h_res)).sum() + (h_post * _t(d_h_post)).sum() + \
        (p * _t(d_p)).sum()
    loss.backward()
    g = {name: t.grad.numpy().copy() for name, t in args.items()}
    g["X_full"] = g["X"]
    g["X_act"] = X_act.grad.numpy().copy()
    g["X"] = g["X_full"] + g["X_act"]
    g["alpha"] = np.array([a.grad.item() for a in al])
    return g
