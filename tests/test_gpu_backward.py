"""GPU parity of the xHC sublayer backward (xhc_post_backward, then
xhc_pre_backward) against the float64 gradient oracle (oracle/hc_grad.py).

Each case runs xhc_pre on the GPU to leave the maps in the workspace, then
both backward calls, and compares element by element with the oracle's two
halves on the same inputs: the maps' gradients (application half), the state
gradient (sum of the halves), d_out and the conv-kernel gradients
(application half), and every weight, bias and scale gradient (generation
half, fed with the oracle's own map gradients).

Tolerance: bf16 cases store dX and d_out in bf16 (relative rounding 2^-9) and
read bf16 inputs, so they take the forward's bf16 bound, with no allowance:
the state gradient's parts (application half, then the generation half's
full-state and active-row passes) are summed in float and rounded once.  Float cases
accumulate in float over up to N*C products per token and T tokens per weight
gradient and run the Sinkhorn tangent through 20 normalisation rounds in
float, which the 1e-3 bound covers with margin (the errors printed are about
1e-5).
"""
import numpy as np
import pytest
import torch

import cases as K
from oracle import hc_grad as G
from oracle import hc_oracle as O
from stream_residual_mixing_amd import synth
from stream_residual_mixing_amd.binding import Config, weights_to_device

pytestmark = pytest.mark.gpu

GTOL = {"bf16": 2e-2, "f32": 1e-3}


def _print(*a):
    print(*a, flush=True)


def run_backward(lib, cfg, X, out, wd, d_inp, d_X, chained=False):
    """Forward maps by xhc_pre (or, chained, by xhc_route + xhc_pre_chained
    as the first sublayer of a chain), then both backward calls."""
    w = weights_to_device(wd)
    Xd, outd = X.cuda(), out.reshape(cfg.T, cfg.C).cuda()
    inp = torch.empty((cfg.T, cfg.C), dtype=cfg.torch_dtype, device="cuda")
    ws = lib.workspace(cfg)
    if chained:
        lib.xhc_route(cfg, w, Xd, ws)
        lib.xhc_pre_chained(cfg, w, None, None, Xd, inp, ws, None)
    else:
        lib.xhc_pre(cfg, w, Xd, inp, ws)
    maps = {k: v.clone() for k, v in lib.ws_arrays(cfg, ws).items()}
    bws = lib.backward_workspace(cfg)
    dX = torch.empty_like(Xd)
    d_out = torch.empty_like(outd)
    d_conv = torch.empty((24, cfg.C), dtype=torch.float32, device="cuda") if cfg.K_r == 4 else None
    d_inpd, d_Xd = d_inp.cuda(), d_X.cuda()
    lib.xhc_post_backward(cfg, w, Xd, outd, d_inpd, d_Xd, d_out, d_conv, ws, bws)
    dmaps = {k: v.clone() for k, v in lib.backward_ws_arrays(cfg, bws).items()}
    g = lib.grads(cfg)
    lib.xhc_pre_backward(cfg, w, Xd, d_inpd, d_Xd, dX, g, ws, bws)
    torch.cuda.synchronize()
    res = dict(X=dX.cpu(), out=d_out.cpu(), **{"d_" + k: v.cpu() for k, v in dmaps.items()},
               **{k: v.cpu() for k, v in g.items()}, I=maps["idx"].cpu().numpy())
    if d_conv is not None:
        res["convs"] = d_conv.cpu()
    return res


def oracle_backward(cfg, X, out, ow, d_inp, d_X):
    X64, out64 = K.f64(X), K.f64(out).reshape(cfg.B, cfg.S, cfg.C)
    alpha = (ow["alpha_pre"], ow["alpha_res"], ow["alpha_post"])
    pre = O.xhc_pre(X64, ow["w_full"], ow["w_act"], cfg.m, cfg.k, cfg.K_r, alpha, ow["b_pre"], ow["b_res"],
                    ow["b_post"], iters=cfg.iters)
    ga = G.xhc_apply_grads(X64, out64, pre["I"], pre["p"], pre["h_pre"], pre["h_res"], pre["h_post"], ow["conv"],
                           K.f64(d_inp), K.f64(d_X), bool(cfg.use_mgs))
    gg = G.xhc_gen_grads(X64, ow["w_full"], ow["w_act"], cfg.m, cfg.k, cfg.K_r, alpha, ow["b_pre"], ow["b_res"],
                         ow["b_post"], pre["I"], ga["h_pre"], ga["h_res"], ga["h_post"], ga["p"], iters=cfg.iters)
    return pre, ga, gg


def dx_err(cfg, dX, ga, gg):
    """The state gradient: the application half's part (through the dense
    read and the mix) plus the generation half's parts (through the
    full-state norms and projections, and through the active rows'), formed
    in float and rounded once to the state dtype; plain relative error."""
    return K.rel_err(K.f64(dX), ga["X"] + gg["X_full"] + gg["X_act"])


def compare(cfg, g, pre, ga, gg):
    errs = {
        "I": 0.0 if np.array_equal(g["I"], pre["I"]) else 1.0,
        "d_h_pre": K.rel_err(K.f64(g["d_h_pre"]), ga["h_pre"]),
        "d_h_res": K.rel_err(K.f64(g["d_h_res"]), ga["h_res"]),
        "d_h_post": K.rel_err(K.f64(g["d_h_post"]), ga["h_post"]),
        "d_p": K.rel_err(K.f64(g["d_p"]), ga["p"]),
        "dX": dx_err(cfg, g["X"], ga, gg),
        "d_out": K.rel_err(K.f64(g["out"]), ga["out"].reshape(cfg.T, cfg.C)),
        "dW_full": K.rel_err(K.f64(g["W_full"]), gg["W_full"], per_token=False),
        "dW_act": K.rel_err(K.f64(g["W_act"]), gg["W_act"], per_token=False),
        "d_b_pre": K.rel_err(K.f64(g["b_pre"]), gg["b_pre"], per_token=False),
        "d_b_res": K.rel_err(K.f64(g["b_res"]), gg["b_res"], per_token=False),
        "d_b_post": K.rel_err(K.f64(g["b_post"]), gg["b_post"], per_token=False),
        "d_alpha": K.rel_err(K.f64(g["alpha"]), gg["alpha"], per_token=False),
    }
    if "convs" in g:
        errs["d_conv"] = K.rel_err(K.f64(g["convs"]), np.concatenate(ga["convs"], axis=0), per_token=False)
    return errs


CASES = [
    # N, k, m, C, B, S, n_convs, use_mgs, dtype
    (16, 4, 2, 256, 2, 24, 3, 1, "bf16"),
    (16, 4, 2, 256, 2, 24, 3, 1, "f32"),
    (16, 4, 2, 128, 1, 30, 3, 0, "f32"),
    (16, 4, 2, 256, 2, 19, 0, 1, "bf16"),
    (16, 4, 2, 96, 2, 17, 0, 1, "f32"),
    (16, 2, 1, 128, 2, 16, 3, 1, "f32"),
    (8, 4, 1, 160, 1, 33, 3, 1, "f32"),
    (4, 4, 4, 64, 2, 14, 3, 1, "f32"),
    (1, 1, 1, 64, 2, 13, 3, 1, "f32"),
    (16, 4, 0, 128, 5, 5, 3, 1, "f32"),     # no fixed streams; sequences shorter than the longest kernel
    (16, 4, 2, 256, 2, 21, 3, 0, "bf16"),    # Gram-Schmidt off, bf16
    (8, 4, 2, 512, 2, 18, 0, 1, "bf16"),
    (16, 2, 1, 256, 3, 9, 3, 1, "bf16"),
    (4, 4, 4, 128, 2, 15, 3, 1, "bf16"),
    (1, 1, 1, 64, 2, 13, 0, 1, "bf16"),
    (16, 2, 1, 96, 2, 11, 0, 1, "bf16"),
    (16, 4, 2, 64, 1, 1, 3, 1, "bf16"),     # one token
    # wide channels: several channel groups per thread, up to the largest C built
    (16, 4, 2, 8192, 1, 40, 3, 1, "bf16"),
    (16, 4, 2, 32768, 1, 14, 3, 1, "bf16"),
    # the benchmark's channel width, 2 x 160 tokens
    (16, 4, 2, 4096, 2, 160, 3, 1, "bf16"),
    (16, 4, 2, 4096, 2, 160, 0, 1, "bf16"),
]


@pytest.mark.parametrize("N,k,m,C,B,S,nconv,mgs,dt", CASES)
def test_backward_matches_gradient_oracle(lib, N, k, m, C, B, S, nconv, mgs, dt):
    cfg = Config(N=N, k=k, m=m, C=C, B=B, S=S, n_convs=nconv, use_mgs=mgs, dtype=dt)
    _print("backward", dict(N=N, k=k, m=m, C=C, B=B, S=S, n_convs=nconv, use_mgs=mgs, dtype=dt))
    X, out, wd, ow = K.xhc_inputs(cfg, seed=61)
    r = np.random.default_rng([61, 5])
    d_inp = synth._round(r.standard_normal((cfg.T, C)), dt)
    d_X = synth._round(r.standard_normal((cfg.T, N, C)), dt)
    g = run_backward(lib, cfg, X, out, wd, d_inp, d_X)
    pre, ga, gg = oracle_backward(cfg, X, out, ow, d_inp, d_X)
    errs = compare(cfg, g, pre, ga, gg)
    _print("  errors", {key: f"{v:.2e}" for key, v in errs.items()})
    assert errs.pop("I") == 0.0, "active indices differ"
    bad = {key: v for key, v in errs.items() if not v <= GTOL[dt]}
    assert not bad, bad


@pytest.mark.parametrize("nconv,dt", [(3, "bf16"), (0, "f32")])
def test_backward_after_chained_forward(lib, nconv, dt):
    """The chained forward calls keep the same per-token sums as xhc_pre in
    the workspace of the sublayer whose routing they finish, so the backward
    runs on a chained workspace too."""
    cfg = Config(N=16, k=4, m=2, C=256, B=2, S=20, n_convs=nconv, dtype=dt)
    X, out, wd, ow = K.xhc_inputs(cfg, seed=65)
    r = np.random.default_rng([65, 5])
    d_inp = synth._round(r.standard_normal((cfg.T, cfg.C)), dt)
    d_X = synth._round(r.standard_normal((cfg.T, cfg.N, cfg.C)), dt)
    g = run_backward(lib, cfg, X, out, wd, d_inp, d_X, chained=True)
    pre, ga, gg = oracle_backward(cfg, X, out, ow, d_inp, d_X)
    errs = compare(cfg, g, pre, ga, gg)
    _print("  chained forward, backward errors", {key: f"{v:.2e}" for key, v in errs.items()})
    assert errs.pop("I") == 0.0, "active indices differ"
    bad = {key: v for key, v in errs.items() if not v <= GTOL[dt]}
    assert not bad, bad


@pytest.mark.parametrize("iters", [0, 1, 3])
def test_backward_few_sinkhorn_rounds(lib, iters):
    """With no Sinkhorn round the map is exp(L - max L), whose row holding the
    largest logit has an entry 1 and positive others: it sums to more than one
    and the row clamp acts (its divide is differentiated).  With one or three
    rounds the map is far from doubly stochastic."""
    cfg = Config(N=16, k=4, m=2, C=128, B=2, S=14, n_convs=3, iters=iters, dtype="f32")
    X, out, wd, ow = K.xhc_inputs(cfg, seed=66 + iters)
    r = np.random.default_rng([66, iters])
    d_inp = synth._round(r.standard_normal((cfg.T, cfg.C)), "f32")
    d_X = synth._round(r.standard_normal((cfg.T, cfg.N, cfg.C)), "f32")
    g = run_backward(lib, cfg, X, out, wd, d_inp, d_X)
    pre, ga, gg = oracle_backward(cfg, X, out, ow, d_inp, d_X)
    errs = compare(cfg, g, pre, ga, gg)
    _print("  sinkhorn rounds", iters, {key: f"{v:.2e}" for key, v in errs.items()})
    assert errs.pop("I") == 0.0, "active indices differ"
    bad = {key: v for key, v in errs.items() if not v <= GTOL["f32"]}
    assert not bad, bad


def test_backward_in_place_gradient(lib):
    """dX may be the d_X buffer itself: same result as a separate buffer."""
    cfg = Config(N=16, k=4, m=2, C=128, B=1, S=20, n_convs=3, dtype="bf16")
    X, out, wd, ow = K.xhc_inputs(cfg, seed=62)
    r = np.random.default_rng([62, 5])
    d_inp = synth._round(r.standard_normal((cfg.T, cfg.C)), "bf16").cuda()
    d_X = synth._round(r.standard_normal((cfg.T, cfg.N, cfg.C)), "bf16").cuda()
    w = weights_to_device(wd)
    Xd, outd = X.cuda(), out.reshape(cfg.T, cfg.C).cuda()
    inp = torch.empty((cfg.T, cfg.C), dtype=torch.bfloat16, device="cuda")
    ws = lib.workspace(cfg)
    lib.xhc_pre(cfg, w, Xd, inp, ws)
    bws = lib.backward_workspace(cfg)
    d_conv = torch.empty((24, cfg.C), dtype=torch.float32, device="cuda")
    res = []
    for in_place in (False, True):
        dX = d_X.clone() if in_place else torch.empty_like(d_X)
        src = dX if in_place else d_X
        d_out = torch.empty_like(outd)
        lib.xhc_post_backward(cfg, w, Xd, outd, d_inp, src, d_out, d_conv, ws, bws)
        g = lib.grads(cfg)
        lib.xhc_pre_backward(cfg, w, Xd, d_inp, src, dX, g, ws, bws)
        torch.cuda.synchronize()
        res.append((dX.cpu(), d_out.cpu(), d_conv.cpu(), {k: v.cpu() for k, v in g.items()}))
    for a, b in zip(res[0][:3], res[1][:3]):
        assert torch.equal(a, b)
    for name in res[0][3]:
        assert torch.equal(res[0][3][name], res[1][3][name]), name


def test_backward_empty_batch_is_a_no_op(lib):
    cfg = Config(N=16, k=4, m=2, C=64, B=0, S=8, n_convs=3, dtype="bf16")
    assert lib.backward_workspace_bytes(cfg) == 0
    w = weights_to_device(synth.xhc_layer_weights(63, 0, 16, 4, 64, 4, "bf16"))
    e = torch.empty((0, 16, 64), dtype=torch.bfloat16, device="cuda")
    e2 = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    ws, bws = lib.workspace(cfg), lib.backward_workspace(cfg)
    d_conv = torch.full((24, 64), 7.0, device="cuda")
    lib.xhc_post_backward(cfg, w, e, e2, e2, e, e2.clone(), d_conv, ws, bws)
    g = lib.grads(cfg)
    lib.xhc_pre_backward(cfg, w, e, e2, e, e.clone(), g, ws, bws)
    torch.cuda.synchronize()
    assert torch.all(d_conv == 7.0), "nothing is written for an empty batch"


# ---------------------------------------------------------------- full size

FULL = dict(N=16, k=4, m=2, C=4096, B=2, S=8192)
FULL_SEED, GRAD_SEED = 64, 564


def _mini_case(cfg, seed, layer, t, attempts):
    """Oracle inputs for sampled token t at full size: the tokens lo..hi of
    its sequence with lo = t - 11 and hi = t + 11 (clipped to the sequence).
    dX[t] and the map gradients at t depend on token t and its output window;
    d_out[t] on the basis gradients of t..t+11, whose bases reach back to
    t - 11.  Rows come from the per-token generator keys."""
    S, N, C = cfg.S, cfg.N, cfg.C
    b, s = divmod(int(t), S)
    lo, hi = b * S + max(0, s - 11), b * S + min(S - 1, s + 11)
    rows = range(lo, hi + 1)
    X = synth.state_rows(seed, rows, N, C, "bf16", attempts)
    out = synth.out_rows(seed, layer, rows, C, "bf16")
    d_X = synth.state_rows(GRAD_SEED, rows, N, C, "bf16")
    d_inp = synth.out_rows(GRAD_SEED, 0, rows, C, "bf16")
    return lo, hi, X, out, d_X, d_inp


def _oracle_token_grads(cfg, ow, t, lo, hi, X, out, d_X, d_inp):
    W = hi - lo + 1
    sub = Config(N=cfg.N, k=cfg.k, m=cfg.m, C=cfg.C, B=1, S=W, n_convs=cfg.n_convs, dtype="bf16")
    pre, ga, gg = oracle_backward(sub, X, out, ow, d_inp, d_X)
    j = t - lo
    return dict(I=pre["I"][j], X=ga["X"][j] + gg["X"][j], X_apply=ga["X"][j], X_full=gg["X_full"][j],
                d_out=ga["out"].reshape(W, cfg.C)[j], h_pre=ga["h_pre"][j], h_res=ga["h_res"][j],
                h_post=ga["h_post"][j], p=ga["p"][j])


@pytest.mark.slow
@pytest.mark.timeout(600)
@pytest.mark.parametrize("nconv,layer", [(3, 0), (0, 1)])
def test_backward_full_size_sampled_tokens(lib, nconv, layer):
    """The benchmark's shape and launch sequence (2 x 8192 tokens, C = 4096,
    xhc_pre then both backward calls); sampled tokens compared with the
    oracle one by one (every token whose maps they depend on has a routing
    margin of at least 1e-4, redrawn otherwise); every token's state
    gradient, d_out and every weight gradient checked finite."""
    cfg = Config(n_convs=nconv, dtype="bf16", **FULL)
    N, k, C, B, S = cfg.N, cfg.k, cfg.C, cfg.B, cfg.S
    wd = synth.xhc_layer_weights(FULL_SEED, layer, N, k, C, cfg.K_r, "bf16")
    ow = K.oracle_weights(wd)
    toks = K.sample_tokens(B, S, 4, FULL_SEED)
    attempts, ref = {}, {}
    for j, t in enumerate(toks):
        t = int(t)
        if j % 8 == 0:
            _print(f"oracle: token {j} of {len(toks)}")
        for _ in range(20):
            lo, hi, X, out, d_X, d_inp = _mini_case(cfg, FULL_SEED, layer, t, attempts)
            z = O.xhc_router_logits(K.f64(X), ow["w_full"][:, :N])
            mg = O.xhc_topk_margin(z, cfg.m, k)
            bad = [lo + i for i in range(t - lo, hi - lo + 1) if mg[i] < K.MARGIN]
            if not bad:
                break
            for r_ in bad:
                attempts[r_] = attempts.get(r_, 0) + 1
        assert not bad, f"token {t}: no draws with routing margin >= {K.MARGIN}"
    # a later window may have redrawn rows of an earlier one: the cases are built after all redraws
    for t in toks:
        lo, hi, X, out, d_X, d_inp = _mini_case(cfg, FULL_SEED, layer, int(t), attempts)
        ref[int(t)] = _oracle_token_grads(cfg, ow, int(t), lo, hi, X, out, d_X, d_inp)
    _print(f"oracle ready: {len(toks)} sampled tokens, {sum(attempts.values())} redraws")

    T = cfg.T
    Xd = synth.state(FULL_SEED, T, N, C, "bf16", attempts).to("cuda")
    outd = synth.sublayer_out(FULL_SEED, layer, B, S, C, "bf16").reshape(T, C).to("cuda")
    d_Xd = synth.state(GRAD_SEED, T, N, C, "bf16").to("cuda")
    d_inpd = synth.sublayer_out(GRAD_SEED, 0, B, S, C, "bf16").reshape(T, C).to("cuda")
    _print(f"inputs on the GPU: T={T} N={N} C={C} n_convs={nconv}")
    w = weights_to_device(wd)
    inp = torch.empty((T, C), dtype=torch.bfloat16, device="cuda")
    ws = lib.workspace(cfg)
    lib.xhc_pre(cfg, w, Xd, inp, ws)
    bws = lib.backward_workspace(cfg)
    dX = torch.empty_like(Xd)
    d_out = torch.empty_like(outd)
    d_conv = torch.empty((24, C), dtype=torch.float32, device="cuda") if nconv else None
    lib.xhc_post_backward(cfg, w, Xd, outd, d_inpd, d_Xd, d_out, d_conv, ws, bws)
    dmaps = {key: v.clone() for key, v in lib.backward_ws_arrays(cfg, bws).items()}
    g = lib.grads(cfg)
    lib.xhc_pre_backward(cfg, w, Xd, d_inpd, d_Xd, dX, g, ws, bws)
    torch.cuda.synchronize()
    for name, v in [("dX", dX), ("d_out", d_out)] + list(g.items()) + ([("d_conv", d_conv)] if nconv else []):
        assert bool(torch.isfinite(v).all()), f"{name} has non-finite entries"
    tk = torch.from_numpy(toks).to("cuda")
    idx = lib.ws_arrays(cfg, ws)["idx"].index_select(0, tk).cpu().numpy()
    got = dict(X=dX.index_select(0, tk).cpu(), d_out=d_out.index_select(0, tk).cpu(),
               **{key: v.index_select(0, tk).cpu() for key, v in dmaps.items()})
    o = {key: np.stack([ref[int(t)][key] for t in toks]) for key in ref[int(toks[0])]}
    assert np.array_equal(idx, o["I"]), "active indices differ"
    errs = {
        "dX": K.rel_err(K.f64(got["X"]), o["X"]),
        "d_out": K.rel_err(K.f64(got["d_out"]), o["d_out"]),
        **{"d_" + key: K.rel_err(K.f64(got[key]), o[key]) for key in ("h_pre", "h_res", "h_post", "p")},
    }
    _print("  errors", {key: f"{v:.2e}" for key, v in errs.items()})
    bad = {key: v for key, v in errs.items() if not v <= GTOL["bf16"]}
    assert not bad, bad
