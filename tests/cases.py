"""Shared helpers of the parity tests: seeded cases, the oracle side, the
GPU side through the C ABI, and the error metric.

The oracle and the HIP library only meet here: both receive the same seeded
values; the oracle never sees a value produced by the GPU.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import hc_oracle as O
from stream_residual_mixing_amd import synth
from stream_residual_mixing_amd.binding import Config, weights_to_device

f64 = synth.as_f64

# Tolerances: bf16 state with fp32 accumulation, and fp32 mode.
TOL = {"bf16": 2e-2, "f32": 1e-4}
MARGIN = 1e-4   # top-k logit margin below which a token is redrawn
WINDOW = 12     # a token plus the longest conv kernel's 11 lags


def _floor_den(r, floor, per_token=True):
    """max(|r|, floor * RMS), the RMS taken over each token's values (the
    first axis indexes tokens), so that tokens of very different scales are
    each measured against their own scale; over the whole array when
    ``per_token`` is false (sums over tokens, such as weight gradients)."""
    if per_token and r.ndim >= 2:
        rms = np.sqrt(np.mean(r.reshape(r.shape[0], -1) ** 2, axis=1)).reshape((-1,) + (1,) * (r.ndim - 1))
    else:
        rms = np.sqrt(np.mean(r * r))
    den = np.maximum(np.abs(r), floor * rms)
    return np.where(den == 0, 1.0, den)


def rel_err(g, r, floor=1e-2, per_token=True):
    """max_e |g - r| / max(|r|, floor * RMS(r)): relative error with a floor
    so that elements near zero are measured against their token's scale."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    return float(np.max(np.abs(g.reshape(r.shape) - r) / _floor_den(r, floor, per_token)))


def term_err(g, r, S, allow=0.0, floor=1e-2):
    """max_e (|g - r| - allow) / max(S, floor * RMS of the token's r), where S
    is the sum of the magnitudes of the terms that make up r (oracle values:
    for a mix sum_i H_i x_i + write, sum_i |H_i x_i| + |write|).  Floating-
    point sums are accurate relative to the size of their terms; a mix that
    cancels to a small result cannot be more accurate than that, in any
    order of summation.  S >= |r|, so without cancellation this is rel_err."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    S = np.asarray(S, np.float64)
    den = np.maximum(S, _floor_den(r, floor) if r.ndim else 1.0)
    return float(np.max(np.maximum(np.abs(g.reshape(r.shape) - r) - allow, 0.0) / den))


def logit_err(g, r):
    """Router logits: max_e |g - r| / max(|r|, RMS of the token's logits).
    Each logit sums N*C products; it ranks streams and, through sigmoid,
    gates them, so it is measured on the scale of its token's logits (a
    logit near zero carries no relative accuracy of its own)."""
    return rel_err(g, r, floor=1.0)


# --------------------------------------------------------------------- oracle

def oracle_weights(wd):
    """float64 copies of a synth weight dict."""
    o = dict(w_full=f64(wd["w_full"]), b_pre=f64(wd["b_pre"]), b_res=f64(wd["b_res"]),
             b_post=f64(wd["b_post"]), alpha_pre=wd["alpha_pre"], alpha_res=wd["alpha_res"],
             alpha_post=wd["alpha_post"])
    if wd.get("w_act") is not None:
        o["w_act"] = f64(wd["w_act"])
    o["conv"] = [f64(c) for c in (wd.get("conv") or [])]
    return o


def oracle_xhc(cfg: Config, X64, out64, ow, dtype=None):
    """Oracle xHC sublayer.  X64 [T,N,C]; out64 [B,S,C].  Besides the
    oracle's results, the scales S_inp and S_X of term_err (from oracle
    values)."""
    r = O.xhc_sublayer(X64, out64, ow["w_full"], ow["w_act"], cfg.m, cfg.k, ow["conv"],
                       (ow["alpha_pre"], ow["alpha_res"], ow["alpha_post"]),
                       ow["b_pre"], ow["b_res"], ow["b_post"], iters=cfg.iters,
                       use_mgs=bool(cfg.use_mgs), dtype=dtype or cfg.dtype)
    X = np.asarray(X64, np.float64)
    T, N, C = X.shape
    V = O.xhc_write_basis(out64, ow["conv"], bool(cfg.use_mgs)).reshape(T, -1, C)     # [T, K_r, C]
    Xa = np.take_along_axis(X, r["I"][:, :, None], axis=1)                          # [T, k, C]
    sa = (np.einsum("tji,tic->tjc", np.abs(r["h_res"]), np.abs(Xa))
          + np.einsum("tjr,trc->tjc", np.abs(r["p"][:, :, None] * r["h_post"]), np.abs(V)))
    S_X = np.abs(X).copy()
    np.put_along_axis(S_X, r["I"][:, :, None], sa, axis=1)
    r["S_X"] = S_X
    r["S_inp"] = np.einsum("tn,tnc->tc", np.abs(r["h_pre"]), np.abs(X))
    return r


def oracle_mhc(cfg: Config, X64, out64, ow, dtype=None):
    r = O.mhc_sublayer(X64, out64.reshape(-1, cfg.C), ow["w_full"],
                       (ow["alpha_pre"], ow["alpha_post"], ow["alpha_res"]),
                       ow["b_pre"], ow["b_post"], ow["b_res"], iters=cfg.iters, dtype=dtype or cfg.dtype)
    X = np.asarray(X64, np.float64)
    out = np.asarray(out64, np.float64).reshape(-1, cfg.C)
    r["S_X"] = (np.einsum("tij,tjc->tic", np.abs(r["h_res"]), np.abs(X))
                + np.abs(r["h_post"])[:, :, None] * np.abs(out)[:, None, :])
    r["S_inp"] = np.einsum("tn,tnc->tc", np.abs(r["h_pre"]), np.abs(X))
    return r


def margins(cfg: Config, X64, ow):
    z = O.xhc_router_logits(X64, ow["w_full"][:, :cfg.N])
    return O.xhc_topk_margin(z, cfg.m, cfg.k)


def xhc_inputs(cfg: Config, seed, layer=0, resample=True, weights=None, affine=False, margin=MARGIN):
    """Seeded X, out and weights for an xHC case; tokens whose routing
    margin (oracle logits) is below ``margin`` are redrawn.  ``weights``
    replaces the workloads' own weight draw (a function of seed, layer, N, k,
    C, K_r and dtype, as synth.xhc_layer_weights); ``affine`` gives every
    state row its own scale and offset."""
    make = weights or synth.xhc_layer_weights
    wd = make(seed, layer, cfg.N, cfg.k, cfg.C, cfg.K_r, cfg.dtype)
    ow = oracle_weights(wd)
    attempts = {}
    X = synth.state(seed, cfg.T, cfg.N, cfg.C, cfg.dtype, affine=affine)
    if resample:
        for _ in range(20):
            bad = np.nonzero(margins(cfg, f64(X), ow) < margin)[0]
            if bad.size == 0:
                break
            for t in bad:
                attempts[int(t)] = attempts.get(int(t), 0) + 1
            X[bad] = synth.state_rows(seed, bad, cfg.N, cfg.C, cfg.dtype, attempts, affine)
    out = synth.sublayer_out(seed, layer, cfg.B, cfg.S, cfg.C, cfg.dtype)
    return X, out, wd, ow


def mhc_inputs(cfg: Config, seed, layer=0, weights=None, affine=False):
    make = weights or synth.mhc_layer_weights
    wd = make(seed, layer, cfg.N, cfg.C, cfg.dtype)
    X = synth.state(seed, cfg.T, cfg.N, cfg.C, cfg.dtype, affine=affine)
    out = synth.sublayer_out(seed, layer, cfg.B, cfg.S, cfg.C, cfg.dtype)
    return X, out, wd, oracle_weights(wd)


# ------------------------------------------------------- sampled full-size

def sample_tokens(B, S, n_random, seed):
    """Flat token ids: sequence starts, the first conv window, tile (16) and
    block edges, the middle and the end of every sequence, plus random ones."""
    rng = np.random.default_rng([seed, 99])
    fixed = [0, 1, 5, 11, 12, 15, 16, 63, 64, 1023, 1024, S // 2, S - 1]
    toks = set()
    for b in range(B):
        toks.update(b * S + s for s in fixed if s < S)
        toks.update(b * S + int(s) for s in rng.integers(0, S, n_random))
    return np.array(sorted(toks), dtype=np.int64)


def out_window(seed, layer, t, S, C, w):
    """float64 rows out[t-w+1 .. t] of token t's sequence, zero before its start."""
    b, s = divmod(int(t), S)
    lo = max(0, s - w + 1)
    win = np.zeros((w, C))
    win[w - (s - lo + 1):] = f64(synth.out_rows(seed, layer, range(b * S + lo, b * S + s + 1), C, "bf16"))
    return win


def oracle_token(cfg, x_t, win, ow):
    """Oracle sublayer for one token from its state row and output window;
    returns that token's results and its routing margin."""
    w = win.shape[0]
    Xw = np.zeros((w, cfg.N, cfg.C))
    Xw[-1] = x_t
    sub = Config(N=cfg.N, k=cfg.k, m=cfg.m, C=cfg.C, B=1, S=w, n_convs=cfg.n_convs, dtype=cfg.dtype)
    r = oracle_xhc(sub, Xw, win[None], ow)
    margin = float(O.xhc_topk_margin(r["z"][-1:], cfg.m, cfg.k)[0])
    return {key: v[-1] for key, v in r.items()}, margin


# ------------------------------------------------------------------ chains

CHAIN_MARGIN = 1e-2   # routing margin kept at every layer of a bf16 chain


def chain_configs(N, k, m, C, B, S, kinds, dtype="bf16"):
    return [Config(N=N, k=k, m=m, C=C, B=B, S=S, n_convs=3 if lk == "M" else 0, dtype=dtype) for lk in kinds]


def oracle_chain(cfgs, X64, outs64, ows):
    """The oracle's sublayers one after the other, each on the state the
    previous one left (rounded to the state dtype).  Returns per-layer results."""
    res = []
    X = X64
    for cfg, out, ow in zip(cfgs, outs64, ows):
        r = oracle_xhc(cfg, X, out, ow)
        res.append(r)
        X = r["X"]
    return res


def xhc_chain_inputs(cfgs, seed, margin, weights=None, affine=False):
    """Seeded state, per-layer outputs and weights of a chain; tokens whose
    routing margin is below `margin` at any layer of the oracle chain are
    redrawn (each state row has its own generator key).  ``weights`` and
    ``affine`` as in xhc_inputs."""
    c0 = cfgs[0]
    make = weights or synth.xhc_layer_weights
    wds = [make(seed, l, c.N, c.k, c.C, c.K_r, c.dtype) for l, c in enumerate(cfgs)]
    ows = [oracle_weights(wd) for wd in wds]
    outs = [synth.sublayer_out(seed, l, c.B, c.S, c.C, c.dtype) for l, c in enumerate(cfgs)]
    outs64 = [f64(o) for o in outs]
    attempts = {}
    X = synth.state(seed, c0.T, c0.N, c0.C, c0.dtype, affine=affine)
    for _ in range(30):
        ref = oracle_chain(cfgs, f64(X), outs64, ows)
        bad = set()
        for cfg, r in zip(cfgs, ref):
            bad.update(np.nonzero(O.xhc_topk_margin(r["z"], cfg.m, cfg.k) < margin)[0].tolist())
        if not bad:
            return X, outs, wds, ref
        bad = sorted(bad)
        for t in bad:
            attempts[t] = attempts.get(t, 0) + 1
        X[bad] = synth.state_rows(seed, bad, c0.N, c0.C, c0.dtype, attempts, affine)
    raise AssertionError("could not draw a chain with the required routing margins")


def gpu_xhc_chain(lib, cfgs, X, outs, wds, stream=None):
    """The chained calls through the C ABI (two workspaces in turn); per layer
    the public workspace arrays after xhc_pre_chained, inp, and the state
    after xhc_post_chained (CPU copies)."""
    ws_ = [weights_to_device(wd) for wd in wds]
    Xd = X.to("cuda")
    inp = torch.empty((cfgs[0].T, cfgs[0].C), dtype=cfgs[0].torch_dtype, device="cuda")
    nb = max(lib.workspace_bytes(c) for c in cfgs)
    wsp = [torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda") for _ in range(2)]
    lib.xhc_route(cfgs[0], ws_[0], Xd, wsp[0], stream)
    res = []
    for l, cfg in enumerate(cfgs):
        nxt = l + 1 < len(cfgs)
        cn, wn, wsn = (cfgs[l + 1], ws_[l + 1], wsp[(l + 1) % 2]) if nxt else (None, None, None)
        lib.xhc_pre_chained(cfg, ws_[l], cn, wn, Xd, inp, wsp[l % 2], wsn, stream)
        arrays = {k: v.clone() for k, v in lib.ws_arrays(cfg, wsp[l % 2]).items()}
        assert int(arrays.pop("status").item()) == 0
        lib.xhc_post_chained(cfg, ws_[l], cn, wn, Xd, outs[l].to("cuda"), wsp[l % 2], wsn, stream)
        torch.cuda.synchronize()
        res.append(dict(inp=inp.cpu(), X=Xd.cpu(), **{k: v.cpu() for k, v in arrays.items()}))
    return res


def ulp_round(x, dtype):
    """What two correct roundings of nearly the same value to the state dtype
    can differ by: one unit in the last place at |x|, taken in the binade
    above when |x| lies within a unit of it (zero where x is zero)."""
    x = np.abs(np.asarray(x, np.float64))
    u = ulp(x * (1.0 + (2.0 ** -7 if dtype == "bf16" else 2.0 ** -23)), dtype)
    return np.where(x == 0, 0.0, u)


def carried_allowances(hist, dtype, ows=None):
    """Allowances for a chain whose sides each carry their own rounded state.

    ``hist`` holds the oracle's results of layers 0..l in order (I [T,k],
    h_pre [T,N], inp [T,C], X [T,N,C] after the layer, z [T,N], h_post
    [T,k,K_r]); ``ows`` the oracle weights of each layer (for the router).
    Both sides start from the same state.  A layer copies the rows it does
    not write bit for bit, so their difference is what it was; it writes an
    active row as a mix of the active rows with non-negative weights summing
    to at most one plus the write, computes that in float32 and rounds it to
    the state dtype.  So the difference of row i after layer l is at most
    A_l[i]: A_{-1} = 0; A_l[i] = A_{l-1}[i] outside the active list;
    A_l[I_j] = sum_i H_res[j][i] A_{l-1}[I_i] + u inside it, where u
    is one rounding (two correct roundings differ by one unit, ulp_round) plus
    the float32 error of the k + K_r products of the mix and the write,
    (k + K_r + 2) 2^-24 times the largest magnitude they involve (the active
    rows before and after the layer at that channel).
    The sublayer input of layer l is allowed one unit of itself plus
    sum_i H_pre[i] A_{l-1}[i].  The router logits of layer l, z = LN(vec X) W_r,
    move to first order by at most (sum_j A_j |W_jn| + mean(A) |sum_j W_jn|)/sd
    + |z_n| RMS(A)/sd (the numerator, the mean and the standard deviation sd
    of the state entering the layer each shifted by the state's difference).
    Computed from oracle values only; any other arithmetic difference must
    stay within the relative bar.  Returns per layer a dict of allowances for
    inp, X and z."""
    out = []
    A = None
    Xprev = None
    for l, r in enumerate(hist):
        I = np.asarray(r["I"], np.int64)
        Xl = np.asarray(r["X"], np.float64)
        T, N, C = Xl.shape
        k = I.shape[1]
        K_r = np.asarray(r["h_post"]).reshape(T, k, -1).shape[2]
        if A is None:
            A = np.zeros(Xl.shape)
        a_inp = ulp_round(r["inp"], dtype) + np.einsum("tn,tnc->tc", np.asarray(r["h_pre"], np.float64), A)
        a_z = np.zeros((T, N))
        if ows is not None and Xprev is not None and np.any(A):
            Wr = np.asarray(ows[l]["w_full"], np.float64)[:, :N]
            xf = Xprev.reshape(T, N * C)
            sd = np.sqrt(np.mean((xf - xf.mean(axis=1, keepdims=True)) ** 2, axis=1))
            Af = A.reshape(T, N * C)
            num = Af @ np.abs(Wr) + Af.mean(axis=1)[:, None] * np.abs(Wr.sum(axis=0))[None, :]
            a_z = (num + np.abs(np.asarray(r["z"], np.float64)) * np.sqrt(np.mean(Af * Af, axis=1))[:, None]) / sd[:, None]
        Aact = np.take_along_axis(A, I[:, :, None], axis=1)                      # [T, k, C]
        prev = np.einsum("tji,tic->tjc", np.asarray(r["h_res"], np.float64), Aact)   # [T, k, C]
        before = Xprev if Xprev is not None else None
        rows = np.take_along_axis(Xl, I[:, :, None], axis=1)                     # [T, k, C]
        mag = np.abs(rows).max(axis=1)
        if before is not None:
            mag = np.maximum(mag, np.abs(np.take_along_axis(before, I[:, :, None], axis=1)).max(axis=1))
        arith = (k + K_r + 2) * 2.0 ** -24 * mag                                  # [T, C]
        A = A.copy()
        newA = prev + ulp_round(rows, dtype) + arith[:, None, :]
        np.put_along_axis(A, I[:, :, None], newA, axis=1)
        out.append(dict(inp=a_inp, X=A, z=a_z))
        Xprev = Xl
    return out


def compare_carried(g, o, l, dtype, allow):
    """Layer l >= 1 of a chain, where each side carries its own rounded state:
    exact indices, per-element maps, and per-element router logits (on their
    token's scale, logit_err), sublayer input and state (term_err) after the
    allowances of carried_allowances (oracle values only), all at the bar of
    the dtype."""
    assert np.array_equal(g["idx"].numpy(), o["I"]), f"layer {l}: active indices differ"
    errs = {key: rel_err(g[key].numpy().astype(np.float64), o[key]) for key in ("h_pre", "h_res", "h_post", "p")}
    if "z" in g:
        errs["z"] = err_with_allowance(g["z"].numpy().astype(np.float64), o["z"], allow["z"], floor=1.0)
    errs["inp"] = term_err(f64(g["inp"]), o["inp"], o["S_inp"], allow["inp"])
    errs["X"] = term_err(f64(g["X"]), o["X"], o["S_X"], allow["X"])
    bad = {key: v for key, v in errs.items() if not v <= TOL[dtype]}
    assert not bad, f"layer {l}: above {TOL[dtype]}: {bad} (all: {errs})"
    return errs


# ------------------------------------------------------------------------ GPU

def gpu_xhc(lib, cfg: Config, X, out, wd, stream=None):
    """Run xhc_pre + xhc_post through the C ABI; returns CPU copies."""
    w = weights_to_device(wd)
    Xd = X.to("cuda")
    outd = out.to("cuda")
    inp = torch.empty((cfg.T, cfg.C), dtype=cfg.torch_dtype, device="cuda")
    ws = lib.workspace(cfg)
    lib.xhc_pre(cfg, w, Xd, inp, ws, stream)
    arrays = {k: v.clone() for k, v in lib.ws_arrays(cfg, ws).items()}
    assert int(arrays.pop("status").item()) == 0, "a wait between workgroups gave up"
    lib.xhc_post(cfg, w, Xd, outd, ws, stream)
    torch.cuda.synchronize()
    return dict(inp=inp.cpu(), X=Xd.cpu(), **{k: v.cpu() for k, v in arrays.items()})


def gpu_mhc(lib, cfg: Config, X, out, wd, stream=None):
    w = weights_to_device(wd)
    Xd = X.to("cuda")
    outd = out.to("cuda")
    inp = torch.empty((cfg.T, cfg.C), dtype=cfg.torch_dtype, device="cuda")
    ws = lib.workspace(cfg, mhc=True)
    lib.mhc_pre(cfg, w, Xd, inp, ws, stream)
    arrays = {k: v.clone() for k, v in lib.ws_arrays(cfg, ws, mhc=True).items()}
    lib.mhc_post(cfg, w, Xd, outd, ws, stream)
    torch.cuda.synchronize()
    return dict(inp=inp.cpu(), X=Xd.cpu(), **{k: v.cpu() for k, v in arrays.items()})


def compare_xhc(g, o, tol, tokens=None):
    """Errors per quantity; indices must match exactly.  inp and X in the
    term_err measure, the maps in rel_err."""
    sel = slice(None) if tokens is None else tokens
    gi = g["idx"].numpy()[sel]
    assert np.array_equal(gi, o["I"][sel] if tokens is None else o["I"]), "active indices differ"
    errs = {}
    for key in ("inp", "X", "h_pre", "h_res", "h_post", "p"):
        gv = f64(g[key])[sel] if key in ("inp", "X") else g[key].numpy().astype(np.float64)[sel]
        errs[key] = term_err(gv, o[key], o["S_" + key]) if key in ("inp", "X") else rel_err(gv, o[key])
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"errors above {tol}: {bad} (all: {errs})"
    return errs


def compare_mhc(g, o, tol, tokens=None):
    sel = slice(None) if tokens is None else tokens
    errs = {}
    for key in ("inp", "X", "h_pre", "h_res", "h_post"):
        gv = f64(g[key])[sel] if key in ("inp", "X") else g[key].numpy().astype(np.float64)[sel]
        errs[key] = term_err(gv, o[key], o["S_" + key]) if key in ("inp", "X") else rel_err(gv, o[key])
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"errors above {tol}: {bad} (all: {errs})"
    return errs


# ---------------------------------------------------------------- xHC-Flash

def flash_oracle_weights(wd):
    o = {n: f64(wd[n]) for n in ("w_full", "w_post_attn", "w_act_mlp", "b_pre_attn", "b_pre_mlp", "b_post_attn",
                                 "b_res", "b_post_mlp")}
    o["conv"] = [f64(c) for c in (wd.get("conv") or [])]
    o["alpha"] = tuple(wd[n] for n in ("alpha_pre_attn", "alpha_pre_mlp", "alpha_post_attn", "alpha_res",
                                       "alpha_post_mlp"))
    return o


def flash_margins(cfg: Config, X64, ow):
    z = O.xhc_router_logits(X64, ow["w_full"][:, :cfg.N])
    return O.xhc_topk_margin(z, cfg.m, cfg.k)


def flash_inputs(cfg: Config, seed, block=0):
    """Seeded block-entry state, the two sublayer outputs and the block's
    weights; tokens whose routing margin is below MARGIN are redrawn."""
    wd = synth.xhcf_block_weights(seed, block, cfg.N, cfg.k, cfg.C, cfg.K_r, cfg.dtype)
    ow = flash_oracle_weights(wd)
    attempts = {}
    X = synth.state(seed, cfg.T, cfg.N, cfg.C, cfg.dtype)
    for _ in range(20):
        bad = np.nonzero(flash_margins(cfg, f64(X), ow) < MARGIN)[0]
        if bad.size == 0:
            break
        for t in bad:
            attempts[int(t)] = attempts.get(int(t), 0) + 1
        X[bad] = synth.state_rows(seed, bad, cfg.N, cfg.C, cfg.dtype, attempts)
    out_a = synth.sublayer_out(seed, 2 * block, cfg.B, cfg.S, cfg.C, cfg.dtype)
    out_m = synth.sublayer_out(seed, 2 * block + 1, cfg.B, cfg.S, cfg.C, cfg.dtype)
    return X, out_a, out_m, wd, ow, attempts


def oracle_flash(cfg: Config, X64, outa64, outm64, ow, dtype=None):
    return O.xhcf_block(X64, outa64, outm64, ow["w_full"], ow["w_post_attn"], ow["w_act_mlp"], cfg.m, cfg.k,
                        ow["conv"], ow["alpha"], ow["b_pre_attn"], ow["b_pre_mlp"], ow["b_post_attn"], ow["b_res"],
                        ow["b_post_mlp"], iters=cfg.iters, use_mgs=bool(cfg.use_mgs), dtype=dtype or cfg.dtype)


def gpu_flash(lib, cfg: Config, X, out_a, out_m, wd, stream=None):
    """xhcf_pre, xhcf_mid, xhcf_post through the C ABI; CPU copies of the
    inputs each call produces, the public workspace arrays, the state after
    the attention write (X1) and after the block (X)."""
    from stream_residual_mixing_amd.binding import flash_weights_to_device
    w = flash_weights_to_device(wd)
    Xd = X.to("cuda")
    inp_a = torch.empty((cfg.T, cfg.C), dtype=cfg.torch_dtype, device="cuda")
    inp_m = torch.empty_like(inp_a)
    ws = lib.flash_workspace(cfg)
    lib.xhcf_pre(cfg, w, Xd, inp_a, inp_m, ws, stream)
    pre = {k: v.clone() for k, v in lib.flash_ws_arrays(cfg, ws).items() if k not in ("h_res", "h_post_mlp")}
    base = inp_m.clone()
    lib.xhcf_mid(cfg, w, Xd, out_a.to("cuda"), inp_m, ws, stream)
    X1 = Xd.clone()
    arr = lib.flash_ws_arrays(cfg, ws)
    maps = dict(h_res=arr["h_res"].clone(), h_post=arr["h_post_mlp"].clone())
    lib.xhcf_post(cfg, w, Xd, out_m.to("cuda"), ws, stream)
    torch.cuda.synchronize()
    res = dict(inp_attn=inp_a.cpu(), inp_mlp_base=base.cpu(), inp_mlp=inp_m.cpu(), X1=X1.cpu(), X=Xd.cpu())
    res.update({k: v.cpu() for k, v in pre.items()})
    res.update({k: v.cpu() for k, v in maps.items()})
    return res


FLASH_KEYS = (("inp_attn", "inp_attn"), ("inp_mlp_base", "inp_mlp_base"), ("inp_mlp", "inp_mlp"), ("X1", "X1"),
              ("X", "X"), ("h_pre_attn", "h_pre_attn"), ("h_pre_mlp", "h_pre_mlp"), ("h_post_attn", "h_post_attn"),
              ("h_res", "h_res"), ("h_post", "h_post"), ("p", "p"))


def ulp(x, dtype):
    """One unit in the last place of the state dtype at |x| (from float64
    values): 2^(E - 7) for bfloat16 and 2^(E - 23) for float32, where
    2^E <= |x| < 2^(E + 1)."""
    _, e = np.frexp(np.asarray(x, np.float64))
    return np.ldexp(1.0, e - (8 if dtype == "bf16" else 24))


def corrected_input_err(g, r, base, dtype, floor=1e-2):
    """Relative error of the corrected MLP input, allowing one unit in the
    last place of the stored base readout.  Both sides store the base in the
    state dtype before the correction, and two correct roundings of it may
    differ by one unit; where a out_A nearly cancels the base, that unit is
    large against the result.  The allowance uses the oracle's base only."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    return float(np.max(np.maximum(np.abs(g - r) - ulp(base, dtype), 0.0) / _floor_den(r, floor))) if r.size else 0.0


def mixed_state_err(g, r, X1, I, dtype, floor=1e-2):
    """Relative error of the state after the MLP write, allowing one unit in
    the last place of the rows it mixes.  Each side mixes the active rows it
    stored after the attention write, and two correct roundings of a row may
    differ by one unit; a mix with non-negative rows summing to at most one
    moves that difference by at most one unit of the largest row mixed at
    that channel.  The allowance uses the oracle's rows only."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    big = np.take_along_axis(np.abs(np.asarray(X1, np.float64)), np.asarray(I)[:, :, None], axis=1).max(axis=1)
    allow = ulp(big, dtype)[:, None, :]
    return float(np.max(np.maximum(np.abs(g - r) - allow, 0.0) / _floor_den(r, floor)))


def compare_flash(g, o, tol, tokens=None, dtype="bf16"):
    """Errors per quantity of a block; active indices must match exactly."""
    sel = slice(None) if tokens is None else tokens
    assert np.array_equal(g["idx"].numpy()[sel], o["I"] if tokens is not None else o["I"]), "active indices differ"
    errs = {}
    for key, okey in FLASH_KEYS:
        gv = g[key]
        gv = (f64(gv) if gv.dtype != torch.float32 or key in ("inp_attn", "inp_mlp_base", "inp_mlp", "X1", "X")
              else gv.numpy().astype(np.float64))[sel]
        if key == "inp_mlp":
            errs[key] = corrected_input_err(gv, o[okey], o["inp_mlp_base"], dtype)
        elif key == "X":
            errs[key] = mixed_state_err(gv, o[okey], o["X1"], o["I"], dtype)
        else:
            errs[key] = rel_err(gv, o[okey])
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"errors above {tol}: {bad} (all: {errs})"
    return errs


# ----------------------------------------------------------- xHC-Flash-4sub

def flash4_oracle_weights(wd):
    return dict(w_full=f64(wd["w_full"]), w_post=[f64(t) for t in wd["w_post"]], w_act_last=f64(wd["w_act_last"]),
                conv=[[f64(c) for c in cs] for cs in wd["conv"]],
                alpha=dict(pre=tuple(wd["alpha_pre"]), post=tuple(wd["alpha_post"]), res=wd["alpha_res"]),
                b=dict(pre=[f64(t) for t in wd["b_pre"]], post=[f64(t) for t in wd["b_post"]], res=f64(wd["b_res"])))


def flash4_inputs(cfg: Config, seed, group=0):
    """Seeded group-entry state, the four sublayer outputs and the group's
    weights; tokens whose routing margin is below MARGIN are redrawn."""
    wd = synth.xhcf4_group_weights(seed, group, cfg.N, cfg.k, cfg.C, cfg.K_r, cfg.dtype)
    ow = flash4_oracle_weights(wd)
    attempts = {}
    X = synth.state(seed, cfg.T, cfg.N, cfg.C, cfg.dtype)
    for _ in range(20):
        z = O.xhc_router_logits(f64(X), ow["w_full"][:, :cfg.N])
        bad = np.nonzero(O.xhc_topk_margin(z, cfg.m, cfg.k) < MARGIN)[0]
        if bad.size == 0:
            break
        for t in bad:
            attempts[int(t)] = attempts.get(int(t), 0) + 1
        X[bad] = synth.state_rows(seed, bad, cfg.N, cfg.C, cfg.dtype, attempts)
    outs = [synth.sublayer_out(seed, 4 * group + q, cfg.B, cfg.S, cfg.C, cfg.dtype) for q in range(4)]
    return X, outs, wd, ow


def oracle_flash4(cfg: Config, X64, outs64, ow, dtype=None):
    convs = ow["conv"] if cfg.K_r == 4 else [[], []]
    return O.xhcf4_group(X64, outs64, ow["w_full"], ow["w_post"], ow["w_act_last"], cfg.m, cfg.k, convs,
                         ow["alpha"], ow["b"], iters=cfg.iters, use_mgs=bool(cfg.use_mgs), dtype=dtype or cfg.dtype)


def gpu_flash4(lib, cfg: Config, X, outs, wd, stream=None):
    """xhcf4_pre and xhcf4_post for q = 1..4 through the C ABI; CPU copies of
    every sublayer's input and post-map, the state after each sublayer, the
    routing and the final MLP's residual map."""
    from stream_residual_mixing_amd.binding import flash4_weights_to_device
    w = flash4_weights_to_device(wd)
    Xd = X.to("cuda")
    inp = torch.empty((cfg.T, cfg.C), dtype=cfg.torch_dtype, device="cuda")
    bases = torch.empty((3, cfg.T, cfg.C), dtype=cfg.torch_dtype, device="cuda")
    ws = lib.flash4_workspace(cfg)
    lib.xhcf4_pre(cfg, w, Xd, inp, bases, ws, stream)
    kq = [1, cfg.K_r, 1, cfg.K_r]
    arr = lib.flash4_ws_arrays(cfg, ws, kq[0])
    res = dict(idx=arr["idx"].cpu(), p=arr["p"].cpu(), h_pre=arr["h_pre"].cpu(), bases=bases.cpu(),
               inputs=[inp.cpu()], h_post=[arr["h_post"].cpu()], states=[])
    for q in range(1, 5):
        lib.xhcf4_post(cfg, w, q, Xd, outs[q - 1].to("cuda"), bases, inp, ws, stream)
        torch.cuda.synchronize()
        res["states"].append(Xd.cpu())
        if q < 4:
            res["inputs"].append(inp.cpu())
            arr = lib.flash4_ws_arrays(cfg, ws, kq[q])
            res["h_post"].append(arr["h_post"].cpu())
            if q == 3:
                res["h_res"] = arr["h_res"].cpu()
    return res


def err_with_allowance(g, r, allow, floor=1e-2, per_token=True):
    """Relative error (floored as in rel_err) after an absolute allowance."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    return float(np.max(np.maximum(np.abs(g.reshape(r.shape) - r) - allow, 0.0) / _floor_den(r, floor, per_token)))


def compare_flash4(g, o, tol, dtype):
    """Every stored tensor of a group.  Each side rounds what it stores (the
    bases, the rewritten active rows after each sublayer), and two correct
    roundings may differ by one unit in the last place; after sublayer q a
    row has been rounded q times, so the state after sublayer q is allowed q
    units of the largest active row at that channel, and the input of
    sublayer q one unit of its base plus q - 1 such units (all from oracle
    values).  Maps and router weights keep the plain bar."""
    assert np.array_equal(g["idx"].numpy(), o["I"]), "active indices differ"
    I = o["I"]
    prev = [None] + o["states"][:3]
    errs = {"p": rel_err(g["p"].numpy(), o["p"]), "h_pre": rel_err(g["h_pre"].numpy(), np.stack(o["h_pre"]))}
    for q in range(4):
        if q == 0:
            errs["inp1"] = rel_err(f64(g["inputs"][0]), o["inputs"][0])
        else:
            big = np.take_along_axis(np.abs(prev[q]), I[:, :, None], axis=1).max(axis=1)
            allow = ulp(o["bases"][q - 1], dtype) + q * ulp(big, dtype)
            errs[f"inp{q + 1}"] = err_with_allowance(f64(g["inputs"][q]), o["inputs"][q], allow)
        st = o["states"][q]
        big = np.take_along_axis(np.abs(st), I[:, :, None], axis=1).max(axis=1)
        errs[f"X{q + 1}"] = err_with_allowance(f64(g["states"][q]), st, (q + 1) * ulp(big, dtype)[:, None, :])
        errs[f"h_post{q + 1}"] = rel_err(g["h_post"][q].numpy().reshape(o["maps"][q]["h_post"].shape),
                                         o["maps"][q]["h_post"])
    errs["h_res"] = rel_err(g["h_res"].numpy(), o["maps"][3]["h_res"])
    errs["bases"] = max(rel_err(f64(g["bases"][i]), o["bases"][i]) for i in range(3))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"errors above {tol}: {bad} (all: {errs})"
    return errs
