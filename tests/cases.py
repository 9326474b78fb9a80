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


def rel_err(g, r, floor=1e-2):
    """max_e |g - r| / max(|r|, floor * RMS(r)): relative error with a floor
    so that elements near zero are measured against the array's scale."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    den = np.maximum(np.abs(r), floor * rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(g - r) / den))


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
    """Oracle xHC sublayer.  X64 [T,N,C]; out64 [B,S,C]."""
    return O.xhc_sublayer(X64, out64, ow["w_full"], ow["w_act"], cfg.m, cfg.k, ow["conv"],
                          (ow["alpha_pre"], ow["alpha_res"], ow["alpha_post"]),
                          ow["b_pre"], ow["b_res"], ow["b_post"], iters=cfg.iters,
                          use_mgs=bool(cfg.use_mgs), dtype=dtype or cfg.dtype)


def oracle_mhc(cfg: Config, X64, out64, ow, dtype=None):
    return O.mhc_sublayer(X64, out64.reshape(-1, cfg.C), ow["w_full"],
                          (ow["alpha_pre"], ow["alpha_post"], ow["alpha_res"]),
                          ow["b_pre"], ow["b_post"], ow["b_res"], iters=cfg.iters, dtype=dtype or cfg.dtype)


def margins(cfg: Config, X64, ow):
    z = O.xhc_router_logits(X64, ow["w_full"][:, :cfg.N])
    return O.xhc_topk_margin(z, cfg.m, cfg.k)


def xhc_inputs(cfg: Config, seed, layer=0, resample=True):
    """Seeded X, out and weights for an xHC case; tokens whose routing
    margin (oracle logits) is below MARGIN are redrawn."""
    wd = synth.xhc_layer_weights(seed, layer, cfg.N, cfg.k, cfg.C, cfg.K_r, cfg.dtype)
    ow = oracle_weights(wd)
    attempts = {}
    X = synth.state(seed, cfg.T, cfg.N, cfg.C, cfg.dtype)
    if resample:
        for _ in range(20):
            bad = np.nonzero(margins(cfg, f64(X), ow) < MARGIN)[0]
            if bad.size == 0:
                break
            for t in bad:
                attempts[int(t)] = attempts.get(int(t), 0) + 1
            X[bad] = synth.state_rows(seed, bad, cfg.N, cfg.C, cfg.dtype, attempts)
    out = synth.sublayer_out(seed, layer, cfg.B, cfg.S, cfg.C, cfg.dtype)
    return X, out, wd, ow


def mhc_inputs(cfg: Config, seed, layer=0):
    wd = synth.mhc_layer_weights(seed, layer, cfg.N, cfg.C, cfg.dtype)
    X = synth.state(seed, cfg.T, cfg.N, cfg.C, cfg.dtype)
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
    """Errors per quantity; indices must match exactly."""
    sel = slice(None) if tokens is None else tokens
    gi = g["idx"].numpy()[sel]
    assert np.array_equal(gi, o["I"][sel] if tokens is None else o["I"]), "active indices differ"
    errs = {}
    for key, okey in (("inp", "inp"), ("X", "X"), ("h_pre", "h_pre"), ("h_res", "h_res"),
                      ("h_post", "h_post"), ("p", "p")):
        gv = f64(g[key])[sel] if key in ("inp", "X") else g[key].numpy().astype(np.float64)[sel]
        errs[key] = rel_err(gv, o[okey])
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"errors above {tol}: {bad} (all: {errs})"
    return errs


def compare_mhc(g, o, tol, tokens=None):
    sel = slice(None) if tokens is None else tokens
    errs = {}
    for key in ("inp", "X", "h_pre", "h_res", "h_post"):
        gv = f64(g[key])[sel] if key in ("inp", "X") else g[key].numpy().astype(np.float64)[sel]
        errs[key] = rel_err(gv, o[key])
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"errors above {tol}: {bad} (all: {errs})"
    return errs
