"""GPU parity of the xHC-Flash block (xhcf_pre, xhcf_mid, xhcf_post through
the C ABI) against the float64 oracle.

Small cases compare every element of every stored tensor: both readouts,
the corrected MLP input, the state after the attention write and after the
block, the maps and router weights; active indices must match exactly.  The
corrected MLP input is held to the same bar after one unit in the last place
of the stored base readout is allowed (both sides round that base to the
state dtype before correcting it, and where the correction nearly cancels
the base, one unit of it is large against the result).  For the same
reason the state after the MLP write, which mixes the active rows each side
stored after the attention write, is allowed one unit of the largest row
mixed at each channel.  Both allowances are computed from oracle values.
Tokens whose routing margin is below 1e-4 are redrawn (several active lists
would then be correct).  A full-size block at N = 16, k = 4, C = 4096,
2 x 8192 tokens (the shape bench.py times) is checked on sampled tokens, each
recomputed by the oracle from its state row and its 12-token output windows,
and on properties of every token.
"""
import numpy as np
import pytest
import torch

import cases as K
from stream_residual_mixing_amd import synth
from stream_residual_mixing_amd.binding import Config, flash_weights_to_device

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


CASES = [
    # N, k, m, C, B, S, n_convs, dtype
    (16, 4, 2, 512, 2, 45, 3, "bf16"),    # ragged 16-token tiles and 64-token blocks, sequence start inside a block
    (16, 4, 2, 4096, 1, 40, 3, "bf16"),   # every channel slice of the bench shape
    (16, 4, 2, 256, 2, 33, 3, "f32"),
    (16, 4, 2, 512, 1, 50, 0, "bf16"),    # MLP side without temporal augmentation
    (16, 4, 0, 256, 1, 30, 3, "bf16"),    # no fixed streams
    (8, 4, 2, 256, 2, 30, 3, "bf16"),
    (4, 4, 2, 256, 1, 37, 3, "bf16"),
    (1, 1, 1, 256, 2, 20, 3, "bf16"),
    (16, 4, 2, 96, 1, 19, 3, "bf16"),     # C not a multiple of the 128-channel slices
    (16, 4, 2, 160, 2, 17, 3, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "N{}k{}m{}C{}_{}x{}_c{}_{}".format(*c))
def test_flash_block_matches_oracle(lib, case):
    N, k, m, C, B, S, nc, dt = case
    cfg = Config(N=N, k=k, m=m, C=C, B=B, S=S, n_convs=nc, dtype=dt)
    _print("flash case", case)
    X, out_a, out_m, wd, ow, _ = K.flash_inputs(cfg, seed=21)
    g = K.gpu_flash(lib, cfg, X, out_a, out_m, wd)
    o = K.oracle_flash(cfg, K.f64(X), K.f64(out_a), K.f64(out_m), ow)
    errs = K.compare_flash(g, o, K.TOL[dt], dtype=dt)
    _print("  errors", {key: f"{v:.1e}" for key, v in errs.items()})


def test_flash_block_leaves_inactive_streams_bit_identical(lib):
    cfg = Config(N=16, k=4, m=2, C=1024, B=2, S=70, n_convs=3, dtype="bf16")
    X, out_a, out_m, wd, ow, _ = K.flash_inputs(cfg, seed=22)
    g = K.gpu_flash(lib, cfg, X, out_a, out_m, wd)
    idx = g["idx"].long()
    act = torch.zeros((cfg.T, cfg.N), dtype=torch.bool)
    act.scatter_(1, idx, True)
    same1 = (g["X1"] == X).all(-1)
    same2 = (g["X"] == X).all(-1)
    assert bool((same1 == ~act).all()), "attention write touched an inactive stream or missed an active one"
    assert bool((same2 | act).all()), "block changed a stream outside the active list"


def test_flash_empty_batch_is_a_no_op(lib):
    cfg = Config(N=16, k=4, m=2, C=256, B=0, S=8, n_convs=3, dtype="bf16")
    wd = synth.xhcf_block_weights(1, 0, 16, 4, 256, 4, "bf16")
    w = flash_weights_to_device(wd)
    X = torch.empty((0, 16, 256), dtype=torch.bfloat16, device="cuda")
    e = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    lib.xhcf_pre(cfg, w, X, e, e.clone(), ws)
    lib.xhcf_mid(cfg, w, X, e.clone(), e.clone(), ws)
    lib.xhcf_post(cfg, w, X, e.clone(), ws)
    torch.cuda.synchronize()


def test_flash_full_size_sampled_tokens(lib):
    """One block at the bench shape, all tokens on the GPU; sampled tokens
    against the oracle, every token against size-independent properties."""
    N, k, m, C, B, S = 16, 4, 2, 4096, 2, 8192
    seed = 5
    cfg = Config(N=N, k=k, m=m, C=C, B=B, S=S, n_convs=3, dtype="bf16")
    T = cfg.T
    wd = synth.xhcf_block_weights(seed, 0, N, k, C, 4, "bf16")
    ow = K.flash_oracle_weights(wd)
    toks = K.sample_tokens(B, S, 12, seed)
    attempts, ref = {}, {}
    for j, t in enumerate(toks):
        t = int(t)
        if j % 16 == 0:
            _print(f"oracle: token {j} of {len(toks)}")
        for _ in range(20):
            x = K.f64(synth.state_rows(seed, [t], N, C, "bf16", attempts))[0]
            if K.flash_margins(cfg, x[None], ow)[0] >= K.MARGIN:
                break
            attempts[t] = attempts.get(t, 0) + 1
        w = K.WINDOW
        Xw = np.zeros((w, N, C))
        Xw[-1] = x
        wa = K.out_window(seed, 0, t, S, C, w)
        wm = K.out_window(seed, 1, t, S, C, w)
        sub = Config(N=N, k=k, m=m, C=C, B=1, S=w, n_convs=3, dtype="bf16")
        r = K.oracle_flash(sub, Xw, wa[None], wm[None], ow)
        ref[t] = {key: v[-1] for key, v in r.items() if isinstance(v, np.ndarray) and v.ndim >= 1}
    _print(f"oracle ready: {len(toks)} sampled tokens, {sum(attempts.values())} redraws")

    X = synth.state(seed, T, N, C, "bf16", attempts).to("cuda")
    X0 = X.clone()
    out_a = synth.sublayer_out(seed, 0, B, S, C, "bf16").to("cuda")
    out_m = synth.sublayer_out(seed, 1, B, S, C, "bf16").to("cuda")
    w = flash_weights_to_device(wd)
    inp_a = torch.empty((T, C), dtype=torch.bfloat16, device="cuda")
    inp_m = torch.empty_like(inp_a)
    ws = lib.flash_workspace(cfg)
    lib.xhcf_pre(cfg, w, X, inp_a, inp_m, ws)
    pre = {key: v.clone() for key, v in lib.flash_ws_arrays(cfg, ws).items() if key not in ("h_res", "h_post_mlp")}
    lib.xhcf_mid(cfg, w, X, out_a, inp_m, ws)
    X1 = X.clone()
    arr = lib.flash_ws_arrays(cfg, ws)
    maps = dict(h_res=arr["h_res"].clone(), h_post=arr["h_post_mlp"].clone())
    lib.xhcf_post(cfg, w, X, out_m, ws)
    torch.cuda.synchronize()
    _print("GPU block done")

    # every token: active lists, gates, row sums, untouched streams
    idx = pre["idx"].long()
    assert bool((idx >= 0).all() and (idx < N).all())
    assert bool((idx[:, :m] == torch.arange(m, device=idx.device)).all())
    srt = idx.sort(dim=1).values
    assert bool((srt[:, 1:] > srt[:, :-1]).all())
    assert bool((pre["p"][:, :m] == 1).all())
    for name, v, lo, hi in (("h_pre_attn", pre["h_pre_attn"], 0, 1), ("h_pre_mlp", pre["h_pre_mlp"], 0, 1),
                            ("h_post_attn", pre["h_post_attn"], 0, 2), ("h_post", maps["h_post"], 0, 2),
                            ("h_res", maps["h_res"], 0, 1 + 1e-4)):
        assert bool(torch.isfinite(v).all() and (v >= lo).all() and (v <= hi).all()), name
    assert float((maps["h_res"].sum(-1) - 1).abs().max()) < 1e-4
    act = torch.zeros((T, N), dtype=torch.bool, device="cuda")
    act.scatter_(1, idx, True)
    assert bool(((X == X0).all(-1) | act).all()), "a stream outside the active list changed"

    # sampled tokens, element by element
    sel = torch.as_tensor(toks, device="cuda")
    g = dict(inp_attn=inp_a[sel].cpu(), inp_mlp=inp_m[sel].cpu(), X1=X1[sel].cpu(), X=X[sel].cpu(),
             idx=pre["idx"][sel].cpu(), p=pre["p"][sel].cpu(), h_pre_attn=pre["h_pre_attn"][sel].cpu(),
             h_pre_mlp=pre["h_pre_mlp"][sel].cpu(), h_post_attn=pre["h_post_attn"][sel].cpu(),
             h_res=maps["h_res"][sel].cpu(), h_post=maps["h_post"][sel].cpu())
    o = {key: np.stack([ref[int(t)][key] for t in toks]) for key in ref[int(toks[0])]}
    assert np.array_equal(g["idx"].numpy(), o["I"]), "active indices differ"
    errs = {}
    for key in ("inp_attn", "inp_mlp", "X1", "X", "h_pre_attn", "h_pre_mlp", "h_post_attn", "h_res", "h_post", "p"):
        gv = K.f64(g[key]) if g[key].dtype == torch.bfloat16 else g[key].numpy().astype(np.float64)
        if key == "inp_mlp":
            errs[key] = K.corrected_input_err(gv, o[key], o["inp_mlp_base"], "bf16")
        elif key == "X":
            errs[key] = K.mixed_state_err(gv, o[key], o["X1"], o["I"], "bf16")
        else:
            errs[key] = K.rel_err(gv, o[key])
    _print("  sampled errors", {key: f"{v:.1e}" for key, v in errs.items()})
    bad = {key: v for key, v in errs.items() if not v <= K.TOL["bf16"]}
    assert not bad, bad
