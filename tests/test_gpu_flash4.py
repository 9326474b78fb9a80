"""GPU parity of the xHC-Flash-4sub group (xhcf4_pre, then xhcf4_post for
the four sublayers, through the C ABI) against the float64 oracle: routing
exactly, and element by element every sublayer's input and post-map, the
non-active bases, the final residual map and the state after each sublayer.
Each side rounds what it stores, so the state after sublayer q and the input
of sublayer q carry an allowance of a few units in the last place of the
values involved, computed from oracle values (see ``cases.compare_flash4``).
Tokens whose routing margin is below 1e-4 are redrawn.
"""
import pytest
import torch

import cases as K
from stream_residual_mixing_amd.binding import Config

pytestmark = pytest.mark.gpu

CASES = [
    # N, k, m, C, B, S, n_convs, dtype
    (16, 4, 2, 512, 2, 45, 3, "bf16"),
    (16, 4, 2, 4096, 1, 40, 3, "bf16"),
    (16, 4, 2, 256, 2, 33, 3, "f32"),
    (16, 4, 2, 512, 1, 50, 0, "bf16"),
    (8, 4, 2, 256, 2, 30, 3, "bf16"),
    (4, 4, 2, 256, 1, 37, 3, "bf16"),
    (1, 1, 1, 256, 2, 20, 3, "bf16"),
    (16, 4, 2, 96, 1, 19, 3, "bf16"),
    (8, 4, 2, 128, 2, 21, 3, "f32"),
    (4, 4, 4, 128, 1, 29, 3, "f32"),
    (1, 1, 1, 64, 2, 17, 3, "f32"),
    (8, 4, 1, 160, 2, 13, 0, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "N{}k{}m{}C{}_{}x{}_c{}_{}".format(*c))
def test_flash4_group_matches_oracle(lib, case):
    N, k, m, C, B, S, nc, dt = case
    cfg = Config(N=N, k=k, m=m, C=C, B=B, S=S, n_convs=nc, dtype=dt)
    print("flash4 case", case, flush=True)
    X, outs, wd, ow = K.flash4_inputs(cfg, seed=31)
    g = K.gpu_flash4(lib, cfg, X, outs, wd)
    o = K.oracle_flash4(cfg, K.f64(X), [K.f64(t) for t in outs], ow)
    errs = K.compare_flash4(g, o, K.TOL[dt], dt)
    print("  errors", {key: f"{v:.1e}" for key, v in errs.items()}, flush=True)


def test_flash4_group_leaves_inactive_streams_bit_identical(lib):
    cfg = Config(N=16, k=4, m=2, C=1024, B=2, S=40, n_convs=3, dtype="bf16")
    X, outs, wd, ow = K.flash4_inputs(cfg, seed=32)
    g = K.gpu_flash4(lib, cfg, X, outs, wd)
    act = torch.zeros((cfg.T, cfg.N), dtype=torch.bool)
    act.scatter_(1, g["idx"].long(), True)
    for q in range(4):
        same = (g["states"][q] == X).all(-1)
        assert bool((same | act).all()), f"sublayer {q + 1} changed a stream outside the active list"


def test_flash4_full_size_sampled_tokens(lib):
    """One group at the bench shape (N = 16, k = 4, C = 4096, 2 x 8192 tokens)
    on the GPU; sampled tokens against the oracle, each recomputed from its
    state row and its 12-token output windows (the two MLP sublayers'
    convolutions look back 11 tokens), under the bars of the small cases;
    every token checked for routing validity and untouched streams."""
    import numpy as np
    from stream_residual_mixing_amd import synth
    from stream_residual_mixing_amd.binding import flash4_weights_to_device
    N, k, m, C, B, S, seed = 16, 4, 2, 4096, 2, 8192, 6
    cfg = Config(N=N, k=k, m=m, C=C, B=B, S=S, n_convs=3, dtype="bf16")
    T = cfg.T
    wd = synth.xhcf4_group_weights(seed, 0, N, k, C, 4, "bf16")
    ow = K.flash4_oracle_weights(wd)
    toks = K.sample_tokens(B, S, 10, seed)
    attempts, ref = {}, {}
    from oracle import hc_oracle as O
    for j, t in enumerate(toks):
        t = int(t)
        if j % 16 == 0:
            print(f"oracle: token {j} of {len(toks)}", flush=True)
        for _ in range(20):
            x = K.f64(synth.state_rows(seed, [t], N, C, "bf16", attempts))[0]
            z = O.xhc_router_logits(x[None], ow["w_full"][:, :N])
            if O.xhc_topk_margin(z, m, k)[0] >= K.MARGIN:
                break
            attempts[t] = attempts.get(t, 0) + 1
        w = K.WINDOW
        Xw = np.zeros((w, N, C))
        Xw[-1] = x
        wins = [K.out_window(seed, q, t, S, C, w)[None] for q in range(4)]
        sub = Config(N=N, k=k, m=m, C=C, B=1, S=w, n_convs=3, dtype="bf16")
        ref[t] = K.oracle_flash4(sub, Xw, wins, ow)
    print(f"oracle ready: {len(toks)} sampled tokens, {sum(attempts.values())} redraws", flush=True)

    X = synth.state(seed, T, N, C, "bf16", attempts).to("cuda")
    X0 = X.clone()
    outs = [synth.sublayer_out(seed, q, B, S, C, "bf16").to("cuda") for q in range(4)]
    w = flash4_weights_to_device(wd)
    inp = torch.empty((T, C), dtype=torch.bfloat16, device="cuda")
    bases = torch.empty((3, T, C), dtype=torch.bfloat16, device="cuda")
    ws = lib.flash4_workspace(cfg)
    sel = torch.as_tensor(toks, device="cuda")
    lib.xhcf4_pre(cfg, w, X, inp, bases, ws)
    kq = [1, 4, 1, 4]
    arr = lib.flash4_ws_arrays(cfg, ws, 1)
    g = dict(idx=arr["idx"][sel].cpu(), p=arr["p"][sel].cpu(), h_pre=arr["h_pre"][:, sel].cpu(),
             bases=bases[:, sel].cpu(), inputs=[inp[sel].cpu()], h_post=[arr["h_post"][sel].cpu()], states=[])
    idx_all = arr["idx"].long().clone()
    for q in range(1, 5):
        lib.xhcf4_post(cfg, w, q, X, outs[q - 1], bases, inp, ws)
        g["states"].append(X[sel].cpu())
        if q < 4:
            g["inputs"].append(inp[sel].cpu())
            arr = lib.flash4_ws_arrays(cfg, ws, kq[q])
            g["h_post"].append(arr["h_post"][sel].cpu())
            if q == 3:
                g["h_res"] = arr["h_res"][sel].cpu()
    torch.cuda.synchronize()
    print("GPU group done", flush=True)
    act = torch.zeros((T, N), dtype=torch.bool, device="cuda")
    act.scatter_(1, idx_all, True)
    assert bool(((X == X0).all(-1) | act).all()), "a stream outside the active list changed"
    srt = idx_all.sort(dim=1).values
    assert bool((srt[:, 1:] > srt[:, :-1]).all()) and bool((idx_all[:, :m] == torch.arange(m, device="cuda")).all())

    o = dict(I=np.stack([ref[int(t)]["I"][-1] for t in toks]), p=np.stack([ref[int(t)]["p"][-1] for t in toks]),
             h_pre=[np.stack([ref[int(t)]["h_pre"][q][-1] for t in toks]) for q in range(4)],
             bases=[np.stack([ref[int(t)]["bases"][q][-1] for t in toks]) for q in range(3)],
             inputs=[np.stack([ref[int(t)]["inputs"][q][-1] for t in toks]) for q in range(4)],
             states=[np.stack([ref[int(t)]["states"][q][-1] for t in toks]) for q in range(4)],
             maps=[dict(h_post=np.stack([ref[int(t)]["maps"][q]["h_post"][-1] for t in toks]),
                        h_res=np.stack([ref[int(t)]["maps"][q]["h_res"][-1] for t in toks])) for q in range(4)])
    errs = K.compare_flash4(g, o, K.TOL["bf16"], "bf16")
    print("  sampled errors", {key: f"{v:.1e}" for key, v in errs.items()}, flush=True)
