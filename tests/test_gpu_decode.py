"""GPU parity of single-token decode (xhc_pre on one new token per sequence,
then xhc_post_decode with the conv history in a 12-slot ring) against the
float64 oracle.

One step: ring contents and positions are seeded (positions before, at and
past the ring length, and a sequence start whose stale ring must not leak);
the new state is compared element by element with the oracle's decode step,
the ring bit for bit (the new output in slot position % 12, every other slot
unchanged), the active lists exactly.  A whole sequence decoded token by
token is compared with the oracle's prefill of the same tokens.
"""
import numpy as np
import pytest
import torch

import cases as K
from oracle import hc_oracle as O
from stream_residual_mixing_amd import synth
from stream_residual_mixing_amd.binding import Config, weights_to_device

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("dt,C,use_mgs", [("bf16", 1024, 1), ("f32", 256, 1), ("bf16", 512, 0), ("bf16", 1120, 1)])
def test_decode_step_matches_oracle(lib, dt, C, use_mgs):
    N, k, m = 16, 4, 2
    steps = np.array([0, 3, 11, 12, 40, 7, 1], dtype=np.int32)
    B = len(steps)
    cfg = Config(N=N, k=k, m=m, C=C, B=B, S=1, n_convs=3, use_mgs=use_mgs, dtype=dt)
    _print("decode step", dt, C, use_mgs)
    X, out, wd, ow = K.xhc_inputs(cfg, seed=41)
    ring = synth._round(np.random.default_rng([41, 9]).standard_normal((B, O.RING, C)), dt)
    # oracle: maps from the pre stage, then one decode step
    pre = O.xhc_pre(K.f64(X), ow["w_full"], ow["w_act"], m, k, 4, (ow["alpha_pre"], ow["alpha_res"], ow["alpha_post"]),
                    ow["b_pre"], ow["b_res"], ow["b_post"], iters=cfg.iters)
    Xo, ringo = O.xhc_decode_post(K.f64(X), K.f64(out).reshape(B, C), K.f64(ring), steps, pre["I"], pre["p"],
                                  pre["h_res"], pre["h_post"], ow["conv"], bool(use_mgs))
    # GPU
    w = weights_to_device(wd)
    Xd, outd, ringd = X.cuda(), out.reshape(B, C).cuda(), ring.cuda()
    inp = torch.empty((B, C), dtype=cfg.torch_dtype, device="cuda")
    ws = lib.workspace(cfg)
    lib.xhc_pre(cfg, w, Xd, inp, ws)
    idx = lib.ws_arrays(cfg, ws)["idx"].cpu().numpy()
    lib.xhc_post_decode(cfg, w, Xd, outd, ringd, torch.from_numpy(steps).cuda(), ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx, pre["I"]), "active indices differ"
    err = K.rel_err(K.f64(Xd.cpu()), O.round_state(Xo, dt))
    _print("  state error", f"{err:.2e}")
    assert err <= K.TOL[dt]
    rg = ringd.cpu()
    for b in range(B):
        for slot in range(O.RING):
            want = out[b, 0] if slot == steps[b] % O.RING else ring[b, slot]
            assert torch.equal(rg[b, slot], want), (b, slot)
    assert np.array_equal(K.f64(rg), ringo)


@pytest.mark.parametrize("N,k,m,dt", [(16, 2, 1, "bf16"), (8, 4, 2, "f32"), (4, 4, 4, "bf16"), (1, 1, 1, "f32"),
                                      (16, 4, 0, "bf16")])
def test_decode_step_other_shapes(lib, N, k, m, dt):
    """Every built (N, k): one decode step against the oracle's, the ring
    bit for bit."""
    C = 192
    steps = np.array([0, 5, 11, 12, 29], dtype=np.int32)
    B = len(steps)
    cfg = Config(N=N, k=k, m=m, C=C, B=B, S=1, n_convs=3, dtype=dt)
    _print("decode step", N, k, m, dt)
    X, out, wd, ow = K.xhc_inputs(cfg, seed=43)
    ring = synth._round(np.random.default_rng([43, 9]).standard_normal((B, O.RING, C)), dt)
    pre = O.xhc_pre(K.f64(X), ow["w_full"], ow["w_act"], m, k, 4, (ow["alpha_pre"], ow["alpha_res"], ow["alpha_post"]),
                    ow["b_pre"], ow["b_res"], ow["b_post"], iters=cfg.iters)
    Xo, ringo = O.xhc_decode_post(K.f64(X), K.f64(out).reshape(B, C), K.f64(ring), steps, pre["I"], pre["p"],
                                  pre["h_res"], pre["h_post"], ow["conv"], True)
    w = weights_to_device(wd)
    Xd, outd, ringd = X.cuda(), out.reshape(B, C).cuda(), ring.cuda()
    inp = torch.empty((B, C), dtype=cfg.torch_dtype, device="cuda")
    ws = lib.workspace(cfg)
    lib.xhc_pre(cfg, w, Xd, inp, ws)
    idx = lib.ws_arrays(cfg, ws)["idx"].cpu().numpy()
    lib.xhc_post_decode(cfg, w, Xd, outd, ringd, torch.from_numpy(steps).cuda(), ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx, pre["I"]), "active indices differ"
    err = K.rel_err(K.f64(Xd.cpu()), O.round_state(Xo, dt))
    _print("  state error", f"{err:.2e}")
    assert err <= K.TOL[dt]
    assert np.array_equal(K.f64(ringd.cpu()), ringo)


def test_decode_sequence_matches_the_prefill(lib):
    """Two sequences of 20 tokens decoded one token at a time (pre + decode
    write per token, the ring carried on the GPU) against the oracle's
    prefill sublayer over the whole sequences."""
    N, k, m, C, B, S = 16, 4, 2, 512, 2, 20
    full = Config(N=N, k=k, m=m, C=C, B=B, S=S, n_convs=3, dtype="bf16")
    X, out, wd, ow = K.xhc_inputs(full, seed=42)
    ref = K.oracle_xhc(full, K.f64(X), K.f64(out), ow)
    step_cfg = Config(N=N, k=k, m=m, C=C, B=B, S=1, n_convs=3, dtype="bf16")
    w = weights_to_device(wd)
    ring = torch.zeros((B, O.RING, C), dtype=torch.bfloat16, device="cuda").normal_()   # stale contents
    ws = lib.workspace(step_cfg)
    inp = torch.empty((B, C), dtype=torch.bfloat16, device="cuda")
    Xg = torch.empty_like(X)
    inps = torch.empty((B * S, C), dtype=torch.bfloat16)
    for s in range(S):
        rows = [b * S + s for b in range(B)]
        Xd = X[rows].cuda()
        lib.xhc_pre(step_cfg, w, Xd, inp, ws)
        steps = torch.full((B,), s, dtype=torch.int32, device="cuda")
        lib.xhc_post_decode(step_cfg, w, Xd, out[:, s].contiguous().cuda(), ring, steps, ws)
        torch.cuda.synchronize()
        Xg[rows] = Xd.cpu()
        inps[rows] = inp.cpu()
    errs = {"X": K.rel_err(K.f64(Xg), ref["X"]), "inp": K.rel_err(K.f64(inps), ref["inp"])}
    _print("  decode vs prefill", {key: f"{v:.2e}" for key, v in errs.items()})
    assert all(v <= K.TOL["bf16"] for v in errs.values()), errs
