"""GPU parity of the HIP library against the float64 oracle, element by
element, at sizes the oracle finishes in seconds (several tiles, ragged
tails, sequence boundaries inside a tile).  Calls go through the C ABI.

Tolerances: active indices exact; fp32 mode <= 1e-4 and bf16 state <= 2e-2
in the floored relative metric of ``cases.rel_err``; special cases that the
pages fix exactly are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import cases as K
from stream_residual_mixing_amd import synth
from stream_residual_mixing_amd.binding import Config

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


# ----------------------------------------------------------------------- mHC

def test_mhc_small_fp32_config(lib):
    """mHC, N=4, C=256, 1 x 64 tokens, fp32 state, seed 0."""
    cfg = Config(N=4, C=256, B=1, S=64, dtype="f32")
    X, out, wd, ow = K.mhc_inputs(cfg, seed=0)
    g = K.gpu_mhc(lib, cfg, X, out, wd)
    o = K.oracle_mhc(cfg, K.f64(X), K.f64(out), ow)
    _print("mhc f32", K.compare_mhc(g, o, K.TOL["f32"]))


@pytest.mark.parametrize("N", [2, 4, 8, 16])
def test_mhc_bf16_ragged(lib, N):
    cfg = Config(N=N, C=256, B=2, S=37, dtype="bf16")
    X, out, wd, ow = K.mhc_inputs(cfg, seed=50 + N)
    g = K.gpu_mhc(lib, cfg, X, out, wd)
    o = K.oracle_mhc(cfg, K.f64(X), K.f64(out), ow)
    _print("mhc bf16", N, K.compare_mhc(g, o, K.TOL["bf16"]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mhc_one_stream_is_plain_residual(lib, dtype):
    """N = 1 with every map fixed at 1 gives x + out, rounded once."""
    cfg = Config(N=1, C=96, B=3, S=7, dtype=dtype)
    X, out, wd, ow = K.mhc_inputs(cfg, seed=60)
    wd = dict(wd, b_pre=torch.tensor([40.0]), alpha_pre=0.0, alpha_res=0.0, alpha_post=0.0)
    g = K.gpu_mhc(lib, cfg, X, out, wd)
    from oracle import hc_oracle as O
    exp = O.round_state(K.f64(X)[:, 0] + K.f64(out).reshape(-1, cfg.C), dtype)
    np.testing.assert_array_equal(K.f64(g["X"])[:, 0], exp)
    np.testing.assert_array_equal(K.f64(g["inp"]), K.f64(X)[:, 0])


# ----------------------------------------------------------------------- xHC

@pytest.mark.parametrize("mlp", [False, True])
def test_xhc_fp32_n16_k4(lib, mlp):
    """xHC fp32: N=16, k=4, m=2, C=256, 2 x 64 tokens."""
    cfg = Config(N=16, k=4, m=2, C=256, B=2, S=64, n_convs=3 if mlp else 0, dtype="f32")
    X, out, wd, ow = K.xhc_inputs(cfg, seed=70 + mlp)
    g = K.gpu_xhc(lib, cfg, X, out, wd)
    o = K.oracle_xhc(cfg, K.f64(X), K.f64(out), ow)
    _print("xhc f32", mlp, K.compare_xhc(g, o, K.TOL["f32"]))


@pytest.mark.parametrize("N,k,m", [(16, 4, 2), (16, 2, 1), (8, 4, 2), (16, 4, 0)])
@pytest.mark.parametrize("mlp", [False, True])
def test_xhc_bf16_ragged(lib, N, k, m, mlp):
    cfg = Config(N=N, k=k, m=m, C=512, B=2, S=77, n_convs=3 if mlp else 0, dtype="bf16")
    X, out, wd, ow = K.xhc_inputs(cfg, seed=80 + N + k + m + mlp)
    g = K.gpu_xhc(lib, cfg, X, out, wd)
    o = K.oracle_xhc(cfg, K.f64(X), K.f64(out), ow)
    _print("xhc bf16", N, k, m, mlp, K.compare_xhc(g, o, K.TOL["bf16"]))


@pytest.mark.parametrize("N,k,m", [(16, 2, 1), (8, 4, 2), (16, 4, 0), (4, 4, 2), (4, 4, 4), (1, 1, 1)])
@pytest.mark.parametrize("mlp", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_xhc_every_built_shape(lib, N, k, m, mlp, dtype):
    """Every built (N, k) in both dtypes, attention- and MLP-type, a ragged tile."""
    cfg = Config(N=N, k=k, m=m, C=192, B=2, S=29, n_convs=3 if mlp else 0, dtype=dtype)
    X, out, wd, ow = K.xhc_inputs(cfg, seed=110 + N + k + m + mlp)
    g = K.gpu_xhc(lib, cfg, X, out, wd)
    o = K.oracle_xhc(cfg, K.f64(X), K.f64(out), ow)
    _print("xhc shape", N, k, m, mlp, dtype, K.compare_xhc(g, o, K.TOL[dtype]))


@pytest.mark.parametrize("B,S", [(3, 13), (5, 1), (1, 130)])
def test_xhc_sequence_boundaries(lib, B, S):
    """Causal convolutions restart at every sequence start, also inside a tile."""
    cfg = Config(N=16, k=4, m=2, C=256, B=B, S=S, n_convs=3, dtype="bf16")
    X, out, wd, ow = K.xhc_inputs(cfg, seed=90 + B + S)
    g = K.gpu_xhc(lib, cfg, X, out, wd)
    o = K.oracle_xhc(cfg, K.f64(X), K.f64(out), ow)
    _print("xhc seq", B, S, K.compare_xhc(g, o, K.TOL["bf16"]))


def test_xhc_without_gram_schmidt(lib):
    cfg = Config(N=16, k=4, m=2, C=256, B=2, S=40, n_convs=3, use_mgs=0, dtype="bf16")
    X, out, wd, ow = K.xhc_inputs(cfg, seed=95)
    g = K.gpu_xhc(lib, cfg, X, out, wd)
    o = K.oracle_xhc(cfg, K.f64(X), K.f64(out), ow)
    _print("xhc no mgs", K.compare_xhc(g, o, K.TOL["bf16"]))


def test_xhc_inactive_rows_are_bit_identical(lib):
    """Only the k active rows of a token are written (explainer, "What xHC
    changes": the other streams pass through untouched)."""
    cfg = Config(N=16, k=4, m=2, C=512, B=2, S=50, n_convs=3, dtype="bf16")
    X, out, wd, ow = K.xhc_inputs(cfg, seed=96)
    g = K.gpu_xhc(lib, cfg, X, out, wd)
    idx = g["idx"].numpy()
    mask = np.ones((cfg.T, cfg.N), bool)
    np.put_along_axis(mask, idx.astype(np.int64), False, axis=1)
    xv = X.view(torch.int16).numpy()
    gv = g["X"].view(torch.int16).numpy()
    assert np.array_equal(xv[mask], gv[mask])
    assert (xv[~mask] != gv[~mask]).mean() > 0.9


def test_xhc_with_one_stream_is_plain_residual(lib):
    cfg = Config(N=1, k=1, m=1, C=64, B=2, S=9, dtype="bf16")
    X, out, wd, ow = K.xhc_inputs(cfg, seed=97)
    wd = dict(wd, b_pre=torch.tensor([40.0]), alpha_pre=0.0, alpha_res=0.0, alpha_post=0.0)
    g = K.gpu_xhc(lib, cfg, X, out, wd)
    from oracle import hc_oracle as O
    exp = O.round_state(K.f64(X)[:, 0] + K.f64(out).reshape(-1, cfg.C), "bf16")
    np.testing.assert_array_equal(K.f64(g["X"])[:, 0], exp)
    np.testing.assert_array_equal(K.f64(g["inp"]), K.f64(X)[:, 0])


def test_xhc_all_active_matches_mhc(lib):
    """k = m = N, K_r = 1 and the same residual / post columns: the sparse
    kernels reproduce the dense ones (xHC paper, Appendix C)."""
    N, C, B, S = 4, 256, 2, 30
    cm = Config(N=N, C=C, B=B, S=S, dtype="bf16")
    X, out, wdm, owm = K.mhc_inputs(cm, seed=98)
    Wm = wdm["w_full"]
    w_router = synth.proj_weight(98, 2, 7, N * C, N, "bf16")
    wdx = dict(w_full=torch.cat([w_router, Wm[:, :N]], 1).contiguous(),
               w_act=torch.cat([Wm[:, 2 * N:], Wm[:, N:2 * N]], 1).contiguous(), conv=[],
               b_pre=wdm["b_pre"], b_res=wdm["b_res"], b_post=wdm["b_post"],
               alpha_pre=wdm["alpha_pre"], alpha_res=wdm["alpha_res"], alpha_post=wdm["alpha_post"])
    cx = Config(N=N, k=N, m=N, C=C, B=B, S=S, dtype="bf16")
    gm = K.gpu_mhc(lib, cm, X, out, wdm)
    gx = K.gpu_xhc(lib, cx, X, out, wdx)
    assert np.array_equal(gx["idx"].numpy(), np.tile(np.arange(N, dtype=np.int32), (cx.T, 1)))
    assert K.rel_err(K.f64(gx["inp"]), K.f64(gm["inp"])) <= K.TOL["bf16"]
    assert K.rel_err(K.f64(gx["X"]), K.f64(gm["X"])) <= K.TOL["bf16"]
    assert K.rel_err(gx["h_res"].numpy(), gm["h_res"].numpy()) <= 1e-5


def test_empty_batch_is_a_no_op(lib):
    cfg = Config(N=16, k=4, m=2, C=256, B=0, S=64, n_convs=3, dtype="bf16")
    wd = synth.xhc_layer_weights(1, 0, 16, 4, 256, 4, "bf16")
    from stream_residual_mixing_amd.binding import weights_to_device
    w = weights_to_device(wd)
    X = torch.empty((0, 16, 256), dtype=torch.bfloat16, device="cuda")
    inp = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    ws = lib.workspace(cfg)
    lib.xhc_pre(cfg, w, X, inp, ws)
    lib.xhc_post(cfg, w, X, torch.empty((0, 64, 256), dtype=torch.bfloat16, device="cuda"), ws)
    torch.cuda.synchronize()


def test_results_are_deterministic(lib):
    cfg = Config(N=16, k=4, m=2, C=512, B=2, S=64, n_convs=3, dtype="bf16")
    X, out, wd, ow = K.xhc_inputs(cfg, seed=99)
    a = K.gpu_xhc(lib, cfg, X, out, wd)
    b = K.gpu_xhc(lib, cfg, X, out, wd)
    for key in ("inp", "X", "h_pre", "h_res", "h_post", "p", "z", "idx"):
        assert torch.equal(a[key], b[key]), key
