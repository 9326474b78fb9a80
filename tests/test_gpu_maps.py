"""GPU parity with maps far from uniform.

At the workloads' own draw (scales alpha = 0.01, biases 0) every map sits
next to its value at zero logits: H_res is nearly the uniform matrix, one
Sinkhorn round gives almost the same map as twenty, and the row clamp never
acts beyond rounding.  These cases draw unit pre/post scales, residual scales
of 1 and 4, biases ~ N(0, 1) with a strong diagonal on the residual bias,
and run 0, 1, 3 and 20 Sinkhorn rounds; test_oracle_stress.py shows on the
CPU that at these draws every pair of round counts, the order of the
normalisations and the clamp each move the oracle's H_res by far more than
the fp32 bar, so a wrong count, order or clamp fails here.  Further cases:
all-zero conv kernels (the write reduces to the sublayer output alone),
lag-0 dominated kernels (each branch nearly parallel to the output, where
Gram-Schmidt removes most of it), and state rows of very different scales
with offsets of up to four standard deviations (the mean and variance
corrections of the router's LayerNorm).  Calls go through the C ABI: the
per-sublayer calls, the chained calls over several layers, and mHC at N = 4
and N = 16.  Bars as everywhere: exact active indices, 1e-4 in fp32 and 2e-2
in bf16 (floored relative error per element).

Explainer "xHC: sixteen residual streams, four written at a time": sections
"mHC: keep the mixing doubly stochastic" (twenty alternating rounds),
"Which constraint survives" (the row clamp), "What xHC changes" (kernels
that start at zero) and "Stability, read closely" (branches close to the
main one); xHC paper, "Mapping generation" (the normalisation statistics).
"""
import functools

import numpy as np
import pytest

import cases as K
from stream_residual_mixing_amd import synth
from stream_residual_mixing_amd.binding import Config

pytestmark = pytest.mark.gpu

# a state row scaled by up to 10 and offset by up to 4 of its own standard
# deviations moves the router logits' float32 rounding by more than on the
# unit draw; such tokens keep a larger routing margin
AFFINE_MARGIN = 1e-3


def _print(*a):
    print(*a, flush=True)


# seeds of the draws below (test_oracle_stress.py checks each draw on the CPU)
def seed_rounds(iters, alpha_res, mlp):
    return 200 + iters + int(alpha_res) + 10 * mlp


def seed_affine(mlp):
    return 240 + mlp


def seed_shape(N, k, m):
    return 250 + N + k + m


def seed_mhc(N, iters, alpha_res):
    return 300 + N + iters + int(alpha_res)


def seed_mhc_affine(N):
    return 330 + N


def xw(alpha_res, conv="draw"):
    return functools.partial(synth.xhc_stress_weights, alpha_res=alpha_res, conv=conv)


def mw(alpha_res):
    return functools.partial(synth.mhc_stress_weights, alpha_res=alpha_res)


def run_xhc(lib, cfg, seed, weights, affine=False):
    margin = AFFINE_MARGIN if affine else K.MARGIN
    X, out, wd, ow = K.xhc_inputs(cfg, seed, weights=weights, affine=affine, margin=margin)
    g = K.gpu_xhc(lib, cfg, X, out, wd)
    o = K.oracle_xhc(cfg, K.f64(X), K.f64(out), ow)
    return K.compare_xhc(g, o, K.TOL[cfg.dtype])


# ------------------------------------------------------------ per sublayer

@pytest.mark.parametrize("iters", [0, 1, 3, 20])
@pytest.mark.parametrize("alpha_res", [1.0, 4.0])
@pytest.mark.parametrize("mlp", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_xhc_maps_sinkhorn_rounds(lib, iters, alpha_res, mlp, dtype):
    """N=16, k=4, m=2, C=256, 2 x 37 tokens; unit scales, biases, 0/1/3/20 rounds."""
    cfg = Config(N=16, k=4, m=2, C=256, B=2, S=37, n_convs=3 if mlp else 0, iters=iters, dtype=dtype)
    errs = run_xhc(lib, cfg, seed_rounds(iters, alpha_res, mlp), xw(alpha_res))
    _print("xhc maps", iters, alpha_res, mlp, dtype, errs)


@pytest.mark.parametrize("conv", ["zero", "lag0"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_xhc_maps_conv_kernels(lib, conv, dtype):
    """MLP-type with all-zero kernels (only the output is written) and with
    lag-0 dominated kernels (cos(g_j, out) >= 0.95, Gram-Schmidt removes most
    of each branch); unit scales and biases."""
    cfg = Config(N=16, k=4, m=2, C=256, B=2, S=37, n_convs=3, dtype=dtype)
    errs = run_xhc(lib, cfg, 230 + (conv == "lag0"), xw(1.0, conv))
    _print("xhc conv", conv, dtype, errs)


@pytest.mark.parametrize("mlp", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_xhc_maps_scaled_offset_state(lib, mlp, dtype):
    """State rows scaled by 10^U(-1, 1) and offset by U(-4, 4) standard
    deviations; residual scale 4, 20 rounds."""
    cfg = Config(N=16, k=4, m=2, C=256, B=2, S=37, n_convs=3 if mlp else 0, dtype=dtype)
    errs = run_xhc(lib, cfg, seed_affine(mlp), xw(4.0), affine=True)
    _print("xhc affine", mlp, dtype, errs)


@pytest.mark.parametrize("N,k,m", [(16, 2, 1), (8, 4, 2), (4, 4, 4), (16, 4, 0)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_xhc_maps_other_shapes(lib, N, k, m, dtype):
    """Every other built (N, k), MLP-type, 3 rounds, residual scale 4."""
    cfg = Config(N=N, k=k, m=m, C=192, B=2, S=29, n_convs=3, iters=3, dtype=dtype)
    errs = run_xhc(lib, cfg, seed_shape(N, k, m), xw(4.0))
    _print("xhc maps shape", N, k, m, dtype, errs)


def test_xhc_maps_c4096(lib):
    """The benchmark's width: C=4096, 1 x 48 tokens, bf16, MLP-type, residual
    scale 4, 20 rounds, scaled and offset state rows."""
    cfg = Config(N=16, k=4, m=2, C=4096, B=1, S=48, n_convs=3, dtype="bf16")
    errs = run_xhc(lib, cfg, 260, xw(4.0), affine=True)
    _print("xhc maps C=4096", errs)


# ------------------------------------------------------------------ chains

def run_chain(lib, cfgs, seed, weights, affine):
    from test_gpu_chain import run_chain as rc
    margin = K.CHAIN_MARGIN if cfgs[0].dtype == "bf16" else (AFFINE_MARGIN if affine else K.MARGIN)
    rc(lib, cfgs, seed, margin, weights=weights, affine=affine)


@pytest.mark.parametrize("iters", [1, 20])
@pytest.mark.parametrize("alpha_res", [1.0, 4.0])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_maps(lib, iters, alpha_res, dtype):
    """4 chained sublayers A M A M, N=16, k=4, m=2, C=256, 2 x 37 tokens,
    unit scales, biases, 1 or 20 rounds, scaled and offset state rows."""
    cfgs = [Config(**{**c.__dict__, "iters": iters}) for c in K.chain_configs(16, 4, 2, 256, 2, 37, "AMAM", dtype=dtype)]
    run_chain(lib, cfgs, 270 + iters + int(alpha_res), xw(alpha_res), affine=True)


def test_chain_maps_c4096(lib):
    """3 chained sublayers M A M at C=4096 (persistent kernels, 16 slices),
    1 x 96 tokens, bf16, residual scale 1, 3 rounds, lag-0 dominated kernels.
    At this width the residual logits already spread with a standard
    deviation of about 0.02 sqrt(4 C) = 2.6 at scale 1 (as at scale 4 with
    C = 256); at scale 4 they would spread by 10, where exp moves the maps by
    percents for a one-unit difference of the carried state."""
    cfgs = [Config(**{**c.__dict__, "iters": 3}) for c in K.chain_configs(16, 4, 2, 4096, 1, 96, "MAM")]
    run_chain(lib, cfgs, 280, xw(1.0, "lag0"), affine=False)


# -------------------------------------------------------------------- mHC

@pytest.mark.parametrize("iters", [0, 1, 3, 20])
@pytest.mark.parametrize("alpha_res", [1.0, 4.0])
@pytest.mark.parametrize("N", [4, 16])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mhc_maps(lib, iters, alpha_res, N, dtype):
    """mHC, C=256, 2 x 37 tokens; unit scales, biases, 0/1/3/20 rounds."""
    cfg = Config(N=N, C=256, B=2, S=37, iters=iters, dtype=dtype)
    X, out, wd, ow = K.mhc_inputs(cfg, seed_mhc(N, iters, alpha_res), weights=mw(alpha_res))
    g = K.gpu_mhc(lib, cfg, X, out, wd)
    o = K.oracle_mhc(cfg, K.f64(X), K.f64(out), ow)
    _print("mhc maps", N, iters, alpha_res, dtype, K.compare_mhc(g, o, K.TOL[dtype]))


@pytest.mark.parametrize("N", [4, 16])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mhc_maps_scaled_offset_state(lib, N, dtype):
    """mHC with scaled and offset state rows, residual scale 4, 20 rounds."""
    cfg = Config(N=N, C=256, B=2, S=37, dtype=dtype)
    X, out, wd, ow = K.mhc_inputs(cfg, seed_mhc_affine(N), weights=mw(4.0), affine=True)
    g = K.gpu_mhc(lib, cfg, X, out, wd)
    o = K.oracle_mhc(cfg, K.f64(X), K.f64(out), ow)
    _print("mhc affine", N, dtype, K.compare_mhc(g, o, K.TOL[dtype]))


def test_mhc_maps_c4096_n16(lib):
    """mHC at N=16, C=4096 (the wide projection), 1 x 80 tokens, bf16,
    residual scale 4, 3 rounds."""
    cfg = Config(N=16, C=4096, B=1, S=80, iters=3, dtype="bf16")
    X, out, wd, ow = K.mhc_inputs(cfg, 340, weights=mw(4.0))
    g = K.gpu_mhc(lib, cfg, X, out, wd)
    o = K.oracle_mhc(cfg, K.f64(X), K.f64(out), ow)
    _print("mhc maps C=4096", K.compare_mhc(g, o, K.TOL["bf16"]))
