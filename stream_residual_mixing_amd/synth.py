"""Seeded synthetic inputs for the residual-stream layer.

Shared by the tests and the benchmark; holds none of the method's
arithmetic.  Every tensor is drawn as float64 standard normals from
``numpy.random.default_rng(key)`` scaled by its standard deviation, then
rounded once to its storage dtype by PyTorch on the CPU.  Keys:

* state X, token t, attempt a:       [seed, 0, 0, t, a]   (one row per token,
  so any token can be regenerated alone; a > 0 only when a test redraws a
  token whose routing margin is too small)
* sublayer output, layer l, token t: [seed, 1, l, t]
* full-state projection, layer l:     [seed, 2, l]
* active-state projection, layer l:   [seed, 3, l]
* conv kernel j, layer l:             [seed, 4 + j, l]
* xHC-Flash attention post-map, block b: [seed, 7, b] (a block's other
  weights use the keys above with l = b; its attention and MLP outputs are
  layers 2b and 2b + 1)
* xHC-Flash-4sub group g: full-state projection [seed, 2, g], post-maps of
  sublayers 1-3 [seed, 8, 3g + q], final MLP maps [seed, 3, g], the two MLPs'
  kernels [seed, 4 + j, 2g + i]; its four outputs are layers 4g .. 4g + 3

Distributions (the workloads' own): X, out ~ N(0, 1); projection weights
~ N(0, 0.02); conv kernel of size kappa ~ N(0, 1/kappa) (second argument
read as the standard deviation).  Scales alpha = 0.01, biases 0.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}
PROJ_STD = 0.02
ALPHA = 0.01


def _draw(key, shape, std=1.0):
    return np.random.default_rng(list(key)).standard_normal(shape) * std


def _round(a64: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a64)).to(DTYPES[dtype])


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a bf16 / f32 tensor's values."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def state_rows(seed, tokens, N, C, dtype, attempts=None) -> torch.Tensor:
    """State rows [len(tokens), N, C] in the storage dtype (CPU)."""
    tokens = list(tokens)
    attempts = attempts or {}
    a = np.empty((len(tokens), N * C))
    for r, t in enumerate(tokens):
        a[r] = _draw((seed, 0, 0, int(t), int(attempts.get(int(t), 0))), N * C)
    return _round(a, dtype).reshape(len(tokens), N, C)


def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def _fill_rows(dst, T, chunk, make):
    """dst[t0:t1] = make(t0, t1) over row chunks, in a thread pool (each row
    has its own generator, so the values do not depend on the schedule)."""
    def job(t0):
        t1 = min(T, t0 + chunk)
        dst[t0:t1] = make(t0, t1)
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, range(0, T, chunk)))
    return dst


def state(seed, T, N, C, dtype, attempts=None, chunk=256) -> torch.Tensor:
    """Full state [T, N, C] in the storage dtype (CPU), built row by row."""
    X = torch.empty((T, N, C), dtype=DTYPES[dtype])
    return _fill_rows(X, T, chunk, lambda t0, t1: state_rows(seed, range(t0, t1), N, C, dtype, attempts))


def out_rows(seed, layer, tokens, C, dtype) -> torch.Tensor:
    """Sublayer-output rows [len(tokens), C] for flat token ids t = b*S + s."""
    tokens = list(tokens)
    a = np.empty((len(tokens), C))
    for r, t in enumerate(tokens):
        a[r] = _draw((seed, 1, layer, int(t)), C)
    return _round(a, dtype)


def sublayer_out(seed, layer, B, S, C, dtype, chunk=1024) -> torch.Tensor:
    """Sublayer output [B, S, C] in the storage dtype (CPU)."""
    T = B * S
    o = torch.empty((T, C), dtype=DTYPES[dtype])
    _fill_rows(o, T, chunk, lambda t0, t1: out_rows(seed, layer, range(t0, t1), C, dtype))
    return o.reshape(B, S, C)


def proj_weight(seed, tensor_id, layer, rows, cols, dtype, std=PROJ_STD) -> torch.Tensor:
    return _round(_draw((seed, tensor_id, layer), (rows, cols), std), dtype)


def conv_kernels(seed, layer, C, kernels=(4, 8, 12)):
    """List of fp32 kernels [kappa_j, C], kernel j ~ N(0, 1/kappa_j)."""
    return [_round(_draw((seed, 4 + j, layer), (kap, C), 1.0 / kap), "f32")
            for j, kap in enumerate(kernels)]


def xhc_layer_weights(seed, layer, N, k, C, K_r, dtype, kernels=(4, 8, 12)):
    """Weights of one xHC sublayer: dict of CPU tensors plus scalars."""
    n_res, n_post = k * k, k * K_r
    return dict(
        w_full=proj_weight(seed, 2, layer, N * C, 2 * N, dtype),
        w_act=proj_weight(seed, 3, layer, k * C, n_res + n_post, dtype),
        conv=conv_kernels(seed, layer, C, kernels) if K_r > 1 else [],
        b_pre=torch.zeros(N), b_res=torch.zeros(n_res), b_post=torch.zeros(n_post),
        alpha_pre=ALPHA, alpha_res=ALPHA, alpha_post=ALPHA,
    )


def mhc_layer_weights(seed, layer, N, C, dtype):
    """Weights of one mHC sublayer (columns pre | post | res)."""
    return dict(
        w_full=proj_weight(seed, 2, layer, N * C, 2 * N + N * N, dtype),
        b_pre=torch.zeros(N), b_post=torch.zeros(N), b_res=torch.zeros(N * N),
        alpha_pre=ALPHA, alpha_res=ALPHA, alpha_post=ALPHA,
    )


def xhcf_block_weights(seed, block, N, k, C, K_r, dtype, kernels=(4, 8, 12)):
    """Weights of one xHC-Flash block: full-state projection [N*C, 3N]
    (router | attention pre-map | MLP pre-map), attention post-map [k*C, k],
    MLP active maps [k*C, k*k + k*K_r], conv kernels; biases 0, scales alpha."""
    return dict(
        w_full=proj_weight(seed, 2, block, N * C, 3 * N, dtype),
        w_post_attn=proj_weight(seed, 7, block, k * C, k, dtype),
        w_act_mlp=proj_weight(seed, 3, block, k * C, k * k + k * K_r, dtype),
        conv=conv_kernels(seed, block, C, kernels) if K_r > 1 else [],
        b_pre_attn=torch.zeros(N), b_pre_mlp=torch.zeros(N), b_post_attn=torch.zeros(k),
        b_res=torch.zeros(k * k), b_post_mlp=torch.zeros(k * K_r),
        alpha_pre_attn=ALPHA, alpha_pre_mlp=ALPHA, alpha_post_attn=ALPHA, alpha_res=ALPHA, alpha_post_mlp=ALPHA,
    )


def xhcf4_group_weights(seed, group, N, k, C, K_r, dtype, kernels=(4, 8, 12)):
    """Weights of one xHC-Flash-4sub group: full-state projection [N*C, 5N]
    (router, four pre-maps), post-maps of sublayers 1-3, final MLP maps
    [k*C, k*k + k*K_r], two MLP kernel sets; biases 0, scales alpha."""
    ncq = (k, k * K_r, k)
    return dict(
        w_full=proj_weight(seed, 2, group, N * C, 5 * N, dtype),
        w_post=[proj_weight(seed, 8, 3 * group + q, k * C, ncq[q], dtype) for q in range(3)],
        w_act_last=proj_weight(seed, 3, group, k * C, k * k + k * K_r, dtype),
        conv=[conv_kernels(seed, 2 * group + i, C, kernels) if K_r > 1 else [] for i in range(2)],
        b_pre=[torch.zeros(N) for _ in range(4)], b_post=[torch.zeros(k), torch.zeros(k * K_r), torch.zeros(k),
                                                          torch.zeros(k * K_r)],
        b_res=torch.zeros(k * k), alpha_pre=(ALPHA,) * 4, alpha_post=(ALPHA,) * 4, alpha_res=ALPHA,
    )
