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
* per-token scale and offset of a state row (token t, attempt a), when asked
  for: [seed, 10, t, a]
* biases away from zero, layer l, bias b (0 pre, 1 res, 2 post): [seed, 12, l, b]

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


def state_rows(seed, tokens, N, C, dtype, attempts=None, affine=False) -> torch.Tensor:
    """State rows [len(tokens), N, C] in the storage dtype (CPU).

    With ``affine``, token t's row is s_t (Z + o_t) with s_t = 10^u,
    u ~ U(-1, 1), and o_t ~ U(-4, 4): rows of very different scales whose
    mean sits up to four standard deviations away from zero."""
    tokens = list(tokens)
    attempts = attempts or {}
    a = np.empty((len(tokens), N * C))
    for r, t in enumerate(tokens):
        at = int(attempts.get(int(t), 0))
        a[r] = _draw((seed, 0, 0, int(t), at), N * C)
        if affine:
            u, o = np.random.default_rng([seed, 10, int(t), at]).uniform(-1.0, 1.0, 2)
            a[r] = (10.0 ** u) * (a[r] + 4.0 * o)
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


def state(seed, T, N, C, dtype, attempts=None, chunk=256, affine=False) -> torch.Tensor:
    """Full state [T, N, C] in the storage dtype (CPU), built row by row."""
    X = torch.empty((T, N, C), dtype=DTYPES[dtype])
    return _fill_rows(X, T, chunk, lambda t0, t1: state_rows(seed, range(t0, t1), N, C, dtype, attempts, affine))


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


# ------------------------------------------------------------------------
# Settings that move the maps away from the uniform ones.  At the workloads'
# own draw (alpha = 0.01, biases 0) every map sits close to its value at
# zero logits (H_res near the uniform matrix), where one Sinkhorn round and
# twenty give nearly the same result.  These draws use unit scales, biases
# ~ N(0, 1) and a residual bias with a strong diagonal, so that the number of
# rounds, their order and the row clamp all change the maps.

def _biases(seed, layer, n_pre, n_res, n_post, k_res, diag):
    b_pre = _draw((seed, 12, layer, 0), n_pre)
    b_res = _draw((seed, 12, layer, 1), n_res) + diag * np.eye(k_res).ravel()
    b_post = _draw((seed, 12, layer, 2), n_post)
    return (torch.from_numpy(b_pre).float(), torch.from_numpy(b_res).float(), torch.from_numpy(b_post).float())


def conv_kernels_lag0(seed, layer, C, kernels=(4, 8, 12), std=0.05):
    """Kernels whose lag-0 tap is 1 and whose other taps are small
    (~ N(0, std)): each convolution branch is then nearly parallel to the
    sublayer output itself, which is where Gram-Schmidt has the most to do."""
    ks = []
    for j, kap in enumerate(kernels):
        w = _draw((seed, 4 + j, layer), (kap, C), std)
        w[0] += 1.0
        ks.append(_round(w, "f32"))
    return ks


def conv_kernels_zero(C, kernels=(4, 8, 12)):
    """All-zero kernels (the temporal branches switched off)."""
    return [torch.zeros((kap, C), dtype=torch.float32) for kap in kernels]


def xhc_stress_weights(seed, layer, N, k, C, K_r, dtype, alpha_res=1.0, conv="draw", diag=3.0,
                       kernels=(4, 8, 12)):
    """An xHC sublayer's weights with unit pre/post scales, residual scale
    ``alpha_res``, biases ~ N(0, 1) (the residual one plus ``diag`` on its
    diagonal) and conv kernels drawn as usual ("draw"), all zero ("zero") or
    lag-0 dominated ("lag0")."""
    wd = xhc_layer_weights(seed, layer, N, k, C, K_r, dtype, kernels)
    b_pre, b_res, b_post = _biases(seed, layer, N, k * k, k * K_r, k, diag)
    wd.update(b_pre=b_pre, b_res=b_res, b_post=b_post, alpha_pre=1.0, alpha_res=float(alpha_res), alpha_post=1.0)
    if K_r > 1 and conv == "zero":
        wd["conv"] = conv_kernels_zero(C, kernels)
    elif K_r > 1 and conv == "lag0":
        wd["conv"] = conv_kernels_lag0(seed, layer, C, kernels)
    return wd


def mhc_stress_weights(seed, layer, N, C, dtype, alpha_res=1.0, diag=3.0):
    """An mHC sublayer's weights with unit pre/post scales, residual scale
    ``alpha_res`` and biases ~ N(0, 1) (the residual one plus ``diag`` on its
    diagonal)."""
    wd = mhc_layer_weights(seed, layer, N, C, dtype)
    b_pre, b_res, b_post = _biases(seed, layer, N, N * N, N, N, diag)
    wd.update(b_pre=b_pre, b_res=b_res, b_post=b_post, alpha_pre=1.0, alpha_res=float(alpha_res), alpha_post=1.0)
    return wd
