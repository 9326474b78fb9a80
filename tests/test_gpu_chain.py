"""GPU parity of the chained xHC calls (xhc_route, xhc_pre_chained,
xhc_post_chained) against the float64 oracle run sublayer after sublayer.

In the chained calls, the routing of sublayer l+1 is accumulated while
sublayer l runs: the rows sublayer l does not write are contracted in its
pre-application, the k rewritten rows after its post-application.  The
oracle computes every sublayer's routing from the whole state it receives,
so these tests check that the split contraction gives the same routing,
maps, sublayer inputs and states.  The first layer sees identical inputs on
both sides; later layers carry each side's own rounded state, and their
state and sublayer input get, per element, the rounding allowance that
cases.carried_allowances derives from oracle values.  Every layer's maps and
router logits are compared per element at the dtype's bar.  Ragged tails,
sequence starts inside a tile and every built (N, k) shape are covered; the
maps away from uniform (unit scales, biases, 1 or 3 Sinkhorn rounds, state
rows of different scales and offsets) in test_gpu_maps.py.
"""
import numpy as np
import pytest

import cases as K

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def run_chain(lib, cfgs, seed, margin, weights=None, affine=False):
    X, outs, wds, ref = K.xhc_chain_inputs(cfgs, seed, margin, weights=weights, affine=affine)
    got = K.gpu_xhc_chain(lib, cfgs, X, outs, wds)
    dt = cfgs[0].dtype
    allow = K.carried_allowances(ref, dt, [K.oracle_weights(wd) for wd in wds])
    for l, (g, o) in enumerate(zip(got, ref)):
        errs = K.compare_xhc(g, o, K.TOL[dt]) if l == 0 else K.compare_carried(g, o, l, dt, allow[l])
        if l == 0:
            z = K.logit_err(g["z"].numpy().astype(np.float64), o["z"])
            assert z <= K.TOL[dt], f"router logits {z}"
            errs["z"] = z
        _print(f"layer {l}:", {k: f"{v:.1e}" for k, v in errs.items()})


def test_chain_bf16_n16_k4_attention_mlp_alternating(lib):
    """4 sublayers A M A M, N=16, k=4, m=2, C=256, 2 x 37 tokens (ragged tile,
    a sequence start inside a tile), bf16."""
    run_chain(lib, K.chain_configs(16, 4, 2, 256, 2, 37, "AMAM"), seed=21, margin=K.CHAIN_MARGIN)


def test_chain_f32_n16_k4(lib):
    """3 sublayers M A M, N=16, k=4, m=2, C=128, 1 x 40 tokens, fp32 state."""
    run_chain(lib, K.chain_configs(16, 4, 2, 128, 1, 40, "MAM", dtype="f32"), seed=22, margin=K.MARGIN)


@pytest.mark.parametrize("N,k,m", [(16, 2, 1), (8, 4, 2), (4, 4, 2), (1, 1, 1)])
def test_chain_other_shapes(lib, N, k, m):
    """2 sublayers A M for every other built (N, k), C=64, 2 x 19 tokens, bf16."""
    run_chain(lib, K.chain_configs(N, k, m, 64, 2, 19, "AM"), seed=30 + N + k, margin=K.CHAIN_MARGIN)


def test_chain_single_sublayer_without_next(lib):
    """A chain of one: xhc_route, then the chained calls with no next sublayer."""
    run_chain(lib, K.chain_configs(16, 4, 2, 256, 1, 50, "M"), seed=23, margin=K.MARGIN)


def test_chain_many_tiles_c4096(lib):
    """3 sublayers A M A at C=4096 (16 channel slices), 1 x 160 tokens, bf16."""
    run_chain(lib, K.chain_configs(16, 4, 2, 4096, 1, 160, "AMA"), seed=24, margin=K.CHAIN_MARGIN)


# The persistent kernels run one workgroup per compute unit: a team of one
# workgroup per 128-channel slice (64 in fp32) walks steps of 32 tokens.  With
# wide C there are few teams, so each walks several steps, through both of its
# register sets and both routing buffers, up to a ragged last step.

@pytest.mark.timeout(300)
def test_chain_one_team_many_steps_c32768(lib):
    """2 sublayers A M, N=16, k=4, m=2, C=32768 (256 slices: a single team
    walks all 4 steps of 1 x 100 tokens), bf16."""
    run_chain(lib, K.chain_configs(16, 4, 2, 32768, 1, 100, "AM"), seed=25, margin=K.CHAIN_MARGIN)


@pytest.mark.timeout(300)
def test_chain_several_steps_per_team_c8192(lib):
    """2 sublayers M A, N=16, k=4, m=2, C=8192 (4 teams, 10 steps of 2 x 150
    tokens, a sequence start inside a step), bf16."""
    run_chain(lib, K.chain_configs(16, 4, 2, 8192, 2, 150, "MA"), seed=26, margin=K.CHAIN_MARGIN)


def test_chain_f32_several_steps_per_team_c4096(lib):
    """3 sublayers M A M, N=16, k=4, m=2, C=4096 in fp32 (64 slices: 4 teams,
    10 steps of 1 x 300 tokens)."""
    run_chain(lib, K.chain_configs(16, 4, 2, 4096, 1, 300, "MAM", dtype="f32"), seed=27, margin=K.MARGIN)


@pytest.mark.parametrize("kinds", ["AM", "MA"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chained_write_is_the_sublayer_write(lib, kinds, dtype):
    """With a next sublayer, the chained post call writes the state in the
    same pass that contracts the new rows for the next routing (after an
    MLP-type sublayer, with the write basis formed there from out and its
    causal convolutions).  Its write must be the per-sublayer write bit for
    bit: same maps (left by the chained pre call), same state, same output.
    N=16, k=4, m=2, C=256, 2 x 16401 tokens, so that xhc_post takes its
    tiled write and the chained pass its ragged last step; the sequence
    start of the second batch item falls inside a tile."""
    import torch
    from stream_residual_mixing_amd import synth
    from stream_residual_mixing_amd.binding import weights_to_device
    cfgs = K.chain_configs(16, 4, 2, 256, 2, 16401, kinds, dtype=dtype)
    c0, c1 = cfgs
    w = [weights_to_device(synth.xhc_layer_weights(41, l, 16, 4, 256, c.K_r, dtype)) for l, c in enumerate(cfgs)]
    X = synth.state(41, c0.T, 16, 256, dtype).to("cuda")
    out = synth.sublayer_out(41, 0, c0.B, c0.S, 256, dtype).reshape(c0.T, 256).to("cuda")
    inp = torch.empty((c0.T, 256), dtype=c0.torch_dtype, device="cuda")
    ws0, ws1 = lib.workspace(c0), lib.workspace(c1)
    lib.xhc_route(c0, w[0], X, ws0)
    lib.xhc_pre_chained(c0, w[0], c1, w[1], X, inp, ws0, ws1)
    Xa, Xb = X.clone(), X.clone()
    lib.xhc_post(c0, w[0], Xa, out, ws0)
    lib.xhc_post_chained(c0, w[0], c1, w[1], Xb, out, ws0, ws1)
    torch.cuda.synchronize()
    assert not torch.equal(Xa, X), "the write changed nothing"
    assert torch.equal(Xa, Xb), f"{int((Xa != Xb).sum())} elements differ"
