"""xhc_post_noalloc against xhc_post, through the C ABI.

The no-allocation write runs the same kernels as xhc_post, with the Gram
partials in the library's own per-device array instead of the workspace, so
the two must agree bit for bit.  Two calls in a row, the second smaller than
the first, check that the array's earlier contents do not leak into a later
call; a third asks for more scratch than the array holds and must be refused
before anything is launched (the state stays as it was).
"""
import ctypes

import pytest
import torch

import cases as K
from stream_residual_mixing_amd import binding
from stream_residual_mixing_amd.binding import Config, weights_to_device

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def run_pair(lib, cfg, seed):
    """xhc_pre once, then xhc_post and xhc_post_noalloc on two copies of the
    state; returns both results and the oracle's comparison of the first."""
    X, out, wd, ow = K.xhc_inputs(cfg, seed)
    w = weights_to_device(wd)
    Xa, Xb = X.to("cuda"), X.to("cuda")
    outd = out.to("cuda")
    inp = torch.empty((cfg.T, cfg.C), dtype=cfg.torch_dtype, device="cuda")
    ws = lib.workspace(cfg)
    lib.xhc_pre(cfg, w, Xa, inp, ws)
    maps = ws.clone()
    lib.xhc_post(cfg, w, Xa, outd, ws)
    lib.xhc_post_noalloc(cfg, w, Xb, outd, maps)
    torch.cuda.synchronize()
    o = K.oracle_xhc(cfg, K.f64(X), K.f64(out), ow)
    g = dict(inp=inp.cpu(), X=Xb.cpu(), **{k: v.cpu() for k, v in lib.ws_arrays(cfg, maps).items()})
    g.pop("status")
    return Xa.cpu(), Xb.cpu(), K.compare_xhc(g, o, K.TOL[cfg.dtype])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_xhc_post_two_calls(lib, dtype):
    big = Config(N=16, k=4, m=2, C=2048, B=2, S=300, n_convs=3, dtype=dtype)
    small = Config(N=16, k=4, m=2, C=512, B=1, S=77, n_convs=3, dtype=dtype)
    for cfg, seed in ((big, 601), (small, 602)):
        _print(f"xhc_post_noalloc {dtype}: C={cfg.C} T={cfg.T}")
        Xa, Xb, errs = run_pair(lib, cfg, seed)
        assert torch.equal(Xa.view(torch.int16 if dtype == "bf16" else torch.int32),
                           Xb.view(torch.int16 if dtype == "bf16" else torch.int32)), "differs from xhc_post"
        _print("   bit-identical to xhc_post; against the oracle:", {k: f"{v:.1e}" for k, v in errs.items()})


def test_noalloc_attention_type(lib):
    cfg = Config(N=16, k=4, m=2, C=1024, B=2, S=600, dtype="bf16")
    Xa, Xb, errs = run_pair(lib, cfg, 603)
    assert torch.equal(Xa.view(torch.int16), Xb.view(torch.int16))


def test_noalloc_refuses_more_than_its_scratch(lib):
    cfg = Config(N=16, k=4, m=2, C=4096, B=1, S=30000, n_convs=3, dtype="bf16")
    need = 80 * ((cfg.C + 1023) // 1024) * cfg.T
    assert need > 8 << 20
    # refused on the host before any launch: small stand-in buffers are never touched
    cfg_s = Config(N=16, k=4, m=2, C=4096, B=1, S=16, n_convs=3, dtype="bf16")
    _, _, wd, _ = K.xhc_inputs(cfg_s, 604)
    w = weights_to_device(wd)
    c, cw = cfg.c(), w.c()
    dummy = torch.zeros(256, dtype=torch.uint8, device="cuda")
    st = lib.dll.xhc_post_noalloc(ctypes.byref(c), ctypes.byref(cw), dummy.data_ptr(), dummy.data_ptr() + 16,
                                  dummy.data_ptr() + 32, None)
    torch.cuda.synchronize()
    assert st == binding.XHC_ERR_INVALID_ARG, st
    assert "scratch" in lib.last_error()
    assert int(dummy.abs().sum()) == 0
