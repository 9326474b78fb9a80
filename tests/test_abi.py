"""CPU checks of the C ABI: the library loads and exports every function
include/xhc.h declares; workspace sizing and layout; argument checks that
reject bad calls before anything is launched.  No compute call is made.
"""
import ctypes
import os
import re

import pytest
import torch

from stream_residual_mixing_amd import binding
from stream_residual_mixing_amd.binding import Config, XhcConfig, XhcWeights

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "xhc.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from stream_residual_mixing_amd import build
        build.build()
    return binding.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return [n for n in names if n not in ("defined",)]


def test_library_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(binding.EXPORTS), names
    for n in names:
        assert hasattr(lib.dll, n), n


def test_struct_layouts_match_the_header(tmp_path):
    """The ctypes mirrors have the sizes and field offsets a C compiler
    gives the header's structs."""
    import subprocess
    structs = {"xhc_config": XhcConfig, "xhc_weights": XhcWeights, "xhc_ws_layout": binding.XhcWsLayout,
               "xhcf_weights": binding.XhcfWeights, "xhcf_ws_layout": binding.XhcfWsLayout,
               "xhcf4_weights": binding.Xhcf4Weights, "xhcf4_ws_layout": binding.Xhcf4WsLayout, "xhc_grads": binding.XhcGrads, "xhc_bwd_ws_layout": binding.XhcBwdWsLayout}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "xhc.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{cname}.{f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0; }")
    src = tmp_path / "probe.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines())
    for cname, cls in structs.items():
        assert int(got[cname]) == ctypes.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert int(got[f"{cname}.{f}"]) == getattr(cls, f).offset, (cname, f)


def _cfg(**kw):
    base = dict(N=16, k=4, m=2, C=4096, B=2, S=8192, n_convs=3, dtype="bf16")
    base.update(kw)
    return Config(**base)


def test_workspace_layout_is_aligned_and_sized(lib):
    for mhc, cfg in ((False, _cfg()), (False, _cfg(n_convs=0)), (True, _cfg(k=0, m=0, n_convs=0)),
                     (True, _cfg(N=4, C=256, B=1, S=64, dtype="f32"))):
        L = lib.layout(cfg, mhc)
        T, N = cfg.T, cfg.N
        offs = [getattr(L, f) for f in ("idx", "p", "h_pre", "h_res", "h_post", "z_router")]
        used = [o for o in offs if o != binding.SIZE_MAX]
        assert all(o % 256 == 0 for o in used)
        assert L.total == lib.workspace_bytes(cfg, mhc) > 0
        if mhc:
            assert L.h_res + T * N * N * 4 <= L.total
        else:
            assert L.z_router + T * N * 4 <= L.total
            assert L.h_post - L.h_res >= T * cfg.k * cfg.k * 4


def test_empty_batch_needs_no_workspace_and_launches_nothing(lib):
    cfg = _cfg(B=0)
    assert lib.workspace_bytes(cfg) == 0
    c, w = cfg.c(), XhcWeights()
    w.w_full = w.w_act = w.b_pre = w.b_res = w.b_post = w.conv_w = 0x10000
    for fn in (lib.dll.xhc_pre, lib.dll.xhc_post):
        assert fn(ctypes.byref(c), ctypes.byref(w), None, None, None, None) == binding.XHC_OK


BAD = [
    (dict(k=17), binding.XHC_ERR_INVALID_ARG, "k_active"),
    (dict(k=5), binding.XHC_ERR_UNSUPPORTED, "not built"),
    (dict(m=5), binding.XHC_ERR_INVALID_ARG, "m_fixed"),
    (dict(C=4100), binding.XHC_ERR_INVALID_ARG, "multiple of 32"),
    (dict(n_convs=2), binding.XHC_ERR_INVALID_ARG, "n_convs"),
    (dict(kernels=(3, 8, 12)), binding.XHC_ERR_UNSUPPORTED, "kernel sizes"),
    (dict(N=17), binding.XHC_ERR_INVALID_ARG, "n_streams"),
    (dict(iters=-1), binding.XHC_ERR_INVALID_ARG, "sinkhorn_iters"),
    (dict(eps_norm=float("nan")), binding.XHC_ERR_INVALID_ARG, "eps_norm"),
    (dict(B=-1), binding.XHC_ERR_INVALID_ARG, "batch"),
]


@pytest.mark.skipif(torch.cuda.is_available(), reason="fake device pointers: run on a host without a GPU only")
@pytest.mark.parametrize("kw,status,msg", BAD)
def test_bad_configs_are_rejected_before_launch(lib, kw, status, msg):
    cfg = _cfg(**kw)
    c, w = cfg.c(), XhcWeights()
    w.w_full = w.w_act = w.b_pre = w.b_res = w.b_post = w.conv_w = 0x10000
    rc = lib.dll.xhc_pre(ctypes.byref(c), ctypes.byref(w), 0x20000, 0x30000, 0x40000, None)
    assert rc == status
    assert msg in lib.last_error()
    assert lib.workspace_bytes(cfg) == 0


@pytest.mark.skipif(torch.cuda.is_available(), reason="fake device pointers: run on a host without a GPU only")
def test_bad_pointers_are_rejected_before_launch(lib):
    cfg = _cfg(B=1, S=16)
    c, w = cfg.c(), XhcWeights()
    w.w_full = w.w_act = w.b_pre = w.b_res = w.b_post = w.conv_w = 0x10000
    pre = lib.dll.xhc_pre
    assert pre(ctypes.byref(c), ctypes.byref(w), 0x20001, 0x30000, 0x40000, None) == binding.XHC_ERR_INVALID_ARG
    assert "aligned" in lib.last_error()
    assert pre(ctypes.byref(c), ctypes.byref(w), 0x20000, 0x20000, 0x40000, None) == binding.XHC_ERR_INVALID_ARG
    assert "alias" in lib.last_error()
    assert pre(ctypes.byref(c), ctypes.byref(w), None, 0x30000, 0x40000, None) == binding.XHC_ERR_INVALID_ARG
    w2 = XhcWeights()
    w2.w_full = 0x10000
    assert pre(ctypes.byref(c), ctypes.byref(w2), 0x20000, 0x30000, 0x40000, None) == binding.XHC_ERR_INVALID_ARG
    assert pre(None, ctypes.byref(w), 0x20000, 0x30000, 0x40000, None) == binding.XHC_ERR_INVALID_ARG
    # post of an MLP-type layer needs the conv kernels
    w.conv_w = 0
    rc = lib.dll.xhc_post(ctypes.byref(c), ctypes.byref(w), 0x20000, 0x30000, 0x40000, None)
    assert rc == binding.XHC_ERR_INVALID_ARG and "conv_w" in lib.last_error()
    # mHC shapes
    cm = _cfg(N=3, k=0, m=0, n_convs=0).c()
    assert lib.dll.mhc_pre(ctypes.byref(cm), ctypes.byref(w), 0x20000, 0x30000, 0x40000, None) == \
        binding.XHC_ERR_UNSUPPORTED


def test_binding_refuses_host_tensors(lib):
    cfg = _cfg(C=64, B=1, S=4)
    wd = binding.Weights(w_full=torch.zeros(16 * 64, 32, dtype=torch.bfloat16), b_pre=torch.zeros(16),
                         b_res=torch.zeros(16), b_post=torch.zeros(16), alpha_pre=0.01, alpha_res=0.01,
                         alpha_post=0.01, w_act=torch.zeros(4 * 64, 32, dtype=torch.bfloat16))
    X = torch.zeros(4, 16, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        lib.xhc_pre(cfg, wd, X, torch.zeros(4, 64, dtype=torch.bfloat16), torch.zeros(1 << 20, dtype=torch.uint8))


def test_flash_layout_and_unsupported_shapes(lib):
    """xHC-Flash workspace sizing and layout; shapes without kernels are
    refused before anything runs."""
    cfg = Config(N=16, k=4, m=2, C=4096, B=2, S=8192, n_convs=3, dtype="bf16")
    n = lib.flash_workspace_bytes(cfg)
    L = lib.flash_layout(cfg)
    assert L.total == n > 0
    T = cfg.T
    offs = sorted([(L.idx, T * 4 * 4), (L.p, T * 4 * 4), (L.h_pre_attn, T * 16 * 4), (L.h_pre_mlp, T * 16 * 4),
                   (L.h_post_attn, T * 4 * 4), (L.h_res, T * 16 * 4), (L.h_post_mlp, T * 16 * 4),
                   (L.z_router, T * 16 * 4)])
    for (o1, s1), (o2, _) in zip(offs, offs[1:]):
        assert o1 % 256 == 0 and o1 + s1 <= o2
    assert offs[-1][0] + offs[-1][1] <= n
    bad = Config(N=16, k=2, m=1, C=256, B=1, S=8, n_convs=3, dtype="bf16")
    assert lib.flash_workspace_bytes(bad) == 0
    with pytest.raises(binding.XhcError) as e:
        lib.flash_layout(bad)
    assert e.value.status == binding.XHC_ERR_UNSUPPORTED
    assert lib.flash_workspace_bytes(Config(N=16, k=4, m=2, C=256, B=0, S=8, n_convs=3)) == 0


def _fw():
    w = binding.XhcfWeights()
    for n in ("w_full", "w_post_attn", "w_act_mlp", "conv_w", "b_pre_attn", "b_pre_mlp", "b_post_attn", "b_res",
              "b_post_mlp"):
        setattr(w, n, 0x10000)
    return w


def _f4w():
    w = binding.Xhcf4Weights()
    w.w_full = w.w_act_last = w.b_res = 0x10000
    for i in range(3):
        w.w_post[i] = 0x10000
    for i in range(2):
        w.conv_w[i] = 0x10000
    for i in range(4):
        w.b_pre[i] = w.b_post[i] = 0x10000
    return w


@pytest.mark.skipif(torch.cuda.is_available(), reason="fake device pointers: run on a host without a GPU only")
def test_flash_decode_and_4sub_calls_reject_bad_arguments_before_launch(lib):
    d = lib.dll
    ok = _cfg(B=1, S=16).c()
    # xHC-Flash: unsupported (N, k), misaligned or aliased buffers, missing weights
    bad = _cfg(k=2, m=1).c()
    assert d.xhcf_pre(ctypes.byref(bad), ctypes.byref(_fw()), 0x20000, 0x30000, 0x50000, 0x40000, None) == \
        binding.XHC_ERR_UNSUPPORTED
    assert d.xhcf_pre(ctypes.byref(ok), ctypes.byref(_fw()), 0x20000, 0x30000, 0x30000, 0x40000, None) == \
        binding.XHC_ERR_INVALID_ARG and "alias" in lib.last_error()
    assert d.xhcf_mid(ctypes.byref(ok), ctypes.byref(_fw()), 0x20000, 0x30000, 0x50008, 0x40000, None) == \
        binding.XHC_ERR_INVALID_ARG and "aligned" in lib.last_error()
    w = _fw()
    w.conv_w = 0
    assert d.xhcf_post(ctypes.byref(ok), ctypes.byref(w), 0x20000, 0x30000, 0x40000, None) == \
        binding.XHC_ERR_INVALID_ARG and "conv_w" in lib.last_error()
    # decode: one token per sequence, MLP-type only, an aligned steps array
    xw = XhcWeights()
    xw.w_full = xw.w_act = xw.b_pre = xw.b_res = xw.b_post = xw.conv_w = 0x10000
    assert d.xhc_post_decode(ctypes.byref(ok), ctypes.byref(xw), 0x20000, 0x30000, 0x50000, 0x60000, 0x40000,
                             None) == binding.XHC_ERR_INVALID_ARG and "seq must be 1" in lib.last_error()
    one = _cfg(B=4, S=1).c()
    attn = _cfg(B=4, S=1, n_convs=0).c()
    assert d.xhc_post_decode(ctypes.byref(attn), ctypes.byref(xw), 0x20000, 0x30000, 0x50000, 0x60000, 0x40000,
                             None) == binding.XHC_ERR_UNSUPPORTED and "xhc_post" in lib.last_error()
    assert d.xhc_post_decode(ctypes.byref(one), ctypes.byref(xw), 0x20000, 0x30000, 0x50000, 0x60002, 0x40000,
                             None) == binding.XHC_ERR_INVALID_ARG and "steps" in lib.last_error()
    assert d.xhc_post_decode(ctypes.byref(one), ctypes.byref(xw), 0x20000, 0x30000, 0x20000, 0x60000, 0x40000,
                             None) == binding.XHC_ERR_INVALID_ARG
    # xHC-Flash-4sub: sublayer index, per-sublayer weights, buffers
    for q in (0, 5):
        assert d.xhcf4_post(ctypes.byref(ok), ctypes.byref(_f4w()), q, 0x20000, 0x30000, 0x50000, 0x60000, 0x40000,
                            None) == binding.XHC_ERR_INVALID_ARG and "outside 1..4" in lib.last_error()
    w4 = _f4w()
    w4.conv_w[1] = 0
    assert d.xhcf4_post(ctypes.byref(ok), ctypes.byref(w4), 4, 0x20000, 0x30000, 0x50000, 0x60000, 0x40000,
                        None) == binding.XHC_ERR_INVALID_ARG and "conv_w[1]" in lib.last_error()
    w4 = _f4w()
    w4.b_res = 0
    assert d.xhcf4_post(ctypes.byref(ok), ctypes.byref(w4), 3, 0x20000, 0x30000, 0x50000, 0x60000, 0x40000,
                        None) == binding.XHC_ERR_INVALID_ARG and "b_res" in lib.last_error()
    assert d.xhcf4_pre(ctypes.byref(ok), ctypes.byref(_f4w()), 0x20000, 0x30000, 0x20000, 0x40000, None) == \
        binding.XHC_ERR_INVALID_ARG and "bases" in lib.last_error()
    w4 = _f4w()
    w4.w_post[1] = 0
    assert d.xhcf4_pre(ctypes.byref(ok), ctypes.byref(w4), 0x20000, 0x30000, 0x50000, 0x40000, None) == \
        binding.XHC_ERR_INVALID_ARG
    assert lib.flash4_workspace_bytes(_cfg(k=2, m=1)) == 0


def test_backward_layout(lib):
    """Backward workspace: public arrays aligned, disjoint, inside the total;
    an empty batch needs none; shapes without kernels are refused."""
    for cfg in (_cfg(), _cfg(n_convs=0), _cfg(N=8, k=4, m=1, C=256, B=1, S=33, dtype="f32")):
        n = lib.backward_workspace_bytes(cfg)
        L = lib.backward_layout(cfg)
        T, N, k, Kr = cfg.T, cfg.N, cfg.k, cfg.K_r
        offs = sorted([(L.d_h_pre, T * N * 4), (L.d_h_res, T * k * k * 4), (L.d_h_post, T * k * Kr * 4),
                       (L.d_p, T * k * 4)])
        for (o1, s1), (o2, _) in zip(offs, offs[1:]):
            assert o1 % 256 == 0 and o1 + s1 <= o2
        assert offs[-1][0] + offs[-1][1] <= n == L.total
    assert lib.backward_workspace_bytes(_cfg(B=0)) == 0
    assert lib.backward_workspace_bytes(_cfg(N=16, k=3, m=1)) == 0
    with pytest.raises(binding.XhcError) as e:
        lib.backward_layout(_cfg(N=16, k=3, m=1))
    assert e.value.status == binding.XHC_ERR_UNSUPPORTED


@pytest.mark.skipif(torch.cuda.is_available(), reason="fake device pointers: run on a host without a GPU only")
def test_backward_calls_reject_bad_arguments_before_launch(lib):
    d = lib.dll
    ok = _cfg(B=1, S=16).c()
    attn = _cfg(B=1, S=16, n_convs=0).c()
    xw = XhcWeights()
    xw.w_full = xw.w_act = xw.b_pre = xw.b_res = xw.b_post = xw.conv_w = 0x10000
    X, out, d_inp, d_X, dX, d_out, d_conv, ws, bws = (0x20000, 0x30000, 0x40000, 0x50000, 0x60000, 0x70000,
                                                      0x80000, 0x90000, 0xa0000)
    post = d.xhc_post_backward

    def pb(c, w, *a):
        return post(ctypes.byref(c), ctypes.byref(w), *a, None)
    args = [X, out, d_inp, d_X, d_out, d_conv, ws, bws]
    # misaligned, NULL, aliased
    bad = list(args)
    bad[4] = 0x70008
    assert pb(ok, xw, *bad) == binding.XHC_ERR_INVALID_ARG and "aligned" in lib.last_error()
    bad = list(args)
    bad[0] = None
    assert pb(ok, xw, *bad) == binding.XHC_ERR_INVALID_ARG
    bad = list(args)
    bad[4] = X
    assert pb(ok, xw, *bad) == binding.XHC_ERR_INVALID_ARG and "alias" in lib.last_error()
    bad = list(args)
    bad[4] = d_X
    assert pb(ok, xw, *bad) == binding.XHC_ERR_INVALID_ARG and "alias" in lib.last_error()
    bad = list(args)
    bad[7] = d_out
    assert pb(ok, xw, *bad) == binding.XHC_ERR_INVALID_ARG
    # MLP-type needs d_conv and the conv kernels; attention-type needs neither
    bad = list(args)
    bad[5] = None
    assert pb(ok, xw, *bad) == binding.XHC_ERR_INVALID_ARG and "d_conv" in lib.last_error()
    w = XhcWeights()
    w.w_full = w.w_act = w.b_pre = w.b_res = w.b_post = 0x10000
    assert pb(ok, w, *args) == binding.XHC_ERR_INVALID_ARG and "conv_w" in lib.last_error()
    # unsupported (N, k) and an empty batch
    assert pb(_cfg(k=3, m=1).c(), xw, *args) == binding.XHC_ERR_UNSUPPORTED
    e = _cfg(B=0).c()
    assert pb(e, xw, *([None] * 8)) == binding.XHC_OK
    # generation half: every gradient pointer, aligned buffers, no aliasing
    # except dX on d_X
    pre = d.xhc_pre_backward
    g = binding.XhcGrads(0xb0000, 0xc0000, 0xd0000, 0xd1000, 0xd2000, 0xd3000)

    def qb(c, *a):
        return pre(ctypes.byref(c), ctypes.byref(xw), *a, None)
    assert qb(ok, X, d_inp, d_X, X, ctypes.byref(g), ws, bws) == \
        binding.XHC_ERR_INVALID_ARG and "alias" in lib.last_error()
    assert qb(ok, X, d_inp, d_X, d_inp, ctypes.byref(g), ws, bws) == \
        binding.XHC_ERR_INVALID_ARG and "alias" in lib.last_error()
    assert qb(ok, X, d_inp, d_X, dX, ctypes.byref(g), ws, d_X) == \
        binding.XHC_ERR_INVALID_ARG and "alias" in lib.last_error()
    assert qb(ok, X, d_inp, d_X, 0x60004, ctypes.byref(g), ws, bws) == \
        binding.XHC_ERR_INVALID_ARG and "aligned" in lib.last_error()
    assert qb(ok, X, None, d_X, dX, ctypes.byref(g), ws, bws) == binding.XHC_ERR_INVALID_ARG
    g2 = binding.XhcGrads(0xb0000, 0xc0000, 0xd0000, 0xd1000, 0xd2000, 0)
    assert qb(ok, X, d_inp, d_X, dX, ctypes.byref(g2), ws, bws) == \
        binding.XHC_ERR_INVALID_ARG and "gradient" in lib.last_error()
    assert qb(ok, X, d_inp, d_X, dX, None, ws, bws) == binding.XHC_ERR_INVALID_ARG
    assert qb(attn, X, d_inp, d_X, dX, ctypes.byref(g), bws, bws) == binding.XHC_ERR_INVALID_ARG


@pytest.mark.skipif(torch.cuda.is_available(), reason="fake device pointers: run on a host without a GPU only")
def test_noalloc_write_refuses_what_its_scratch_cannot_hold(lib):
    """xhc_post_noalloc: an MLP-type write with Gram-Schmidt needs
    80 * ceil(C / 1024) * T bytes of scratch; above the library's array it is
    refused on the host, with nothing launched; the attention type needs none."""
    w = XhcWeights()
    w.w_full = w.w_act = w.b_pre = w.b_res = w.b_post = w.conv_w = 0x10000
    fit = _cfg(C=4096, B=1, S=(8 << 20) // 320)
    over = _cfg(C=4096, B=1, S=(8 << 20) // 320 + 1)
    assert 80 * 4 * fit.T <= 8 << 20 < 80 * 4 * over.T
    rc = lib.dll.xhc_post_noalloc(ctypes.byref(over.c()), ctypes.byref(w), 0x20000, 0x30000, 0x40000, None)
    assert rc == binding.XHC_ERR_INVALID_ARG and "scratch" in lib.last_error()
    nomgs = _cfg(C=4096, B=1, S=(8 << 20) // 320 + 1, use_mgs=0)
    rc = lib.dll.xhc_post_noalloc(ctypes.byref(nomgs.c()), ctypes.byref(w), 0x20001, 0x30000, 0x40000, None)
    assert rc == binding.XHC_ERR_INVALID_ARG and "aligned" in lib.last_error()   # past the scratch check
    attn = _cfg(C=4096, B=1, S=(8 << 20) // 320 + 1, n_convs=0)
    rc = lib.dll.xhc_post_noalloc(ctypes.byref(attn.c()), ctypes.byref(w), 0x20000, 0x20000, 0x40000, None)
    assert rc == binding.XHC_ERR_INVALID_ARG and "alias" in lib.last_error()     # past the scratch check
