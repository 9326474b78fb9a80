"""ctypes binding of libxhc: the same calls as include/xhc.h.

Argument marshalling only: PyTorch tensors are checked (device, dtype,
shape, contiguity) so that no host pointer or undersized buffer reaches a
kernel, then their device pointers and the current HIP stream are passed to
the C ABI.  Every step of the layer runs in the HIP library; there is no
other code path.  ``load()`` raises when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libxhc.so")

XHC_OK, XHC_ERR_INVALID_ARG, XHC_ERR_UNSUPPORTED, XHC_ERR_HIP = 0, 1, 2, 3
XHC_F32, XHC_BF16 = 0, 1
_DT = {"f32": (XHC_F32, torch.float32), "bf16": (XHC_BF16, torch.bfloat16)}
SIZE_MAX = ctypes.c_size_t(-1).value

# Exported symbols, in the order include/xhc.h declares them.
EXPORTS = (
    "xhc_workspace_bytes", "mhc_workspace_bytes", "xhc_workspace_layout", "mhc_workspace_layout",
    "xhc_pre", "xhc_post", "xhc_post_noalloc", "mhc_pre", "mhc_post", "xhc_route", "xhc_pre_chained", "xhc_post_chained",
    "xhc_post_decode", "xhcf_workspace_bytes", "xhcf_workspace_layout", "xhcf_pre", "xhcf_mid", "xhcf_post",
    "xhcf4_workspace_bytes", "xhcf4_workspace_layout", "xhcf4_pre", "xhcf4_post",
    "xhc_backward_workspace_bytes", "xhc_backward_workspace_layout", "xhc_post_backward", "xhc_pre_backward",
    "xhc_probe_read", "xhc_last_error",
)


class XhcConfig(ctypes.Structure):
    _fields_ = [
        ("n_streams", ctypes.c_int32), ("k_active", ctypes.c_int32), ("m_fixed", ctypes.c_int32),
        ("channels", ctypes.c_int32), ("batch", ctypes.c_int32), ("seq", ctypes.c_int32),
        ("n_convs", ctypes.c_int32), ("conv_kernel", ctypes.c_int32 * 3), ("use_mgs", ctypes.c_int32),
        ("sinkhorn_iters", ctypes.c_int32), ("dtype", ctypes.c_int32), ("eps_norm", ctypes.c_float),
        ("eps_mgs", ctypes.c_float),
    ]


class XhcWeights(ctypes.Structure):
    _fields_ = [
        ("w_full", ctypes.c_void_p), ("w_act", ctypes.c_void_p), ("conv_w", ctypes.c_void_p),
        ("b_pre", ctypes.c_void_p), ("b_res", ctypes.c_void_p), ("b_post", ctypes.c_void_p),
        ("alpha_pre", ctypes.c_float), ("alpha_res", ctypes.c_float), ("alpha_post", ctypes.c_float),
    ]


class XhcWsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("idx", "p", "h_pre", "h_res", "h_post", "z_router", "status", "total")]


class XhcfWeights(ctypes.Structure):
    _fields_ = [
        ("w_full", ctypes.c_void_p), ("w_post_attn", ctypes.c_void_p), ("w_act_mlp", ctypes.c_void_p),
        ("conv_w", ctypes.c_void_p), ("b_pre_attn", ctypes.c_void_p), ("b_pre_mlp", ctypes.c_void_p),
        ("b_post_attn", ctypes.c_void_p), ("b_res", ctypes.c_void_p), ("b_post_mlp", ctypes.c_void_p),
        ("alpha_pre_attn", ctypes.c_float), ("alpha_pre_mlp", ctypes.c_float), ("alpha_post_attn", ctypes.c_float),
        ("alpha_res", ctypes.c_float), ("alpha_post_mlp", ctypes.c_float),
    ]


class XhcfWsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("idx", "p", "h_pre_attn", "h_pre_mlp", "h_post_attn", "h_res",
                                               "h_post_mlp", "z_router", "total")]


class Xhcf4Weights(ctypes.Structure):
    _fields_ = [
        ("w_full", ctypes.c_void_p), ("w_post", ctypes.c_void_p * 3), ("w_act_last", ctypes.c_void_p),
        ("conv_w", ctypes.c_void_p * 2), ("b_pre", ctypes.c_void_p * 4), ("b_post", ctypes.c_void_p * 4),
        ("b_res", ctypes.c_void_p), ("alpha_pre", ctypes.c_float * 4), ("alpha_post", ctypes.c_float * 4),
        ("alpha_res", ctypes.c_float),
    ]


class Xhcf4WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("idx", "p", "h_pre", "h_post", "h_res", "z_router", "total")]


class XhcGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("dW_full", "dW_act", "d_b_pre", "d_b_res", "d_b_post", "d_alpha")]


class XhcBwdWsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("d_h_pre", "d_h_res", "d_h_post", "d_p", "total")]


class XhcError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"libxhc status {status}: {msg}")
        self.status = status


@dataclass
class Config:
    """Python view of xhc_config.  K_r = 4 when n_convs == 3, else 1."""
    N: int
    C: int
    B: int
    S: int
    k: int = 0
    m: int = 0
    n_convs: int = 0
    kernels: tuple = (4, 8, 12)
    use_mgs: int = 1
    iters: int = 20
    dtype: str = "bf16"
    eps_norm: float = 1e-6
    eps_mgs: float = 1e-6

    @property
    def T(self):
        return self.B * self.S

    @property
    def K_r(self):
        return 4 if self.n_convs == 3 else 1

    @property
    def torch_dtype(self):
        return _DT[self.dtype][1]

    def c(self) -> XhcConfig:
        c = XhcConfig()
        c.n_streams, c.k_active, c.m_fixed, c.channels = self.N, self.k, self.m, self.C
        c.batch, c.seq, c.n_convs = self.B, self.S, self.n_convs
        for i in range(3):
            c.conv_kernel[i] = int(self.kernels[i]) if i < len(self.kernels) else 0
        c.use_mgs, c.sinkhorn_iters = int(self.use_mgs), self.iters
        c.dtype = _DT[self.dtype][0] if self.dtype in _DT else int(self.dtype)
        c.eps_norm, c.eps_mgs = self.eps_norm, self.eps_mgs
        return c


@dataclass
class Weights:
    """Device tensors of one sublayer (kept alive by this object)."""
    w_full: torch.Tensor
    b_pre: torch.Tensor
    b_res: torch.Tensor
    b_post: torch.Tensor
    alpha_pre: float
    alpha_res: float
    alpha_post: float
    w_act: torch.Tensor | None = None
    conv_w: torch.Tensor | None = None   # [sum kappa, C] float32, lag-major
    _keep: list = field(default_factory=list, repr=False)

    def c(self) -> XhcWeights:
        w = XhcWeights()
        ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)
        w.w_full, w.w_act, w.conv_w = ptr(self.w_full), ptr(self.w_act), ptr(self.conv_w)
        w.b_pre, w.b_res, w.b_post = ptr(self.b_pre), ptr(self.b_res), ptr(self.b_post)
        w.alpha_pre, w.alpha_res, w.alpha_post = self.alpha_pre, self.alpha_res, self.alpha_post
        return w


@dataclass
class FlashWeights:
    """Device tensors of one xHC-Flash block (kept alive by this object)."""
    w_full: torch.Tensor        # [N*C, 3N]
    w_post_attn: torch.Tensor   # [k*C, k]
    w_act_mlp: torch.Tensor     # [k*C, k*k + k*K_r]
    b_pre_attn: torch.Tensor
    b_pre_mlp: torch.Tensor
    b_post_attn: torch.Tensor
    b_res: torch.Tensor
    b_post_mlp: torch.Tensor
    alpha_pre_attn: float
    alpha_pre_mlp: float
    alpha_post_attn: float
    alpha_res: float
    alpha_post_mlp: float
    conv_w: torch.Tensor | None = None

    def c(self) -> XhcfWeights:
        w = XhcfWeights()
        ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)
        for name in ("w_full", "w_post_attn", "w_act_mlp", "conv_w", "b_pre_attn", "b_pre_mlp", "b_post_attn",
                     "b_res", "b_post_mlp"):
            setattr(w, name, ptr(getattr(self, name)))
        for name in ("alpha_pre_attn", "alpha_pre_mlp", "alpha_post_attn", "alpha_res", "alpha_post_mlp"):
            setattr(w, name, float(getattr(self, name)))
        return w


@dataclass
class Flash4Weights:
    """Device tensors of one xHC-Flash-4sub group (kept alive by this object)."""
    w_full: torch.Tensor          # [N*C, 5N]
    w_post: list                  # 3 tensors: [k*C, k], [k*C, k*K_r], [k*C, k]
    w_act_last: torch.Tensor      # [k*C, k*k + k*K_r]
    b_pre: list                   # 4 x [N]
    b_post: list                  # [k], [k*K_r], [k], [k*K_r]
    b_res: torch.Tensor
    alpha_pre: tuple
    alpha_post: tuple
    alpha_res: float
    conv_w: list = field(default_factory=lambda: [None, None])

    def c(self) -> Xhcf4Weights:
        w = Xhcf4Weights()
        ptr = lambda t: t.data_ptr() if t is not None else 0
        w.w_full, w.w_act_last, w.b_res = ptr(self.w_full), ptr(self.w_act_last), ptr(self.b_res)
        for i in range(3):
            w.w_post[i] = ptr(self.w_post[i])
        for i in range(2):
            w.conv_w[i] = ptr(self.conv_w[i])
        for i in range(4):
            w.b_pre[i], w.b_post[i] = ptr(self.b_pre[i]), ptr(self.b_post[i])
            w.alpha_pre[i], w.alpha_post[i] = float(self.alpha_pre[i]), float(self.alpha_post[i])
        w.alpha_res = float(self.alpha_res)
        return w


def _check(t, name, shape, dtype):
    if t is None:
        raise ValueError(f"{name} is required")
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_out(t, cfg):
    shape = (cfg.T, cfg.C) if (t is not None and t.dim() == 2) else (cfg.B, cfg.S, cfg.C)
    _check(t, "out", shape, cfg.torch_dtype)


def _stream_ptr(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


class Lib:
    def __init__(self, path=LIB_PATH):
        if not os.path.exists(path):
            raise RuntimeError(f"libxhc is not built ({path} missing): run __graft_entry__.build()")
        self.path = path
        self.dll = ctypes.CDLL(path)
        d = self.dll
        d.xhc_workspace_bytes.restype = ctypes.c_size_t
        d.xhc_workspace_bytes.argtypes = [ctypes.POINTER(XhcConfig)]
        d.mhc_workspace_bytes.restype = ctypes.c_size_t
        d.mhc_workspace_bytes.argtypes = [ctypes.POINTER(XhcConfig)]
        for fn in (d.xhc_workspace_layout, d.mhc_workspace_layout):
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.POINTER(XhcConfig), ctypes.POINTER(XhcWsLayout)]
        for fn in (d.xhc_pre, d.xhc_post, d.xhc_post_noalloc, d.mhc_pre, d.mhc_post):
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.POINTER(XhcConfig), ctypes.POINTER(XhcWeights), ctypes.c_void_p,
                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        d.xhc_route.restype = ctypes.c_int
        d.xhc_route.argtypes = [ctypes.POINTER(XhcConfig), ctypes.POINTER(XhcWeights), ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_void_p]
        for fn in (d.xhc_pre_chained, d.xhc_post_chained):
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.POINTER(XhcConfig), ctypes.POINTER(XhcWeights), ctypes.POINTER(XhcConfig),
                           ctypes.POINTER(XhcWeights), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                           ctypes.c_void_p, ctypes.c_void_p]
        d.xhc_post_decode.restype = ctypes.c_int
        d.xhc_post_decode.argtypes = [ctypes.POINTER(XhcConfig), ctypes.POINTER(XhcWeights), ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p]
        d.xhcf_workspace_bytes.restype = ctypes.c_size_t
        d.xhcf_workspace_bytes.argtypes = [ctypes.POINTER(XhcConfig)]
        d.xhcf_workspace_layout.restype = ctypes.c_int
        d.xhcf_workspace_layout.argtypes = [ctypes.POINTER(XhcConfig), ctypes.POINTER(XhcfWsLayout)]
        for fn in (d.xhcf_pre, d.xhcf_mid):
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.POINTER(XhcConfig), ctypes.POINTER(XhcfWeights), ctypes.c_void_p,
                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        d.xhcf_post.restype = ctypes.c_int
        d.xhcf_post.argtypes = [ctypes.POINTER(XhcConfig), ctypes.POINTER(XhcfWeights), ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        d.xhcf4_workspace_bytes.restype = ctypes.c_size_t
        d.xhcf4_workspace_bytes.argtypes = [ctypes.POINTER(XhcConfig)]
        d.xhcf4_workspace_layout.restype = ctypes.c_int
        d.xhcf4_workspace_layout.argtypes = [ctypes.POINTER(XhcConfig), ctypes.POINTER(Xhcf4WsLayout)]
        d.xhcf4_pre.restype = ctypes.c_int
        d.xhcf4_pre.argtypes = [ctypes.POINTER(XhcConfig), ctypes.POINTER(Xhcf4Weights), ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        d.xhcf4_post.restype = ctypes.c_int
        d.xhcf4_post.argtypes = [ctypes.POINTER(XhcConfig), ctypes.POINTER(Xhcf4Weights), ctypes.c_int32,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p]
        d.xhc_backward_workspace_bytes.restype = ctypes.c_size_t
        d.xhc_backward_workspace_bytes.argtypes = [ctypes.POINTER(XhcConfig)]
        d.xhc_backward_workspace_layout.restype = ctypes.c_int
        d.xhc_backward_workspace_layout.argtypes = [ctypes.POINTER(XhcConfig), ctypes.POINTER(XhcBwdWsLayout)]
        d.xhc_post_backward.restype = ctypes.c_int
        d.xhc_post_backward.argtypes = [ctypes.POINTER(XhcConfig), ctypes.POINTER(XhcWeights)] + \
            [ctypes.c_void_p] * 9
        d.xhc_pre_backward.restype = ctypes.c_int
        d.xhc_pre_backward.argtypes = [ctypes.POINTER(XhcConfig), ctypes.POINTER(XhcWeights)] + \
            [ctypes.c_void_p] * 4 + [ctypes.POINTER(XhcGrads), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        d.xhc_last_error.restype = ctypes.c_char_p
        d.xhc_probe_read.restype = ctypes.c_int
        d.xhc_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        d.xhc_last_error.argtypes = []

    # -------------------------------------------------------------- helpers
    def probe_read(self, src, sink, mode=0, stream=None):
        """Measurement helper: one read-only pass over the device tensor src."""
        if not (src.is_cuda and sink.is_cuda and sink.dtype == torch.int32 and sink.numel() >= 4096):
            raise ValueError("probe_read: src and a 4096-word int32 sink on the GPU")
        self._ok(self.dll.xhc_probe_read(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(), mode,
                                         _stream_ptr(stream)))

    def last_error(self) -> str:
        return self.dll.xhc_last_error().decode()

    def _ok(self, status):
        if status != XHC_OK:
            raise XhcError(status, self.last_error())

    def workspace_bytes(self, cfg: Config, mhc=False) -> int:
        c = cfg.c()
        fn = self.dll.mhc_workspace_bytes if mhc else self.dll.xhc_workspace_bytes
        return int(fn(ctypes.byref(c)))

    def layout(self, cfg: Config, mhc=False) -> XhcWsLayout:
        c, L = cfg.c(), XhcWsLayout()
        fn = self.dll.mhc_workspace_layout if mhc else self.dll.xhc_workspace_layout
        self._ok(fn(ctypes.byref(c), ctypes.byref(L)))
        return L

    def workspace(self, cfg: Config, mhc=False, device="cuda") -> torch.Tensor:
        n = self.workspace_bytes(cfg, mhc)
        if n == 0 and cfg.T > 0:
            self.layout(cfg, mhc)   # raises with the library's message
        return torch.empty(max(n, 256), dtype=torch.uint8, device=device)

    def ws_arrays(self, cfg: Config, ws: torch.Tensor, mhc=False) -> dict:
        """Views of the public workspace arrays (see xhc_ws_layout)."""
        L = self.layout(cfg, mhc)
        T, N, k, Kr = cfg.T, cfg.N, (cfg.N if mhc else cfg.k), cfg.K_r

        def view(off, shape, dt=torch.float32):
            n = 1
            for s in shape:
                n *= s
            return ws[off: off + 4 * n].view(dt).reshape(shape)

        if mhc:
            return dict(h_pre=view(L.h_pre, (T, N)), h_res=view(L.h_res, (T, N, N)),
                        h_post=view(L.h_post, (T, N)))
        return dict(idx=view(L.idx, (T, k), torch.int32), p=view(L.p, (T, k)), h_pre=view(L.h_pre, (T, N)),
                    h_res=view(L.h_res, (T, k, k)), h_post=view(L.h_post, (T, k, Kr)),
                    z=view(L.z_router, (T, N)), status=view(L.status, (1,), torch.int32))

    def _check_common(self, cfg, w, X, ws, mhc, pre):
        dt = cfg.torch_dtype
        _check(X, "X", (cfg.T, cfg.N, cfg.C), dt)
        need = self.workspace_bytes(cfg, mhc)
        if ws is None or not ws.is_cuda or ws.numel() * ws.element_size() < need:
            raise ValueError(f"workspace must be a GPU tensor of at least {need} bytes")
        if pre:
            ncol = 2 * cfg.N + (cfg.N * cfg.N if mhc else 0)
            _check(w.w_full, "w_full", (cfg.N * cfg.C, ncol), dt)
            k = cfg.N if mhc else cfg.k
            _check(w.b_pre, "b_pre", (cfg.N,), torch.float32)
            _check(w.b_res, "b_res", (k * k,), torch.float32)
            _check(w.b_post, "b_post", ((cfg.N,) if mhc else (k * cfg.K_r,)), torch.float32)
            if not mhc:
                _check(w.w_act, "w_act", (k * cfg.C, k * k + k * cfg.K_r), dt)
        elif not mhc and cfg.K_r == 4:
            _check(w.conv_w, "conv_w", (sum(cfg.kernels), cfg.C), torch.float32)

    # -------------------------------------------------------------- the ABI
    def xhc_pre(self, cfg: Config, w: Weights, X, inp, ws, stream=None):
        self._check_common(cfg, w, X, ws, False, True)
        _check(inp, "inp", (cfg.T, cfg.C), cfg.torch_dtype)
        c, cw = cfg.c(), w.c()
        self._ok(self.dll.xhc_pre(ctypes.byref(c), ctypes.byref(cw), X.data_ptr(), inp.data_ptr(),
                                  ws.data_ptr(), _stream_ptr(stream)))

    def xhc_post(self, cfg: Config, w: Weights, X, out, ws, stream=None):
        self._check_common(cfg, w, X, ws, False, False)
        _check_out(out, cfg)
        c, cw = cfg.c(), w.c()
        self._ok(self.dll.xhc_post(ctypes.byref(c), ctypes.byref(cw), X.data_ptr(), out.data_ptr(),
                                   ws.data_ptr(), _stream_ptr(stream)))

    def xhc_post_noalloc(self, cfg: Config, w: Weights, X, out, ws, stream=None):
        """xhc_post with the workspace read only and the library's own scratch."""
        self._check_common(cfg, w, X, ws, False, False)
        _check_out(out, cfg)
        c, cw = cfg.c(), w.c()
        self._ok(self.dll.xhc_post_noalloc(ctypes.byref(c), ctypes.byref(cw), X.data_ptr(), out.data_ptr(),
                                           ws.data_ptr(), _stream_ptr(stream)))

    # chained sublayers: routing of sublayer l+1 prepared while sublayer l runs
    def xhc_route(self, cfg: Config, w: Weights, X, ws, stream=None):
        _check(X, "X", (cfg.T, cfg.N, cfg.C), cfg.torch_dtype)
        _check(w.w_full, "w_full", (cfg.N * cfg.C, 2 * cfg.N), cfg.torch_dtype)
        _check(w.b_pre, "b_pre", (cfg.N,), torch.float32)
        self._check_ws(cfg, ws)
        c, cw = cfg.c(), w.c()
        self._ok(self.dll.xhc_route(ctypes.byref(c), ctypes.byref(cw), X.data_ptr(), ws.data_ptr(),
                                    _stream_ptr(stream)))

    def _check_ws(self, cfg, ws):
        need = self.workspace_bytes(cfg)
        if ws is None or not ws.is_cuda or ws.numel() * ws.element_size() < need:
            raise ValueError(f"workspace must be a GPU tensor of at least {need} bytes")

    def _next(self, cfg_next, w_next, ws_next):
        if cfg_next is None:
            return None, None, 0
        _check(w_next.w_full, "w_next.w_full", (cfg_next.N * cfg_next.C, 2 * cfg_next.N), cfg_next.torch_dtype)
        _check(w_next.b_pre, "w_next.b_pre", (cfg_next.N,), torch.float32)
        self._check_ws(cfg_next, ws_next)
        return ctypes.byref(cfg_next.c()), ctypes.byref(w_next.c()), ws_next.data_ptr()

    def xhc_pre_chained(self, cfg: Config, w: Weights, cfg_next, w_next, X, inp, ws, ws_next, stream=None):
        self._check_common(cfg, w, X, ws, False, True)
        _check(inp, "inp", (cfg.T, cfg.C), cfg.torch_dtype)
        cn, wn, wsn = self._next(cfg_next, w_next, ws_next)
        c, cw = cfg.c(), w.c()
        self._ok(self.dll.xhc_pre_chained(ctypes.byref(c), ctypes.byref(cw), cn, wn, X.data_ptr(), inp.data_ptr(),
                                          ws.data_ptr(), wsn, _stream_ptr(stream)))

    def xhc_post_chained(self, cfg: Config, w: Weights, cfg_next, w_next, X, out, ws, ws_next, stream=None):
        self._check_common(cfg, w, X, ws, False, False)
        _check_out(out, cfg)
        cn, wn, wsn = self._next(cfg_next, w_next, ws_next)
        c, cw = cfg.c(), w.c()
        self._ok(self.dll.xhc_post_chained(ctypes.byref(c), ctypes.byref(cw), cn, wn, X.data_ptr(), out.data_ptr(),
                                           ws.data_ptr(), wsn, _stream_ptr(stream)))

    def mhc_pre(self, cfg: Config, w: Weights, X, inp, ws, stream=None):
        self._check_common(cfg, w, X, ws, True, True)
        _check(inp, "inp", (cfg.T, cfg.C), cfg.torch_dtype)
        c, cw = cfg.c(), w.c()
        self._ok(self.dll.mhc_pre(ctypes.byref(c), ctypes.byref(cw), X.data_ptr(), inp.data_ptr(),
                                  ws.data_ptr(), _stream_ptr(stream)))

    def mhc_post(self, cfg: Config, w: Weights | None, X, out, ws, stream=None):
        self._check_common(cfg, w, X, ws, True, False)
        _check_out(out, cfg)
        c = cfg.c()
        cw = w.c() if w is not None else XhcWeights()
        self._ok(self.dll.mhc_post(ctypes.byref(c), ctypes.byref(cw), X.data_ptr(), out.data_ptr(),
                                   ws.data_ptr(), _stream_ptr(stream)))


    # single-token decode: the conv history of each sequence in a 12-slot ring
    def xhc_post_decode(self, cfg: Config, w: Weights, X, out, conv_state, steps, ws, stream=None):
        if cfg.S != 1:
            raise ValueError("decode takes one new token per sequence (S == 1)")
        self._check_common(cfg, w, X, ws, False, False)
        _check(out, "out", (cfg.T, cfg.C), cfg.torch_dtype)
        _check(conv_state, "conv_state", (cfg.B, 12, cfg.C), cfg.torch_dtype)
        _check(steps, "steps", (cfg.B,), torch.int32)
        c, cw = cfg.c(), w.c()
        self._ok(self.dll.xhc_post_decode(ctypes.byref(c), ctypes.byref(cw), X.data_ptr(), out.data_ptr(),
                                          conv_state.data_ptr(), steps.data_ptr(), ws.data_ptr(),
                                          _stream_ptr(stream)))

    # backward of one xHC sublayer
    def backward_workspace_bytes(self, cfg: Config) -> int:
        c = cfg.c()
        return int(self.dll.xhc_backward_workspace_bytes(ctypes.byref(c)))

    def backward_layout(self, cfg: Config) -> XhcBwdWsLayout:
        c, L = cfg.c(), XhcBwdWsLayout()
        self._ok(self.dll.xhc_backward_workspace_layout(ctypes.byref(c), ctypes.byref(L)))
        return L

    def backward_workspace(self, cfg: Config, device="cuda") -> torch.Tensor:
        n = self.backward_workspace_bytes(cfg)
        if n == 0 and cfg.T > 0:
            self.backward_layout(cfg)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=device)

    def backward_ws_arrays(self, cfg: Config, bws: torch.Tensor) -> dict:
        """Views of the map gradients in a backward workspace."""
        L = self.backward_layout(cfg)
        T, N, k, Kr = cfg.T, cfg.N, cfg.k, cfg.K_r

        def view(off, shape):
            n = 1
            for s in shape:
                n *= s
            return bws[off: off + 4 * n].view(torch.float32).reshape(shape)

        return dict(h_pre=view(L.d_h_pre, (T, N)), h_res=view(L.d_h_res, (T, k, k)),
                    h_post=view(L.d_h_post, (T, k, Kr)), p=view(L.d_p, (T, k)))

    def grads(self, cfg: Config, device="cuda") -> dict:
        """Float gradient buffers for xhc_pre_backward (dict of tensors)."""
        N, k, C, Kr = cfg.N, cfg.k, cfg.C, cfg.K_r
        f = dict(dtype=torch.float32, device=device)
        return dict(W_full=torch.empty((N * C, 2 * N), **f), W_act=torch.empty((k * C, k * k + k * Kr), **f),
                    b_pre=torch.empty(N, **f), b_res=torch.empty(k * k, **f), b_post=torch.empty(k * Kr, **f),
                    alpha=torch.empty(3, **f))

    def _check_bws(self, cfg, bws):
        need = self.backward_workspace_bytes(cfg)
        if bws is None or not bws.is_cuda or bws.numel() * bws.element_size() < need:
            raise ValueError(f"backward workspace must be a GPU tensor of at least {need} bytes")

    def xhc_post_backward(self, cfg: Config, w: Weights, X, out, d_inp, d_X, d_out, d_conv, ws, bws, stream=None):
        self._check_common(cfg, w, X, ws, False, False)
        dt = cfg.torch_dtype
        for t, name, shape in ((out, "out", (cfg.T, cfg.C)), (d_inp, "d_inp", (cfg.T, cfg.C)),
                               (d_X, "d_X", (cfg.T, cfg.N, cfg.C)), (d_out, "d_out", (cfg.T, cfg.C))):
            _check(t, name, shape, dt)
        if cfg.K_r == 4:
            _check(d_conv, "d_conv", (sum(cfg.kernels), cfg.C), torch.float32)
        self._check_bws(cfg, bws)
        c, cw = cfg.c(), w.c()
        self._ok(self.dll.xhc_post_backward(ctypes.byref(c), ctypes.byref(cw), X.data_ptr(), out.data_ptr(),
                                            d_inp.data_ptr(), d_X.data_ptr(), d_out.data_ptr(),
                                            d_conv.data_ptr() if d_conv is not None else None, ws.data_ptr(),
                                            bws.data_ptr(), _stream_ptr(stream)))

    def xhc_pre_backward(self, cfg: Config, w: Weights, X, d_inp, d_X, dX, g: dict, ws, bws, stream=None):
        self._check_common(cfg, w, X, ws, False, True)
        for t, name, shape in ((d_inp, "d_inp", (cfg.T, cfg.C)), (d_X, "d_X", (cfg.T, cfg.N, cfg.C)),
                               (dX, "dX", (cfg.T, cfg.N, cfg.C))):
            _check(t, name, shape, cfg.torch_dtype)
        ref = self.grads(cfg, device="meta")
        for name, t in ref.items():
            _check(g[name], "d_" + name, tuple(t.shape), torch.float32)
        self._check_bws(cfg, bws)
        c, cw = cfg.c(), w.c()
        gg = XhcGrads(g["W_full"].data_ptr(), g["W_act"].data_ptr(), g["b_pre"].data_ptr(), g["b_res"].data_ptr(),
                      g["b_post"].data_ptr(), g["alpha"].data_ptr())
        self._ok(self.dll.xhc_pre_backward(ctypes.byref(c), ctypes.byref(cw), X.data_ptr(), d_inp.data_ptr(),
                                           d_X.data_ptr(), dX.data_ptr(), ctypes.byref(gg), ws.data_ptr(),
                                           bws.data_ptr(), _stream_ptr(stream)))

    # xHC-Flash block: attention + MLP sharing one routing
    def flash_workspace_bytes(self, cfg: Config) -> int:
        c = cfg.c()
        return int(self.dll.xhcf_workspace_bytes(ctypes.byref(c)))

    def flash_layout(self, cfg: Config) -> XhcfWsLayout:
        c, L = cfg.c(), XhcfWsLayout()
        self._ok(self.dll.xhcf_workspace_layout(ctypes.byref(c), ctypes.byref(L)))
        return L

    def flash_workspace(self, cfg: Config, device="cuda") -> torch.Tensor:
        n = self.flash_workspace_bytes(cfg)
        if n == 0 and cfg.T > 0:
            self.flash_layout(cfg)   # raises with the library's message
        return torch.empty(max(n, 256), dtype=torch.uint8, device=device)

    def flash_ws_arrays(self, cfg: Config, ws: torch.Tensor) -> dict:
        """Views of the public arrays of an xHC-Flash workspace."""
        L = self.flash_layout(cfg)
        T, N, k, Kr = cfg.T, cfg.N, cfg.k, cfg.K_r

        def view(off, shape, dt=torch.float32):
            n = 1
            for s in shape:
                n *= s
            return ws[off: off + 4 * n].view(dt).reshape(shape)

        return dict(idx=view(L.idx, (T, k), torch.int32), p=view(L.p, (T, k)),
                    h_pre_attn=view(L.h_pre_attn, (T, N)), h_pre_mlp=view(L.h_pre_mlp, (T, N)),
                    h_post_attn=view(L.h_post_attn, (T, k)), h_res=view(L.h_res, (T, k, k)),
                    h_post_mlp=view(L.h_post_mlp, (T, k, Kr)), z=view(L.z_router, (T, N)))

    def _check_flash(self, cfg, w, X, ws, stage):
        dt = cfg.torch_dtype
        _check(X, "X", (cfg.T, cfg.N, cfg.C), dt)
        need = self.flash_workspace_bytes(cfg)
        if ws is None or not ws.is_cuda or ws.numel() * ws.element_size() < need:
            raise ValueError(f"workspace must be a GPU tensor of at least {need} bytes")
        k, N = cfg.k, cfg.N
        if stage == 0:
            _check(w.w_full, "w_full", (N * cfg.C, 3 * N), dt)
            _check(w.w_post_attn, "w_post_attn", (k * cfg.C, k), dt)
            _check(w.w_act_mlp, "w_act_mlp", (k * cfg.C, k * k + k * cfg.K_r), dt)
            _check(w.b_pre_attn, "b_pre_attn", (N,), torch.float32)
            _check(w.b_pre_mlp, "b_pre_mlp", (N,), torch.float32)
            _check(w.b_post_attn, "b_post_attn", (k,), torch.float32)
        elif stage == 1:
            _check(w.b_res, "b_res", (k * k,), torch.float32)
            _check(w.b_post_mlp, "b_post_mlp", (k * cfg.K_r,), torch.float32)
        elif cfg.K_r == 4:
            _check(w.conv_w, "conv_w", (sum(cfg.kernels), cfg.C), torch.float32)

    def xhcf_pre(self, cfg: Config, w: FlashWeights, X, inp_attn, inp_mlp, ws, stream=None):
        self._check_flash(cfg, w, X, ws, 0)
        _check(inp_attn, "inp_attn", (cfg.T, cfg.C), cfg.torch_dtype)
        _check(inp_mlp, "inp_mlp", (cfg.T, cfg.C), cfg.torch_dtype)
        c, cw = cfg.c(), w.c()
        self._ok(self.dll.xhcf_pre(ctypes.byref(c), ctypes.byref(cw), X.data_ptr(), inp_attn.data_ptr(),
                                   inp_mlp.data_ptr(), ws.data_ptr(), _stream_ptr(stream)))

    def xhcf_mid(self, cfg: Config, w: FlashWeights, X, out_attn, inp_mlp, ws, stream=None):
        self._check_flash(cfg, w, X, ws, 1)
        _check_out(out_attn, cfg)
        _check(inp_mlp, "inp_mlp", (cfg.T, cfg.C), cfg.torch_dtype)
        c, cw = cfg.c(), w.c()
        self._ok(self.dll.xhcf_mid(ctypes.byref(c), ctypes.byref(cw), X.data_ptr(), out_attn.data_ptr(),
                                   inp_mlp.data_ptr(), ws.data_ptr(), _stream_ptr(stream)))

    def xhcf_post(self, cfg: Config, w: FlashWeights, X, out_mlp, ws, stream=None):
        self._check_flash(cfg, w, X, ws, 2)
        _check_out(out_mlp, cfg)
        c, cw = cfg.c(), w.c()
        self._ok(self.dll.xhcf_post(ctypes.byref(c), ctypes.byref(cw), X.data_ptr(), out_mlp.data_ptr(),
                                    ws.data_ptr(), _stream_ptr(stream)))


    # xHC-Flash-4sub group: two blocks sharing one routing
    def flash4_workspace_bytes(self, cfg: Config) -> int:
        c = cfg.c()
        return int(self.dll.xhcf4_workspace_bytes(ctypes.byref(c)))

    def flash4_layout(self, cfg: Config) -> Xhcf4WsLayout:
        c, L = cfg.c(), Xhcf4WsLayout()
        self._ok(self.dll.xhcf4_workspace_layout(ctypes.byref(c), ctypes.byref(L)))
        return L

    def flash4_workspace(self, cfg: Config, device="cuda") -> torch.Tensor:
        n = self.flash4_workspace_bytes(cfg)
        if n == 0 and cfg.T > 0:
            self.flash4_layout(cfg)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=device)

    def flash4_ws_arrays(self, cfg: Config, ws: torch.Tensor, K_q: int) -> dict:
        """Views of the public arrays; h_post has K_q components (those of the
        next sublayer to write)."""
        L = self.flash4_layout(cfg)
        T, N, k = cfg.T, cfg.N, cfg.k

        def view(off, shape, dt=torch.float32):
            n = 1
            for s in shape:
                n *= s
            return ws[off: off + 4 * n].view(dt).reshape(shape)

        return dict(idx=view(L.idx, (T, k), torch.int32), p=view(L.p, (T, k)), h_pre=view(L.h_pre, (4, T, N)),
                    h_post=view(L.h_post, (T, k, K_q)), h_res=view(L.h_res, (T, k, k)), z=view(L.z_router, (T, N)))

    def _check_flash4(self, cfg, w, X, ws):
        _check(X, "X", (cfg.T, cfg.N, cfg.C), cfg.torch_dtype)
        need = self.flash4_workspace_bytes(cfg)
        if ws is None or not ws.is_cuda or ws.numel() * ws.element_size() < need:
            raise ValueError(f"workspace must be a GPU tensor of at least {need} bytes")
        dt, k, N, Kr = cfg.torch_dtype, cfg.k, cfg.N, cfg.K_r
        _check(w.w_full, "w_full", (N * cfg.C, 5 * N), dt)
        for i, nc in enumerate((k, k * Kr, k)):
            _check(w.w_post[i], f"w_post[{i}]", (k * cfg.C, nc), dt)
        _check(w.w_act_last, "w_act_last", (k * cfg.C, k * k + k * Kr), dt)
        for i in range(4):
            _check(w.b_pre[i], f"b_pre[{i}]", (N,), torch.float32)
            _check(w.b_post[i], f"b_post[{i}]", ((k * Kr) if i % 2 else k,), torch.float32)
        _check(w.b_res, "b_res", (k * k,), torch.float32)
        if Kr == 4:
            for i in range(2):
                _check(w.conv_w[i], f"conv_w[{i}]", (sum(cfg.kernels), cfg.C), torch.float32)

    def xhcf4_pre(self, cfg: Config, w: Flash4Weights, X, inp, bases, ws, stream=None):
        self._check_flash4(cfg, w, X, ws)
        _check(inp, "inp", (cfg.T, cfg.C), cfg.torch_dtype)
        _check(bases, "bases", (3, cfg.T, cfg.C), cfg.torch_dtype)
        c, cw = cfg.c(), w.c()
        self._ok(self.dll.xhcf4_pre(ctypes.byref(c), ctypes.byref(cw), X.data_ptr(), inp.data_ptr(),
                                    bases.data_ptr(), ws.data_ptr(), _stream_ptr(stream)))

    def xhcf4_post(self, cfg: Config, w: Flash4Weights, q, X, out, bases, inp, ws, stream=None):
        self._check_flash4(cfg, w, X, ws)
        _check_out(out, cfg)
        _check(inp, "inp", (cfg.T, cfg.C), cfg.torch_dtype)
        _check(bases, "bases", (3, cfg.T, cfg.C), cfg.torch_dtype)
        c, cw = cfg.c(), w.c()
        self._ok(self.dll.xhcf4_post(ctypes.byref(c), ctypes.byref(cw), int(q), X.data_ptr(), out.data_ptr(),
                                     bases.data_ptr(), inp.data_ptr(), ws.data_ptr(), _stream_ptr(stream)))


_INSTANCE = None


def load(path=LIB_PATH) -> Lib:
    """The loaded library (cached).  Raises RuntimeError if it is not built."""
    global _INSTANCE
    if _INSTANCE is None or _INSTANCE.path != path:
        _INSTANCE = Lib(path)
    return _INSTANCE


def weights_to_device(wd: dict, device="cuda") -> Weights:
    """Move a dict from ``synth.xhc_layer_weights`` / ``mhc_layer_weights``
    (CPU tensors) to the GPU as a Weights object."""
    conv = wd.get("conv") or []
    conv_w = torch.cat(conv, 0).contiguous().to(device) if conv else None
    return Weights(
        w_full=wd["w_full"].contiguous().to(device), w_act=(wd["w_act"].contiguous().to(device)
                                                            if wd.get("w_act") is not None else None),
        conv_w=conv_w, b_pre=wd["b_pre"].float().contiguous().to(device),
        b_res=wd["b_res"].float().contiguous().to(device), b_post=wd["b_post"].float().contiguous().to(device),
        alpha_pre=float(wd["alpha_pre"]), alpha_res=float(wd["alpha_res"]), alpha_post=float(wd["alpha_post"]))


def flash_weights_to_device(wd: dict, device="cuda") -> FlashWeights:
    """Move a dict from ``synth.xhcf_block_weights`` (CPU tensors) to the GPU."""
    conv = wd.get("conv") or []
    dev = lambda t: t.contiguous().to(device)
    return FlashWeights(
        w_full=dev(wd["w_full"]), w_post_attn=dev(wd["w_post_attn"]), w_act_mlp=dev(wd["w_act_mlp"]),
        conv_w=torch.cat(conv, 0).contiguous().to(device) if conv else None,
        **{n: dev(wd[n].float()) for n in ("b_pre_attn", "b_pre_mlp", "b_post_attn", "b_res", "b_post_mlp")},
        **{n: float(wd[n]) for n in ("alpha_pre_attn", "alpha_pre_mlp", "alpha_post_attn", "alpha_res",
                                     "alpha_post_mlp")})


def flash4_weights_to_device(wd: dict, device="cuda") -> Flash4Weights:
    """Move a dict from ``synth.xhcf4_group_weights`` (CPU tensors) to the GPU."""
    dev = lambda t: t.contiguous().to(device)
    convs = [torch.cat(c, 0).contiguous().to(device) if c else None for c in wd["conv"]]
    return Flash4Weights(
        w_full=dev(wd["w_full"]), w_post=[dev(t) for t in wd["w_post"]], w_act_last=dev(wd["w_act_last"]),
        b_pre=[dev(t.float()) for t in wd["b_pre"]], b_post=[dev(t.float()) for t in wd["b_post"]],
        b_res=dev(wd["b_res"].float()), alpha_pre=tuple(wd["alpha_pre"]), alpha_post=tuple(wd["alpha_post"]),
        alpha_res=float(wd["alpha_res"]), conv_w=convs)
