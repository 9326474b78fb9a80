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
