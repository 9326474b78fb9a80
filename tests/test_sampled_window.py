"""Host checks of the sampled full-size parity method: the oracle run on one
token's 12-token output window (with zero state rows for the window's other
tokens) must give that token exactly the results of the oracle run on the
whole sequence, and the window must cover sequence starts and batch edges.
"""
import numpy as np
import pytest

import cases as K
from stream_residual_mixing_amd import synth
from stream_residual_mixing_amd.binding import Config


def test_out_window_matches_the_sequence_rows():
    S, C = 20, 8
    full = K.f64(synth.sublayer_out(5, 1, 2, S, C, "bf16"))
    for t in (0, 3, 11, 12, 19, 20, 21, 33, 39):
        b, s = divmod(t, S)
        win = K.out_window(5, 1, t, S, C, K.WINDOW)
        for i in range(K.WINDOW):
            src = s - (K.WINDOW - 1 - i)
            want = full[b, src] if src >= 0 else np.zeros(C)
            assert np.array_equal(win[i], want), (t, i)


@pytest.mark.parametrize("n_convs", [0, 3])
def test_one_token_window_equals_the_whole_sequence(n_convs):
    cfg = Config(N=6, k=3, m=1, C=32, B=2, S=30, n_convs=n_convs, dtype="bf16")
    seed = 11
    wd = synth.xhc_layer_weights(seed, 0, cfg.N, cfg.k, cfg.C, cfg.K_r, "bf16")
    ow = K.oracle_weights(wd)
    X = K.f64(synth.state(seed, cfg.T, cfg.N, cfg.C, "bf16"))
    out = K.f64(synth.sublayer_out(seed, 0, cfg.B, cfg.S, cfg.C, "bf16"))
    whole = K.oracle_xhc(cfg, X, out, ow)
    for t in K.sample_tokens(cfg.B, cfg.S, 4, seed):
        w = K.WINDOW if n_convs else 1
        r, _ = K.oracle_token(cfg, X[t], K.out_window(seed, 0, t, cfg.S, cfg.C, w), ow)
        for key in ("I", "p", "h_pre", "h_res", "h_post", "inp", "X", "z"):
            np.testing.assert_allclose(r[key], whole[key][t], rtol=0, atol=1e-12, err_msg=f"{key} t={t}")


def test_sample_covers_starts_ends_and_tile_edges():
    toks = K.sample_tokens(2, 8192, 5, 3)
    for b in range(2):
        for s in (0, 11, 12, 15, 16, 8191):
            assert b * 8192 + s in toks
    assert len(np.unique(toks)) == len(toks) and toks.max() < 2 * 8192
