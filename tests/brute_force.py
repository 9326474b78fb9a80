"""Scalar-loop re-derivation of one mHC / xHC sublayer for tiny shapes.

A second, deliberately different implementation used only to pin the
vectorised oracle: plain Python floats and loops, top-k by enumerating every
subset of routed streams, convolution by explicit lags, Gram-Schmidt by
explicit dot products.  It imports nothing from the oracle.
"""
from __future__ import annotations

import itertools
import math


def _sig(z):
    return 1.0 / (1.0 + math.exp(-z)) if z >= 0 else math.exp(z) / (1.0 + math.exp(z))


def _flat(Xt):
    return [v for row in Xt for v in row]


def _rms_scale(v, eps=1e-6):
    return 1.0 / math.sqrt(sum(a * a for a in v) / len(v) + eps)


def _ln(v, eps=1e-6):
    n = len(v)
    mu = sum(v) / n
    sd = math.sqrt(sum((a - mu) ** 2 for a in v) / n)
    return [(a - mu) / (sd + eps) for a in v]


def _matvec(v, W, col0, ncol):
    return [sum(v[r] * W[r][col0 + j] for r in range(len(v))) for j in range(ncol)]


def _sinkhorn(L, iters):
    n = len(L)
    mx = max(max(r) for r in L)
    M = [[math.exp(L[i][j] - mx) for j in range(n)] for i in range(n)]
    for _ in range(iters):
        for j in range(n):
            s = sum(M[i][j] for i in range(n))
            for i in range(n):
                M[i][j] /= s
        for i in range(n):
            s = sum(M[i])
            M[i] = [a / s for a in M[i]]
    return M


def mhc_token(Xt, out_t, W, alpha, b_pre, b_post, b_res, iters):
    """Xt: N lists of C floats.  Returns (inp, new state)."""
    N, C = len(Xt), len(Xt[0])
    x = _flat(Xt)
    sc = _rms_scale(x)
    xn = [a * sc for a in x]
    z = _matvec(xn, W, 0, 2 * N + N * N)
    hp = [_sig(alpha[0] * z[i] + b_pre[i]) for i in range(N)]
    ho = [2 * _sig(alpha[1] * z[N + i] + b_post[i]) for i in range(N)]
    L = [[alpha[2] * z[2 * N + i * N + j] + b_res[i * N + j] for j in range(N)] for i in range(N)]
    H = _sinkhorn(L, iters)
    inp = [sum(hp[i] * Xt[i][c] for i in range(N)) for c in range(C)]
    new = [[sum(H[i][j] * Xt[j][c] for j in range(N)) + ho[i] * out_t[c] for c in range(C)]
           for i in range(N)]
    return inp, new


def xhc_route_token(Xt, W_full, m, k):
    """Router by subset enumeration: the routed set is the (k-m)-subset of
    streams m..N-1 with the largest total score; then listed by descending
    score (ties to the lower index).  Returns (I, p, z)."""
    N = len(Xt)
    x = _ln(_flat(Xt))
    z = _matvec(x, W_full, 0, N)
    best, best_sum = None, -math.inf
    for sub in itertools.combinations(range(m, N), k - m):
        tot = sum(_sig(z[i]) for i in sub)
        if tot > best_sum:
            best, best_sum = sub, tot
    routed = sorted(best, key=lambda i: (-z[i], i))
    I = list(range(m)) + routed
    p = [1.0] * m + [_sig(z[i]) for i in routed]
    return I, p, z


def conv_seq(out_seq, w):
    """out_seq: S lists of C floats; w: kappa lists of C floats."""
    S, C = len(out_seq), len(out_seq[0])
    g = [[0.0] * C for _ in range(S)]
    for t in range(S):
        for lag in range(len(w)):
            if t - lag < 0:
                continue
            for c in range(C):
                g[t][c] += w[lag][c] * out_seq[t - lag][c]
    return g


def _dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def mgs_token(vecs, eps=1e-6):
    basis = [list(vecs[0])]
    for g in vecs[1:]:
        u = list(g)
        for v in basis:
            c = _dot(u, v) / (_dot(v, v) + eps)
            u = [a - c * b for a, b in zip(u, v)]
        basis.append(u)
    return basis


def xhc_sublayer(X, out, W_full, W_act, m, k, convs, alpha, b_pre, b_res, b_post, iters,
                 use_mgs=True):
    """X: T x N x C nested lists (T = B*S, batch-major); out: B x S x C.
    Returns dict(inp, X, I, p, h_pre, h_res, h_post)."""
    B, S = len(out), len(out[0])
    T, N, C = len(X), len(X[0]), len(X[0][0])
    K_r = 1 + len(convs)
    g_all = [[conv_seq(out[b], w) for w in convs] for b in range(B)]
    res = dict(inp=[], X=[], I=[], p=[], h_pre=[], h_res=[], h_post=[])
    for t in range(T):
        b, s = divmod(t, S)
        Xt = X[t]
        I, p, _ = xhc_route_token(Xt, W_full, m, k)
        x = _flat(Xt)
        sc = _rms_scale(x)
        zp = _matvec([a * sc for a in x], W_full, N, N)
        hp = [_sig(alpha[0] * zp[i] + b_pre[i]) for i in range(N)]
        inp = [sum(hp[i] * Xt[i][c] for i in range(N)) for c in range(C)]
        xa = [v for j in range(k) for v in Xt[I[j]]]
        sca = _rms_scale(xa)
        la = _matvec([a * sca for a in xa], W_act, 0, k * k + k * K_r)
        L = [[alpha[1] * la[i * k + j] + b_res[i * k + j] for j in range(k)] for i in range(k)]
        H = _sinkhorn(L, iters)
        H = [[a / max(sum(row), 1.0) for a in row] for row in H]
        P = [[2 * _sig(alpha[2] * la[k * k + j * K_r + r] + b_post[j * K_r + r]) for r in range(K_r)]
             for j in range(k)]
        comps = [out[b][s]] + [g_all[b][j][s] for j in range(len(convs))]
        V = mgs_token(comps) if (use_mgs and len(comps) > 1) else comps
        newX = [list(row) for row in Xt]
        for j in range(k):
            for c in range(C):
                mix = sum(H[j][i] * Xt[I[i]][c] for i in range(k))
                wr = sum(P[j][r] * V[r][c] for r in range(K_r))
                newX[I[j]][c] = mix + p[j] * wr
        res["inp"].append(inp)
        res["X"].append(newX)
        res["I"].append(I)
        res["p"].append(p)
        res["h_pre"].append(hp)
        res["h_res"].append(H)
        res["h_post"].append(P)
    return res


def xhcf_block(X, out_a, out_m, W_full, W_pa, W_am, m, k, convs, alpha, b_pa, b_pm, b_po, b_res, b_pm2,
               iters, use_mgs=True):
    """One xHC-Flash block (attention, then MLP) by scalar loops, in float64
    without rounding.  W_full has 3N columns (router | attention pre-map |
    MLP pre-map); W_pa is [k*C][k]; W_am is [k*C][k*k + k*K_r].
    alpha = (pre_attn, pre_mlp, post_attn, res, post_mlp).
    Returns dict(inp_attn, inp_mlp, X1, X, I, p, alpha_corr)."""
    B, S = len(out_m), len(out_m[0])
    T, N, C = len(X), len(X[0]), len(X[0][0])
    K_r = 1 + len(convs)
    g_all = [[conv_seq(out_m[b], w) for w in convs] for b in range(B)]
    res = dict(inp_attn=[], inp_mlp=[], X1=[], X=[], I=[], p=[], alpha_corr=[])
    for t in range(T):
        b, s = divmod(t, S)
        Xt = X[t]
        I, p, _ = xhc_route_token(Xt, W_full, m, k)
        x = _flat(Xt)
        sc = _rms_scale(x)
        xn = [a * sc for a in x]
        za = _matvec(xn, W_full, N, N)
        zm = _matvec(xn, W_full, 2 * N, N)
        hpa = [_sig(alpha[0] * za[i] + b_pa[i]) for i in range(N)]
        hpm = [_sig(alpha[1] * zm[i] + b_pm[i]) for i in range(N)]
        inp_a = [sum(hpa[i] * Xt[i][c] for i in range(N)) for c in range(C)]
        xa = [v for j in range(k) for v in Xt[I[j]]]
        sca = _rms_scale(xa)
        la = _matvec([a * sca for a in xa], W_pa, 0, k)
        hpo = [2 * _sig(alpha[2] * la[j] + b_po[j]) for j in range(k)]
        oa = out_a[b][s]
        # attention write, then the MLP input as the dense read of that state
        X1 = [list(row) for row in Xt]
        for j in range(k):
            for c in range(C):
                X1[I[j]][c] = Xt[I[j]][c] + p[j] * hpo[j] * oa[c]
        inp_m = [sum(hpm[i] * X1[i][c] for i in range(N)) for c in range(C)]
        acorr = sum(hpm[I[j]] * p[j] * hpo[j] for j in range(k))
        # MLP maps from the rewritten active rows, then full xHC's write
        xa1 = [v for j in range(k) for v in X1[I[j]]]
        sc1 = _rms_scale(xa1)
        l1 = _matvec([a * sc1 for a in xa1], W_am, 0, k * k + k * K_r)
        L = [[alpha[3] * l1[i * k + j] + b_res[i * k + j] for j in range(k)] for i in range(k)]
        H = _sinkhorn(L, iters)
        H = [[a / max(sum(row), 1.0) for a in row] for row in H]
        P = [[2 * _sig(alpha[4] * l1[k * k + j * K_r + r] + b_pm2[j * K_r + r]) for r in range(K_r)]
             for j in range(k)]
        comps = [out_m[b][s]] + [g_all[b][j][s] for j in range(len(convs))]
        V = mgs_token(comps) if (use_mgs and len(comps) > 1) else comps
        X2 = [list(row) for row in X1]
        for j in range(k):
            for c in range(C):
                mix = sum(H[j][i] * X1[I[i]][c] for i in range(k))
                wr = sum(P[j][r] * V[r][c] for r in range(K_r))
                X2[I[j]][c] = mix + p[j] * wr
        for key, v in (("inp_attn", inp_a), ("inp_mlp", inp_m), ("X1", X1), ("X", X2), ("I", I), ("p", p),
                       ("alpha_corr", acorr)):
            res[key].append(v)
    return res
