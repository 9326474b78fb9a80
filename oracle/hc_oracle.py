"""Float64 reference of the mHC and xHC residual-stream layer.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Notation follows the pages: a token's state is X in R^{N x C} (N streams of
C channels); vec X is its stream-major flattening (index i*C + c); the
sublayer F is given, so its output ``out`` is an input here.  Tokens are
batched as T = B*S rows in batch-major order (t = b*S + s); only the causal
convolution looks across tokens, and only within one batch item.

Readings of points the pages leave open are listed in the design notes and
repeated at the function that takes them.
"""
from __future__ import annotations

import numpy as np

EPS_NORM = 1e-6   # RMSNorm / LayerNorm epsilon (explainer, "What xHC changes")
EPS_MGS = 1e-6    # Gram-Schmidt epsilon on <v, v> (same listing; the paper
                  # text leaves it unstated: explainer, "What I could not check")


# --------------------------------------------------------------------------
# elementary pieces
# --------------------------------------------------------------------------

def sigmoid(z):
    """Logistic function 1 / (1 + e^{-z}), evaluated without overflow."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def rms_normalize(v, eps=EPS_NORM):
    """x / sqrt(mean(x^2) + eps) over the last axis, no gain.

    The RMSNorm that feeds the pre-map and the active-stream maps
    (explainer, "What xHC changes"; xHC paper, "Mapping generation").
    """
    v = np.asarray(v, dtype=np.float64)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps)


def ln_normalize(v, eps=EPS_NORM):
    """(x - mean) / (population std + eps) over the last axis, no affine.

    The LayerNorm of the router (explainer, "What xHC changes"; summary
    3.4.1).  Reading: the std is the population one and eps is added to the
    std, not to the variance, as in the explainer's sublayer code.
    """
    v = np.asarray(v, dtype=np.float64)
    mu = np.mean(v, axis=-1, keepdims=True)
    sd = np.sqrt(np.mean((v - mu) ** 2, axis=-1, keepdims=True))
    return (v - mu) / (sd + eps)


def sinkhorn(logits, iters):
    """Sinkhorn-Knopp projection of a (batch of) square logit matrices.

    The map is K = exp(logits) scaled on both sides, diag(r) K diag(c).  A
    round first picks the column scales c that give every column of
    diag(r) K diag(c) a sum of one, then the row scales r that give every
    row a sum of one; r and c start at one, so zero rounds leave K itself.
    This is the alternating column-then-row normalisation (explainer, "mHC:
    keep the mixing doubly stochastic"; xHC paper, "Manifold-Constrained
    HC") kept as two scale vectors per matrix.  Rows are settled last, so
    rows sum to one and what is left of the error sits on the columns.  K
    is formed after subtracting each matrix's largest logit, which cancels
    in every ratio.
    """
    lg = np.asarray(logits, dtype=np.float64)
    K = np.exp(lg - lg.max(axis=(-2, -1), keepdims=True))
    r = np.ones(K.shape[:-1])           # row scales  [..., n]
    c = np.ones(K.shape[:-2] + K.shape[-1:])   # column scales [..., n]
    for _ in range(iters):
        c = 1.0 / np.einsum("...i,...ij->...j", r, K)
        r = 1.0 / np.einsum("...ij,...j->...i", K, c)
    return r[..., :, None] * K * c[..., None, :]


def row_clamp(H):
    """Divide each row by max(row sum, 1).

    The post-Sinkhorn patch of xHC's appendix A as reported in the explainer
    ("Which constraint survives").  Reading: applied to xHC's k x k map only.
    """
    H = np.asarray(H, dtype=np.float64)
    rs = H.sum(axis=-1, keepdims=True)
    return H / np.maximum(rs, 1.0)


def round_to_bf16(x):
    """Round float64 values to the nearest bfloat16 (ties to even), as float64.

    bfloat16 keeps 8 significant bits and float32's exponent range; values
    here are far from its subnormal and overflow ranges.  Rounding is done
    directly from float64 (no float32 step, so no double rounding).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                 # x = m * 2^e, 0.5 <= |m| < 1
    q = np.rint(m * 256.0)             # 8 significant bits, ties to even
    return np.ldexp(q / 256.0, e)


def round_state(x, dtype):
    """Round once to the state dtype ('bf16' or 'f32'), returned as float64."""
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# mHC (dense N x N mixing)
# --------------------------------------------------------------------------

def mhc_pre(X, W_full, alpha, b_pre, b_post, b_res, iters=20):
    """mHC mapping generation and dense read for T tokens.

    X: [T, N, C].  W_full: [N*C, 2N + N^2], columns ordered pre | post | res
    (res row-major, entry (i, j) at column 2N + i*N + j).
    alpha = (alpha_pre, alpha_post, alpha_res).

    x' = RMSNorm(vec X); one projection gives the three logit groups;
    H_pre = sigmoid, H_post = 2*sigmoid, H_res = Sinkhorn; every logit is
    alpha * (x' W) + b (xHC paper, "Manifold-Constrained HC"; summary 3.1;
    explainer, "mHC: keep the mixing doubly stochastic").  The sublayer input
    is the H_pre-weighted sum of the N streams (summary 3.1).

    Returns inp [T, C], H_pre [T, N], H_post [T, N], H_res [T, N, N].
    """
    X = np.asarray(X, dtype=np.float64)
    T, N, C = X.shape
    a_pre, a_post, a_res = alpha
    x = X.reshape(T, N * C)
    z = rms_normalize(x) @ np.asarray(W_full, dtype=np.float64)
    h_pre = sigmoid(a_pre * z[:, :N] + np.asarray(b_pre))
    h_post = 2.0 * sigmoid(a_post * z[:, N:2 * N] + np.asarray(b_post))
    L = a_res * z[:, 2 * N:].reshape(T, N, N) + np.asarray(b_res).reshape(N, N)
    H_res = sinkhorn(L, iters)
    inp = np.einsum("tn,tnc->tc", h_pre, X)
    return inp, h_pre, h_post, H_res


def mhc_post(X, out, H_post, H_res):
    """mHC write-back and mix: row i of the new state is
    sum_j H_res[i, j] X_j + H_post[i] * out  (xHC paper, "Hyper-Connections"
    and "Information Supply Bottleneck"; summary 3.1-3.2).

    X: [T, N, C]; out: [T, C].  Returns the unrounded new state.
    """
    X = np.asarray(X, dtype=np.float64)
    out = np.asarray(out, dtype=np.float64)
    mixed = np.einsum("tij,tjc->tic", H_res, X)
    return mixed + H_post[:, :, None] * out[:, None, :]


# --------------------------------------------------------------------------
# xHC (router, dense read, sparse k x k mix, temporal augmentation)
# --------------------------------------------------------------------------

def xhc_router_logits(X, W_r):
    """z = LN(vec X) W_r, one logit per stream (summary 3.4.1; explainer,
    "What xHC changes").  No scale or bias.  Returns [T, N]."""
    X = np.asarray(X, dtype=np.float64)
    T, N, C = X.shape
    return ln_normalize(X.reshape(T, N * C)) @ np.asarray(W_r, dtype=np.float64)


def xhc_select(z, m, k):
    """Fixed-m plus routed top-(k-m) active set and router weights.

    Streams 0..m-1 are always active; the k-m streams of m..N-1 with the
    largest score join them (summary 3.4.1; explainer, "What xHC changes").
    The score is sigmoid(z); ranking uses z itself, which orders identically
    and does not saturate.  Reading: the routed streams are listed by
    descending score, ties to the lower stream index; p is 1 for fixed
    streams and the sigmoid score for routed ones.

    Returns I [T, k] (int64) and p [T, k].
    """
    z = np.asarray(z, dtype=np.float64)
    T, N = z.shape
    I = np.empty((T, k), dtype=np.int64)
    p = np.empty((T, k), dtype=np.float64)
    s = sigmoid(z)
    for t in range(T):
        I[t, :m] = np.arange(m)
        cand = list(range(m, N))
        # descending z, ties -> lower index
        cand.sort(key=lambda i: (-z[t, i], i))
        I[t, m:] = cand[: k - m]
    p[:, :m] = 1.0
    if k > m:
        p[:, m:] = np.take_along_axis(s, I[:, m:], axis=1)
    return I, p


def xhc_topk_margin(z, m, k):
    """Smallest gap between consecutive routed logits among the top k-m+1
    candidates: when it is positive the routed set and its order are unique.
    Returns +inf where no routed choice exists (k == m or N - m == k - m)."""
    z = np.asarray(z, dtype=np.float64)
    T, N = z.shape
    r = k - m
    if r == 0 or N - m <= r:
        return np.full(T, np.inf)
    zs = -np.sort(-z[:, m:], axis=1)[:, : r + 1]
    return np.min(zs[:, :-1] - zs[:, 1:], axis=1)


def xhc_pre(X, W_full, W_act, m, k, K_r, alpha, b_pre, b_res, b_post, iters=20):
    """xHC mapping generation and dense read for T tokens.

    X: [T, N, C].
    W_full: [N*C, 2N]; columns 0..N-1 are the router W_r, N..2N-1 the
        pre-map W_pre (rows stream-major).
    W_act: [k*C, k*k + k*K_r]; rows j*C + c for position j of the active
        list; columns 0..k^2-1 are W_res (entry (i, j) at i*k + j), then
        W_post (entry (j, r) at k^2 + j*K_r + r).
    alpha = (alpha_pre, alpha_res, alpha_post); the router has none.

    Steps (summary 3.4.1-3.4.3; xHC paper, "Mapping generation";
    explainer, "What xHC changes"):
      router: z = LN(vec X) W_r; I, p by fixed-m + routed top-(k-m);
      dense read: H_pre = sigmoid(alpha_pre * RMSNorm(vec X) W_pre + b_pre),
                  inp = sum_i H_pre[i] X_i over all N streams;
      active maps from X_act = X[I] (k x C), x~ = RMSNorm(vec X_act):
        H_res  = rowclamp(SK(alpha_res * mat_kxk(x~ W_res) + b_res)),
        H_post = 2 sigmoid(alpha_post * mat_kxK_r(x~ W_post) + b_post).

    Returns dict with inp [T,C], z [T,N], I [T,k], p [T,k], h_pre [T,N],
    h_res [T,k,k], h_post [T,k,K_r].
    """
    X = np.asarray(X, dtype=np.float64)
    W_full = np.asarray(W_full, dtype=np.float64)
    W_act = np.asarray(W_act, dtype=np.float64)
    T, N, C = X.shape
    a_pre, a_res, a_post = alpha
    x = X.reshape(T, N * C)

    z = ln_normalize(x) @ W_full[:, :N]
    I, p = xhc_select(z, m, k)

    h_pre = sigmoid(a_pre * (rms_normalize(x) @ W_full[:, N:2 * N]) + np.asarray(b_pre))
    # dense read: token t's input is the row vector h_pre[t] times its N x C state
    inp = np.matmul(h_pre[:, None, :], X)[:, 0, :]

    # the k active rows of each token, in list order, flattened to k*C
    x_act = X[np.arange(T)[:, None], I].reshape(T, k * C)
    proj = rms_normalize(x_act) @ W_act
    res_logits = proj[:, : k * k].reshape(T, k, k)
    post_logits = proj[:, k * k:].reshape(T, k, K_r)
    h_res = row_clamp(sinkhorn(a_res * res_logits + np.asarray(b_res).reshape(k, k), iters))
    # the post map ranges over (0, 2): twice a logistic function
    h_post = 2.0 * sigmoid(a_post * post_logits + np.asarray(b_post).reshape(k, K_r))
    return dict(inp=inp, z=z, I=I, p=p, h_pre=h_pre, h_res=h_res, h_post=h_post)


def causal_dwconv(out, w):
    """Causal depthwise 1-D convolution along the sequence.

    out: [B, S, C]; w: [kappa, C].  g[b, t] = sum_{i<kappa} w[i] * out[b, t-i],
    with out[b, t'] = 0 for t' < 0 (no history before a sequence starts, and
    nothing crosses batch items).  Reading: w[i] multiplies lag i, no bias
    (explainer, "What xHC changes"; summary 3.3).
    """
    out = np.asarray(out, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, S, C = out.shape
    g = np.zeros_like(out)
    for i in range(w.shape[0]):
        if i >= S:
            break
        g[:, i:, :] += w[i][None, None, :] * out[:, : S - i, :]
    return g


def gram_schmidt(comps, eps=EPS_MGS):
    """Modified Gram-Schmidt along C, token by token, without normalisation.

    comps: list [out, g_1, ..., g_r] of [..., C] arrays.  v_1 = out; for each
    g_j in order, the projection on each earlier v_i is removed one at a time
    from the running vector, u <- u - <u, v_i> / (<v_i, v_i> + eps) v_i, and
    the result is v_{j+1} (summary 3.3; explainer, "What xHC changes").
    """
    # Once component i is final, its projection is taken out of every later
    # component (each later one then sees the projections on v_1, v_2, ...
    # in that order, applied to what is left of it, as the recurrence asks).
    work = [np.array(c, dtype=np.float64) for c in comps]
    for i, v in enumerate(work):
        norm2 = np.einsum("...c,...c->...", v, v)[..., None] + eps
        for j in range(i + 1, len(work)):
            work[j] = work[j] - (np.einsum("...c,...c->...", work[j], v)[..., None] / norm2) * v
    return work


def xhc_write_basis(out, conv_ws, use_mgs=True, eps=EPS_MGS):
    """The K_r write components for every token: [B, S, K_r, C].

    Attention-type sublayers (no kernels): the single component out.
    MLP-type: out and one causal conv of out per kernel, Gram-Schmidt'ed
    (or left as they are when use_mgs is False, the Muon variant of the
    xHC paper's optimizer section).
    """
    out = np.asarray(out, dtype=np.float64)
    comps = [out] + [causal_dwconv(out, w) for w in conv_ws]
    if use_mgs and len(comps) > 1:
        comps = gram_schmidt(comps, eps)
    return np.stack(comps, axis=2)


def xhc_post(X, out, I, p, h_res, h_post, conv_ws=(), use_mgs=True, eps=EPS_MGS):
    """xHC sparse mix, gated write and scatter.

    X: [B*S, N, C]; out: [B, S, C]; I, p: [T, k]; h_res [T, k, k];
    h_post [T, k, K_r]; conv_ws: list of [kappa_j, C] (empty for attention).

    New active rows: X_act' = H_res X_act + diag(p) H_post [v_1; ...; v_K_r];
    they are scattered back to positions I and the other N-k streams are
    returned unchanged (summary 3.4.3; explainer, "What xHC changes").
    The router weight gates only the write, not the mix.

    Returns the unrounded new state [T, N, C].
    """
    X = np.asarray(X, dtype=np.float64)
    T, N, C = X.shape
    B, S, _ = np.shape(out)
    assert B * S == T
    V = xhc_write_basis(out, conv_ws, use_mgs, eps).reshape(T, -1, C)   # [T, K_r, C]
    Xa = np.take_along_axis(X, I[:, :, None], axis=1)                   # [T, k, C]
    new_a = np.einsum("tij,tjc->tic", h_res, Xa) + p[:, :, None] * np.einsum("tjr,trc->tjc", h_post, V)
    Xn = X.copy()
    np.put_along_axis(Xn, I[:, :, None], new_a, axis=1)
    return Xn


# --------------------------------------------------------------------------
# whole sublayers (pre, then the given sublayer output, then post)
# --------------------------------------------------------------------------

def mhc_sublayer(X, out, W_full, alpha, b_pre, b_post, b_res, iters=20, dtype="f64"):
    """One mHC sublayer; inp and the new state are rounded once to dtype."""
    inp, h_pre, h_post, H_res = mhc_pre(X, W_full, alpha, b_pre, b_post, b_res, iters)
    Xn = mhc_post(X, out.reshape(-1, np.shape(X)[2]), h_post, H_res)
    return dict(inp=round_state(inp, dtype), X=round_state(Xn, dtype),
                h_pre=h_pre, h_post=h_post, h_res=H_res)


def xhc_sublayer(X, out, W_full, W_act, m, k, conv_ws, alpha, b_pre, b_res, b_post,
                 iters=20, use_mgs=True, dtype="f64"):
    """One xHC sublayer; K_r = 1 + len(conv_ws).  out: [B, S, C]."""
    K_r = 1 + len(conv_ws)
    pre = xhc_pre(X, W_full, W_act, m, k, K_r, alpha, b_pre, b_res, b_post, iters)
    Xn = xhc_post(X, out, pre["I"], pre["p"], pre["h_res"], pre["h_post"], conv_ws, use_mgs)
    res = dict(pre)
    res["inp"] = round_state(pre["inp"], dtype)
    res["X"] = round_state(Xn, dtype)
    return res


def effective_mixing(I, h_res, N):
    """The full N x N mixing map of one xHC sublayer for each token: the
    k x k block on the active streams, identity elsewhere (explainer,
    "Which constraint survives").  Returns [T, N, N]."""
    T, k = I.shape
    E = np.tile(np.eye(N), (T, 1, 1))
    for t in range(T):
        idx = I[t]
        E[t][np.ix_(idx, idx)] = h_res[t]
    return E


def xhc_param_count(N, k, C, conv_kernels=(4, 8, 12)):
    """Parameters of one Transformer layer (attention + MLP sublayer) with
    the weight shapes used here: router N^2 C, pre-map N^2 C, residual map
    k^3 C, post map k^2 C (attention) or k^2 K_r C (MLP), conv sum(kappa) C
    (xHC paper, Appendix C).  Scales and biases are O(1) and not counted."""
    K_r = 1 + len(conv_kernels)
    attn = N * C * N + N * C * N + k * C * k * k + k * C * k
    mlp = N * C * N + N * C * N + k * C * k * k + k * C * k * K_r + sum(conv_kernels) * C
    return attn + mlp


def mhc_param_count(N, C):
    """Parameters of one Transformer layer of mHC: two sublayers, each
    with an N C x (2N + N^2) projection (xHC paper, Appendix C)."""
    return 2 * (N * C * (2 * N + N * N))


# --------------------------------------------------------------------------
# xHC-Flash: one routing and two pre-maps shared by an attention + MLP block
# --------------------------------------------------------------------------
#
# Readings (the pages' Algorithm 2 and the Appendix E.1 displays were lost in
# extraction; the prose of the xHC paper's "xHC-Flash" section, its Eqs. 17-19
# and the explainer's "What it costs" section fix the rest):
#   * routing (z, I, p) and both pre-maps come from the block-entry state;
#   * the attention sublayer has no residual map: its k active rows get
#     x + p_j H_post^A_j out_A (Eq. 18), with H_post^A (K_r = 1) generated,
#     like full xHC's active maps, from RMSNorm of the block-entry active rows;
#   * the MLP's active maps H_res (k x k, Sinkhorn + row clamp) and H_post^M
#     (k x K_r) are generated from the active rows as they stand after the
#     attention write, the pages naming only routing and pre-maps as fixed at
#     the block entry;
#   * the MLP base readout is a stored tensor of the state dtype that the
#     correction of Eq. 19 updates.

def xhcf_pre(X, W_full, W_post_attn, m, k, alpha, b_pre_attn, b_pre_mlp, b_post_attn):
    """xHC-Flash mapping generation and the two base readouts of a block.

    X: [T, N, C] block-entry state.
    W_full: [N*C, 3N]; columns 0..N-1 router W_r, N..2N-1 attention pre-map,
        2N..3N-1 MLP pre-map (rows stream-major).
    W_post_attn: [k*C, k]; row j*C + c for position j of the active list,
        column j gives the attention post-map logit of position j.
    alpha = (alpha_pre_attn, alpha_pre_mlp, alpha_post_attn); the router has
    no scale or bias.

    One projection of vec X gives the router and both pre-map logits; the two
    readouts are the pre-map weighted sums of all N streams (xHC paper,
    "xHC-Flash", Eq. 17, and "xHC-Flash kernel fusion").

    Returns dict with z [T,N], I [T,k], p [T,k], h_pre_attn [T,N],
    h_pre_mlp [T,N], inp_attn [T,C], inp_mlp [T,C] (base readout, unrounded),
    h_post_attn [T,k].
    """
    X = np.asarray(X, dtype=np.float64)
    W_full = np.asarray(W_full, dtype=np.float64)
    T, N, C = X.shape
    a_pa, a_pm, a_po = alpha
    x = X.reshape(T, N * C)
    z = ln_normalize(x) @ W_full[:, :N]
    I, p = xhc_select(z, m, k)
    xr = rms_normalize(x)
    h_pa = sigmoid(a_pa * (xr @ W_full[:, N:2 * N]) + np.asarray(b_pre_attn))
    h_pm = sigmoid(a_pm * (xr @ W_full[:, 2 * N:3 * N]) + np.asarray(b_pre_mlp))
    inp_a = np.einsum("tn,tnc->tc", h_pa, X)
    inp_m = np.einsum("tn,tnc->tc", h_pm, X)
    Xa = np.take_along_axis(X, I[:, :, None], axis=1)
    la = rms_normalize(Xa.reshape(T, k * C)) @ np.asarray(W_post_attn, dtype=np.float64)
    h_po = 2.0 * sigmoid(a_po * la + np.asarray(b_post_attn))
    return dict(z=z, I=I, p=p, h_pre_attn=h_pa, h_pre_mlp=h_pm, inp_attn=inp_a, inp_mlp=inp_m,
                h_post_attn=h_po)


def xhcf_attn_write(X, out_a, I, p, h_post_attn):
    """Attention write-back of xHC-Flash: no residual mixing, each active row
    gains p_j H_post^A_j out_A; the other streams are untouched (xHC paper,
    "xHC-Flash", Eq. 18).  X: [T, N, C]; out_a: [T, C].  Returns the
    unrounded new state."""
    X = np.asarray(X, dtype=np.float64)
    out_a = np.asarray(out_a, dtype=np.float64).reshape(X.shape[0], X.shape[2])
    Xa = np.take_along_axis(X, I[:, :, None], axis=1)
    new_a = Xa + (p * h_post_attn)[:, :, None] * out_a[:, None, :]
    Xn = X.copy()
    np.put_along_axis(Xn, I[:, :, None], new_a, axis=1)
    return Xn


def xhcf_mlp_input(inp_mlp, out_a, I, p, h_pre_mlp, h_post_attn):
    """The MLP input from its base readout, corrected for the attention write
    by one token-wise scalar: inp_M + a out_A with
    a = sum_j H_pre^M[I_j] p_j H_post^A_j (xHC paper, "xHC-Flash", Eq. 19).
    Returns (input [T, C] unrounded, a [T])."""
    inp_mlp = np.asarray(inp_mlp, dtype=np.float64)
    out_a = np.asarray(out_a, dtype=np.float64).reshape(inp_mlp.shape)
    hpI = np.take_along_axis(np.asarray(h_pre_mlp, dtype=np.float64), I, axis=1)
    a = np.sum(hpI * p * h_post_attn, axis=1)
    return inp_mlp + a[:, None] * out_a, a


def xhcf_mlp_maps(X1, I, W_act_mlp, K_r, alpha_res, alpha_post, b_res, b_post, iters=20):
    """The MLP's active maps from the active rows after the attention write:
    x~ = RMSNorm(vec X1[I]); H_res = rowclamp(SK(alpha_res mat_kxk(x~ W_res)
    + b_res)), H_post = 2 sigmoid(alpha_post mat_kxK_r(x~ W_post) + b_post),
    the same generation as full xHC's (W_act_mlp: [k*C, k^2 + k K_r], columns
    W_res then W_post).  Returns (h_res [T,k,k], h_post [T,k,K_r])."""
    X1 = np.asarray(X1, dtype=np.float64)
    T, N, C = X1.shape
    k = I.shape[1]
    Xa = np.take_along_axis(X1, I[:, :, None], axis=1)
    la = rms_normalize(Xa.reshape(T, k * C)) @ np.asarray(W_act_mlp, dtype=np.float64)
    L = alpha_res * la[:, : k * k].reshape(T, k, k) + np.asarray(b_res).reshape(k, k)
    h_res = row_clamp(sinkhorn(L, iters))
    h_post = 2.0 * sigmoid(alpha_post * la[:, k * k:].reshape(T, k, K_r) + np.asarray(b_post).reshape(k, K_r))
    return h_res, h_post


def xhcf_block(X, out_a, out_m, W_full, W_post_attn, W_act_mlp, m, k, conv_ws, alpha, b_pre_attn,
               b_pre_mlp, b_post_attn, b_res, b_post_mlp, iters=20, use_mgs=True, dtype="f64"):
    """One xHC-Flash block (attention, then MLP) on T = B*S tokens.

    X: [T, N, C]; out_a, out_m: [B, S, C] (the two sublayers' outputs, given).
    alpha = (pre_attn, pre_mlp, post_attn, res, post_mlp).
    Stored tensors are rounded once to dtype where the block stores them: the
    attention input, the MLP base readout, the state after the attention
    write, the corrected MLP input and the state after the MLP write.  The
    MLP write is full xHC's (temporal augmentation, Gram-Schmidt, k x k mix).
    """
    a_pa, a_pm, a_po, a_res, a_pm2 = alpha
    K_r = 1 + len(conv_ws)
    pre = xhcf_pre(X, W_full, W_post_attn, m, k, (a_pa, a_pm, a_po), b_pre_attn, b_pre_mlp, b_post_attn)
    I, p = pre["I"], pre["p"]
    inp_a = round_state(pre["inp_attn"], dtype)
    base_m = round_state(pre["inp_mlp"], dtype)
    X1 = round_state(xhcf_attn_write(X, out_a, I, p, pre["h_post_attn"]), dtype)
    inp_m, a = xhcf_mlp_input(base_m, out_a, I, p, pre["h_pre_mlp"], pre["h_post_attn"])
    h_res, h_post = xhcf_mlp_maps(X1, I, W_act_mlp, K_r, a_res, a_pm2, b_res, b_post_mlp, iters)
    X2 = xhc_post(X1, out_m, I, p, h_res, h_post, conv_ws, use_mgs)
    res = dict(pre)
    res.update(inp_attn=inp_a, inp_mlp_base=base_m, X1=X1, inp_mlp=round_state(inp_m, dtype), alpha=a,
               h_res=h_res, h_post=h_post, X=round_state(X2, dtype))
    return res


# --------------------------------------------------------------------------
# single-token decode: the MLP-type write with the conv history in a ring
# --------------------------------------------------------------------------

RING = 12   # slots: the current output and the 11 lags of the longest kernel


def xhc_decode_post(X, out, ring, steps, I, p, h_res, h_post, conv_ws, use_mgs=True, eps=EPS_MGS):
    """One decode step of xHC's MLP-type write for B sequences, each adding
    one token.  The causal convolutions need the sublayer outputs of the 11
    tokens before the new one in its sequence; a decoder keeps them in a ring
    (the pages' prefill computes the same convolutions over the whole
    sequence: summary 3.3; explainer, "What xHC changes").

    X: [B, N, C] the new tokens' states; out: [B, C] their sublayer outputs;
    ring: [B, RING, C], slot s % RING holds the output of position s of the
    sequence; steps: [B] position of the new token (earlier positions are
    zero history when they do not exist).  I, p, h_res, h_post as xhc_post.

    Returns (new state [B, N, C] unrounded, new ring with the new output in
    slot steps % RING).
    """
    X = np.asarray(X, dtype=np.float64)
    out = np.asarray(out, dtype=np.float64)
    ring = np.asarray(ring, dtype=np.float64)
    B, N, C = X.shape
    hist = np.zeros((B, RING, C))          # hist[b, i] = out of position steps[b] - i
    hist[:, 0] = out
    for b in range(B):
        for i in range(1, RING):
            if i <= steps[b]:
                hist[b, i] = ring[b, (steps[b] - i) % RING]
    comps = [out] + [np.einsum("ic,bic->bc", np.asarray(w, dtype=np.float64), hist[:, : len(w)]) for w in conv_ws]
    if use_mgs and len(comps) > 1:
        comps = gram_schmidt(comps, eps)
    V = np.stack(comps, axis=1)                                         # [B, K_r, C]
    Xa = np.take_along_axis(X, I[:, :, None], axis=1)
    new_a = np.einsum("tij,tjc->tic", h_res, Xa) + p[:, :, None] * np.einsum("tjr,trc->tjc", h_post, V)
    Xn = X.copy()
    np.put_along_axis(Xn, I[:, :, None], new_a, axis=1)
    ring_n = ring.copy()
    for b in range(B):
        ring_n[b, steps[b] % RING] = out[b]
    return Xn, ring_n


# --------------------------------------------------------------------------
# xHC-Flash-4sub: one routing and four pre-maps shared by two blocks
# --------------------------------------------------------------------------
#
# Readings (the xHC paper's "Four-sublayer extension" paragraph and Appendix
# E.2; the E.2 displays were lost in extraction):
#   * routing (z, I, p) and the four pre-maps H_pre^q, q = 1..4, come from the
#     group-entry state X^(0), from one projection onto [W_r | W_pre^1..4];
#   * the input of sublayer q is the non-active base sum_{i not in I}
#     H_pre^q_i x_i^(0) plus sum_j H_pre^q[I_j] x_act_j^(q), the active rows as
#     they stand before sublayer q (for q = 1 this is the plain dense read);
#   * sublayers 1-3 write only the active rows, without residual mixing:
#     x_act_j += p_j sum_r H_post^q_jr v_r^(q) (K_r = 1 after attention, the
#     temporal basis after the first MLP); the final MLP mixes with H_res and
#     writes as full xHC does;
#   * each sublayer's active-side maps (H_post^q, and H_res at the final MLP)
#     come from RMSNorm of the active rows before that sublayer;
#   * stored tensors (the bases, each input, the state after each write) are
#     rounded to the state dtype where they are stored.

def xhcf4_pre(X, W_full, m, k, alpha_pre, b_pre):
    """Group entry of xHC-Flash-4sub.  X: [T, N, C]; W_full: [N*C, 5N] with
    columns router | pre^1 | pre^2 | pre^3 | pre^4; alpha_pre, b_pre: four
    scales and four [N] biases.  Returns z, I, p, h_pre [4][T, N], the first
    sublayer's input (dense read with H_pre^1) and the non-active bases of
    sublayers 2..4 [3][T, C] (xHC paper, "Four-sublayer extension";
    Appendix E.2)."""
    X = np.asarray(X, dtype=np.float64)
    W_full = np.asarray(W_full, dtype=np.float64)
    T, N, C = X.shape
    x = X.reshape(T, N * C)
    z = ln_normalize(x) @ W_full[:, :N]
    I, p = xhc_select(z, m, k)
    xr = rms_normalize(x)
    h_pre = [sigmoid(alpha_pre[q] * (xr @ W_full[:, (q + 1) * N:(q + 2) * N]) + np.asarray(b_pre[q]))
             for q in range(4)]
    inactive = np.ones((T, N))
    np.put_along_axis(inactive, I, 0.0, axis=1)
    inp1 = np.einsum("tn,tnc->tc", h_pre[0], X)
    bases = [np.einsum("tn,tnc->tc", h_pre[q] * inactive, X) for q in (1, 2, 3)]
    return dict(z=z, I=I, p=p, h_pre=h_pre, inp1=inp1, bases=bases)


def xhcf4_input(base, Xa, I, h_pre_q):
    """Input of a later sublayer: its non-active base plus its pre-map applied
    to the current active rows Xa [T, k, C] (reading of Appendix E.2)."""
    hI = np.take_along_axis(np.asarray(h_pre_q, dtype=np.float64), I, axis=1)
    return np.asarray(base, dtype=np.float64) + np.einsum("tj,tjc->tc", hI, np.asarray(Xa, dtype=np.float64))


def xhcf4_post_map(Xa, W_post, K_r, alpha_post, b_post):
    """H_post of an unmixed sublayer from its active rows: 2 sigmoid(alpha
    RMSNorm(vec Xa) W_post + b), W_post [k*C, k*K_r] (entry (j, r) at column
    j*K_r + r).  Returns [T, k, K_r]."""
    Xa = np.asarray(Xa, dtype=np.float64)
    T, k, C = Xa.shape
    la = rms_normalize(Xa.reshape(T, k * C)) @ np.asarray(W_post, dtype=np.float64)
    return 2.0 * sigmoid(alpha_post * la.reshape(T, k, K_r) + np.asarray(b_post).reshape(k, K_r))


def xhcf4_group(X, outs, W_full, W_posts, W_act_last, m, k, conv_ws, alpha, b, iters=20, use_mgs=True,
                dtype="f64"):
    """Two blocks (attention, MLP, attention, MLP) of xHC-Flash-4sub.

    X: [T, N, C]; outs: four [B, S, C] sublayer outputs; W_full [N*C, 5N];
    W_posts: [W_post^1 [k*C, k], W_post^2 [k*C, k*K_r], W_post^3 [k*C, k]];
    W_act_last: [k*C, k*k + k*K_r] (W_res, then W_post^4); conv_ws: kernels of
    the two MLP sublayers (lists of [kappa, C]); alpha = dict(pre=(4), post=(4),
    res); b = dict(pre=[4 x N], post=[4 arrays], res).

    Returns the group's inputs [4][T, C], the state after each sublayer
    [4][T, N, C], the maps and the routing."""
    X = np.asarray(X, dtype=np.float64)
    T, N, C = X.shape
    pre = xhcf4_pre(X, W_full, m, k, alpha["pre"], b["pre"])
    I, p = pre["I"], pre["p"]
    bases = [round_state(bq, dtype) for bq in pre["bases"]]
    inputs = [round_state(pre["inp1"], dtype)]
    states, maps = [], []
    Xc = X.copy()
    for q in range(4):
        Xa = np.take_along_axis(Xc, I[:, :, None], axis=1)
        if q > 0:
            inputs.append(round_state(xhcf4_input(bases[q - 1], Xa, I, pre["h_pre"][q]), dtype))
        mlp = q % 2 == 1
        K_r = 1 + len(conv_ws[q // 2]) if mlp else 1
        if q < 3:
            h_post = xhcf4_post_map(Xa, W_posts[q], K_r, alpha["post"][q], b["post"][q])
            h_res = np.tile(np.eye(k), (T, 1, 1))
        else:
            h_res, h_post = xhcf_mlp_maps(Xc, I, W_act_last, K_r, alpha["res"], alpha["post"][3], b["res"],
                                          b["post"][3], iters)
        convs = conv_ws[q // 2] if mlp else []
        Xc = round_state(xhc_post(Xc, outs[q], I, p, h_res, h_post, convs, use_mgs), dtype)
        states.append(Xc)
        maps.append(dict(h_post=h_post, h_res=h_res))
    return dict(z=pre["z"], I=I, p=p, h_pre=pre["h_pre"], inputs=inputs, bases=bases, states=states, maps=maps)
