/*
 * libxhc — hyper-connection residual-stream layer (mHC and xHC) for one
 * AMD Instinct MI355X (gfx950) GPU.
 *
 * One sublayer of a multi-stream residual network keeps, per token, a state
 * X in R^{N x C} (N streams of C channels).  Around the sublayer F (attention
 * or MLP, not part of this library) two calls run:
 *
 *   *_pre  : mapping generation from the state and the dense read that forms
 *            F's input  (xHC paper "xHC: Expanded Hyper-Connections",
 *            paragraphs "Mapping generation" and "Mapping application");
 *   *_post : after F, the write-back of F's output and the stream mix,
 *            in place on X (same paragraphs; summary "小红书xHC：时序特征增强
 *            + 稀疏写回", sections 3.1 and 3.4.3).
 *
 * mHC (dense): H_pre = sigmoid, H_post = 2 sigmoid and H_res = 20-step
 * Sinkhorn-Knopp of one projection of RMSNorm(vec X) (xHC paper,
 * "Manifold-Constrained HC"; explainer "xHC: sixteen residual streams, four
 * written at a time", section "mHC: keep the mixing doubly stochastic").
 *
 * xHC (sparse): a sigmoid router over LayerNorm(vec X) picks m fixed and
 * k-m routed active streams per token; the read stays dense over all N
 * streams; only the k active streams are mixed (k x k Sinkhorn, then each
 * row divided by max(row sum, 1)) and written; after MLP-type sublayers the
 * write basis is F's output plus three causal depthwise convolutions of it
 * (kernel sizes 4, 8, 12) orthogonalised by modified Gram-Schmidt along C
 * (explainer, "What xHC changes" and "Which constraint survives"; summary
 * 3.3-3.4).
 *
 * Conventions
 *   - Tokens: T = batch * seq, flat index t = b * seq + s (batch-major).
 *     The causal convolutions run along s inside one batch item.
 *   - X: [T][N][C], out and inp: [T][C], all of the state dtype (cfg.dtype),
 *     row-major, device memory, 16-byte aligned.
 *   - vec X is stream-major: element (i, c) is row i*C + c of the
 *     full-state projection weight.
 *   - Every pointer in these calls is a device pointer unless it is the
 *     config or weights struct itself (host memory, read during the call).
 *   - The caller owns every buffer.  No call allocates memory.  Between
 *     calls the library keeps only cached device properties (the number of
 *     compute units) and, once xhc_post_noalloc has run on a device, the
 *     address of that device's scratch array.
 *   - Calls are asynchronous on `stream` and stream-ordered: *_pre, then F,
 *     then *_post on the same workspace.  Calls that share a workspace must
 *     not overlap.
 *   - Arguments are checked before anything is launched; a check that fails
 *     returns XHC_ERR_INVALID_ARG or XHC_ERR_UNSUPPORTED and launches
 *     nothing.  A launch error returns XHC_ERR_HIP.  xhc_last_error() gives
 *     the message (per host thread).  No C++ exception crosses this ABI.
 *   - Results are deterministic: fixed reduction orders, no float atomics.
 *   - T == 0 is valid and launches nothing.
 */
#ifndef XHC_H
#define XHC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same object as HIP's hipStream_t; NULL selects the default stream. */
typedef struct ihipStream_t* xhc_stream_t;

typedef enum {
  XHC_OK = 0,
  XHC_ERR_INVALID_ARG = 1,
  XHC_ERR_UNSUPPORTED = 2,
  XHC_ERR_HIP = 3
} xhc_status;

typedef enum { XHC_F32 = 0, XHC_BF16 = 1 } xhc_dtype;

/* Layer shape and options (host struct, read during the call). */
typedef struct {
  int32_t n_streams;      /* N: 1..16 (mHC: 1, 2, 4, 8, 16; xHC: see below) */
  int32_t k_active;       /* k: active streams (xHC only) */
  int32_t m_fixed;        /* m: always-active streams 0..m-1, 0 <= m <= k (xHC only) */
  int32_t channels;       /* C: multiple of 32 */
  int32_t batch;          /* B >= 0 */
  int32_t seq;            /* S >= 0 */
  int32_t n_convs;        /* 0: attention-type, K_r = 1; 3: MLP-type, K_r = 4 (xHC only) */
  int32_t conv_kernel[3]; /* kernel sizes when n_convs == 3: {4, 8, 12} */
  int32_t use_mgs;        /* 1: Gram-Schmidt the write basis; 0: use it as is */
  int32_t sinkhorn_iters; /* 0..1000, 20 in the pages */
  int32_t dtype;          /* xhc_dtype of X, out, inp and projection weights */
  float eps_norm;         /* RMSNorm / LayerNorm epsilon, 1e-6 in the pages */
  float eps_mgs;          /* Gram-Schmidt epsilon on <v, v>, 1e-6 */
} xhc_config;

/* Weights of one sublayer (host struct holding device pointers). */
typedef struct {
  /* xHC: [N*C][2N], columns 0..N-1 router W_r, N..2N-1 pre-map W_pre.
   * mHC: [N*C][2N + N*N], columns pre | post | res (res entry (i, j) at
   *      column 2N + i*N + j).  State dtype, row-major. */
  const void* w_full;
  /* xHC: [k*C][k*k + k*K_r]; row j*C + c multiplies channel c of the j-th
   * active stream (order of the active list); columns 0..k^2-1 W_res
   * (entry (i, j) at i*k + j), then W_post (entry (j, r) at k^2 + j*K_r + r).
   * State dtype.  mHC: unused (may be NULL). */
  const void* w_act;
  /* xHC MLP-type: [4 + 8 + 12][C] float; row off_j + i holds kernel j's
   * weight for lag i (it multiplies out[t - i]).  NULL when n_convs == 0. */
  const float* conv_w;
  /* Biases, float.  xHC: b_pre [N], b_res [k*k], b_post [k*K_r].
   *                 mHC: b_pre [N], b_res [N*N], b_post [N]. */
  const float* b_pre;
  const float* b_res;
  const float* b_post;
  float alpha_pre, alpha_res, alpha_post;  /* learnable scales */
} xhc_weights;

/* Byte offsets of the public arrays inside a workspace; fields that do not
 * apply are SIZE_MAX.  All arrays are float except idx (int32). */
typedef struct {
  size_t idx;       /* xHC: [T][k] active streams: 0..m-1, then routed by descending score */
  size_t p;         /* xHC: [T][k] router weights (1 for fixed streams) */
  size_t h_pre;     /* [T][N] */
  size_t h_res;     /* xHC: [T][k][k]; mHC: [T][N][N] */
  size_t h_post;    /* xHC: [T][k][K_r]; mHC: [T][N] */
  size_t z_router;  /* xHC: [T][N] router logits */
  size_t status;    /* xHC: one int32, 0 after a normal xhc_pre; 1 if a wait between
                       workgroups of the one-pass kernel gave up (results invalid) */
  size_t total;     /* bytes the caller must allocate (0 when T == 0) */
} xhc_ws_layout;

/* Workspace needed by xhc_pre / xhc_post (resp. mhc_pre / mhc_post) for
 * this config; 0 for an invalid config or T == 0. */
size_t xhc_workspace_bytes(const xhc_config* cfg);
size_t mhc_workspace_bytes(const xhc_config* cfg);
xhc_status xhc_workspace_layout(const xhc_config* cfg, xhc_ws_layout* out);
xhc_status mhc_workspace_layout(const xhc_config* cfg, xhc_ws_layout* out);

/* xHC before the sublayer: router logits, active set I and weights p, H_pre,
 * dense read inp = sum_i H_pre[i] X_i (all N streams), and the active maps
 * H_res, H_post from RMSNorm(vec X[I]).  X: [T][N][C] (read only);
 * inp: [T][C] (written); ws: xhc_workspace_bytes(cfg) bytes (written).
 * (xHC paper, "Mapping generation"; summary 3.4.1-3.4.3.)
 * Supported (N, k): (16, 4), (16, 2), (8, 4), (4, 4), (1, 1). */
xhc_status xhc_pre(const xhc_config* cfg, const xhc_weights* w,
                   const void* X, void* inp, void* ws, xhc_stream_t stream);

/* xHC after the sublayer: for MLP-type configs the causal convolutions of
 * out and Gram-Schmidt; then for each token the k active rows become
 * H_res X_act + diag(p) H_post [v_1..v_K_r], written in place; the other
 * N - k rows are not touched.  X: [T][N][C] (in place); out: [T][C];
 * ws: the workspace filled by xhc_pre (also used as scratch).
 * (xHC paper, "Mapping application" and "Temporal feature augmentation";
 * summary 3.3, 3.4.3.) */
xhc_status xhc_post(const xhc_config* cfg, const xhc_weights* w,
                    void* X, const void* out, void* ws, xhc_stream_t stream);

/* xhc_post for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same write, bit for bit, with the workspace read only.  The only memory
 * the write needs beyond X, out and the maps in ws, the Gram partials of an
 * MLP-type write with Gram-Schmidt (80 * ceil(C / 1024) * T bytes), lives in
 * an array inside the library: XHC_NOALLOC_SCRATCH_BYTES bytes per GPU, held
 * from the first call on that GPU until the process ends.  A call that would
 * need more returns XHC_ERR_INVALID_ARG and launches nothing.  The call
 * allocates nothing.  Calls that overlap on one GPU share that array and
 * race: order them (one stream, or events).
 * X: [T][N][C] (in place); out: [T][C]; ws: the workspace filled by xhc_pre
 * (read only). */
#define XHC_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
xhc_status xhc_post_noalloc(const xhc_config* cfg, const xhc_weights* w,
                            void* X, const void* out, const void* ws, xhc_stream_t stream);

/* mHC before the sublayer: H_pre, H_post, H_res (Sinkhorn, no clamp) from
 * RMSNorm(vec X), and inp = sum_i H_pre[i] X_i.
 * (xHC paper, "Manifold-Constrained HC"; summary 3.1.) */
xhc_status mhc_pre(const xhc_config* cfg, const xhc_weights* w,
                   const void* X, void* inp, void* ws, xhc_stream_t stream);

/* mHC after the sublayer: X <- H_res X + H_post out^T for all N rows, in
 * place.  (xHC paper, "Hyper-Connections"; summary 3.1-3.2.) */
xhc_status mhc_post(const xhc_config* cfg, const xhc_weights* w,
                    void* X, const void* out, void* ws, xhc_stream_t stream);

/* ---------------------------------------------------------------------------
 * xHC sublayers in a chain.  The mapping generation of a sublayer is a linear
 * contraction of vec X, and a sublayer changes only its k active rows, so the
 * routing of sublayer l+1 (router logits, active set, router weights, H_pre)
 * can be accumulated while sublayer l runs: the rows sublayer l leaves alone
 * are contracted while xhc_pre_chained reads the state anyway, the k
 * rewritten rows after xhc_post_chained has written them.  Results are those
 * of xhc_pre / xhc_post up to rounding order (xHC paper "xHC: Expanded
 * Hyper-Connections", paragraphs "Mapping generation" and "Mapping
 * application"; explainer "xHC: sixteen residual streams, four written at a
 * time", section "What xHC changes").
 *
 * Use, for sublayers 0..L-1 with configs cfg[l], weights w[l] and two
 * workspaces used in turn (ws[l % 2], each xhc_workspace_bytes(cfg[l]) large
 * for the layer it serves):
 *
 *   xhc_route(cfg[0], w[0], X, ws[0])
 *   for l: xhc_pre_chained (cfg[l], w[l], cfg[l+1], w[l+1], X, inp, ws[l%2], ws[(l+1)%2])
 *          F
 *          xhc_post_chained(cfg[l], w[l], cfg[l+1], w[l+1], X, out, ws[l%2], ws[(l+1)%2])
 *
 * with cfg_next, w_next and ws_next NULL for the last sublayer.  cfg and
 * cfg_next must agree in N, k, m, C, batch, seq and dtype (n_convs may
 * differ).  The public arrays of a workspace after its layer's
 * xhc_pre_chained are those xhc_pre writes (status stays 0).
 * ------------------------------------------------------------------------- */

/* Routing of the state X for the sublayer (cfg, w): router logits, active set
 * and router weights, H_pre, into ws.  X: [T][N][C] (read only). */
xhc_status xhc_route(const xhc_config* cfg, const xhc_weights* w, const void* X, void* ws, xhc_stream_t stream);

/* xhc_pre for a sublayer whose routing is already in ws (from xhc_route or
 * the previous sublayer's xhc_post_chained): inp, H_res and H_post.  With a
 * next sublayer, also its partial routing over the rows this sublayer does
 * not write, into ws_next.  X is read once. */
xhc_status xhc_pre_chained(const xhc_config* cfg, const xhc_weights* w, const xhc_config* cfg_next,
                           const xhc_weights* w_next, const void* X, void* inp, void* ws, void* ws_next,
                           xhc_stream_t stream);

/* xhc_post, then (with a next sublayer) the rewritten rows' share of the
 * next sublayer's routing and that routing itself, into ws_next (the
 * workspace given to this sublayer's xhc_pre_chained as ws_next). */
xhc_status xhc_post_chained(const xhc_config* cfg, const xhc_weights* w, const xhc_config* cfg_next,
                            const xhc_weights* w_next, void* X, const void* out, void* ws, void* ws_next,
                            xhc_stream_t stream);

/* Single-token decode of an MLP-type sublayer's write.  cfg.seq must be 1:
 * each of the cfg.batch tokens is the newest token of its own sequence, and
 * the causal convolutions take its 11 earlier outputs from a ring instead of
 * from neighbouring tokens (the convolutions are those of xhc_post: explainer
 * "xHC: sixteen residual streams, four written at a time", section "What xHC
 * changes"; summary 3.3).  n_convs must be 3 (an attention-type sublayer has
 * no history: use xhc_post).
 *   X:          [B][N][C], the new tokens' states, written in place (k rows)
 *   out:        [B][C], the sublayer outputs of the new tokens
 *   conv_state: [B][12][C] of the state dtype, caller-owned: slot s % 12 of
 *               sequence b holds the output of its position s.  Lag i of
 *               the new token (position steps[b]) is read from slot
 *               (steps[b] - i) % 12 when i <= steps[b] and is zero before
 *               the sequence start; the new output is then stored to slot
 *               steps[b] % 12.  Contents need no clearing between sequences.
 *   steps:      [B] int32, device: position of each new token in its
 *               sequence (read only; the caller advances it)
 *   ws:         the workspace xhc_pre filled for the same cfg
 * The other rows of X are not touched. */
xhc_status xhc_post_decode(const xhc_config* cfg, const xhc_weights* w, void* X, const void* out, void* conv_state,
                           const int32_t* steps, void* ws, xhc_stream_t stream);

/* ---------------------------------------------------------------------------
 * xHC-Flash: one attention + MLP block sharing a single routing decision
 * (xHC paper "xHC: Expanded Hyper-Connections", section "xHC-Flash", Eqs.
 * 17-19 and Appendix E.1; explainer "xHC: sixteen residual streams, four
 * written at a time", section "What it costs").
 *
 * From the block-entry state X one projection gives the router logits and
 * two separate pre-maps; the active set I and router weights p are shared by
 * both sublayers.  The attention sublayer has no residual map: each active
 * row gains p_j H_post^Attn_j out_Attn (Eq. 18).  The MLP input is the MLP
 * pre-map's readout of the block-entry state corrected by one scalar per
 * token, inp_M + a out_Attn with a = sum_j H_pre^MLP[I_j] p_j H_post^Attn_j
 * (Eq. 19), which equals the MLP pre-map applied to the state after the
 * attention write.  The MLP side is full xHC's: H_res (k x k, Sinkhorn + row
 * clamp) and H_post^MLP (k x K_r) from RMSNorm of the active rows after the
 * attention write, temporal augmentation and Gram-Schmidt when n_convs == 3,
 * and the k x k mix with the gated write.
 *
 * Per block, on one stream and one workspace:
 *
 *   xhcf_pre (cfg, w, X, inp_attn, inp_mlp, ws)   inp_mlp = base readout
 *   out_attn = Attention(inp_attn)
 *   xhcf_mid (cfg, w, X, out_attn, inp_mlp, ws)   X written, inp_mlp corrected
 *   out_mlp = MLP(inp_mlp)
 *   xhcf_post(cfg, w, X, out_mlp, ws)             X written
 *
 * cfg is the block's config: N, k, m, C, batch, seq, dtype, sinkhorn_iters,
 * eps; n_convs (0 or 3) and use_mgs describe the MLP sublayer.  Supported
 * (N, k): (16, 4), (8, 4), (4, 4), (1, 1).  Every buffer is caller-owned
 * device memory of the state dtype ([T][N][C] state, [T][C] inputs and
 * outputs), 16-byte aligned; X must not alias any other argument.
 * ------------------------------------------------------------------------- */

/* Weights of one xHC-Flash block (host struct holding device pointers). */
typedef struct {
  /* [N*C][3N], state dtype: columns 0..N-1 router W_r, N..2N-1 attention
   * pre-map, 2N..3N-1 MLP pre-map (rows stream-major, i*C + c). */
  const void* w_full;
  /* [k*C][k], state dtype: attention post-map; row j*C + c multiplies channel
   * c of the j-th active stream, column j is position j's logit. */
  const void* w_post_attn;
  /* [k*C][k*k + k*K_r], state dtype: MLP residual map W_res (entry (i, j) at
   * column i*k + j), then MLP post-map (entry (j, r) at k^2 + j*K_r + r). */
  const void* w_act_mlp;
  /* [4 + 8 + 12][C] float, lag-major (as xhc_weights.conv_w); NULL when
   * n_convs == 0. */
  const float* conv_w;
  /* float biases: [N], [N], [k], [k*k], [k*K_r] */
  const float *b_pre_attn, *b_pre_mlp, *b_post_attn, *b_res, *b_post_mlp;
  float alpha_pre_attn, alpha_pre_mlp, alpha_post_attn, alpha_res, alpha_post_mlp;
} xhcf_weights;

/* Byte offsets of the public arrays of an xHC-Flash workspace (float unless
 * noted).  After xhcf_pre: idx, p, h_pre_attn, h_pre_mlp, h_post_attn,
 * z_router.  After xhcf_mid: h_res, h_post_mlp (the MLP maps). */
typedef struct {
  size_t idx;          /* [T][k] int32: 0..m-1, then routed streams by descending logit */
  size_t p;            /* [T][k] router weights (1 for fixed streams) */
  size_t h_pre_attn;   /* [T][N] */
  size_t h_pre_mlp;    /* [T][N] */
  size_t h_post_attn;  /* [T][k] */
  size_t h_res;        /* [T][k][k] */
  size_t h_post_mlp;   /* [T][k][K_r] */
  size_t z_router;     /* [T][N] router logits */
  size_t total;        /* bytes the caller must allocate (0 when T == 0) */
} xhcf_ws_layout;

size_t xhcf_workspace_bytes(const xhc_config* cfg);
xhc_status xhcf_workspace_layout(const xhc_config* cfg, xhcf_ws_layout* out);

/* Block entry: routing, both pre-maps and their readouts of X (read only),
 * and the attention post-map.  inp_attn, inp_mlp: [T][C] (written; inp_mlp
 * is the MLP pre-map's readout of X, corrected later by xhcf_mid). */
xhc_status xhcf_pre(const xhc_config* cfg, const xhcf_weights* w, const void* X, void* inp_attn, void* inp_mlp,
                    void* ws, xhc_stream_t stream);

/* After the attention sublayer: the active rows of X gain p_j H_post^Attn_j
 * out_attn (in place), inp_mlp gains a out_attn (in place), and the MLP maps
 * H_res, H_post^MLP are generated from the rewritten active rows. */
xhc_status xhcf_mid(const xhc_config* cfg, const xhcf_weights* w, void* X, const void* out_attn, void* inp_mlp,
                    void* ws, xhc_stream_t stream);

/* After the MLP sublayer: full xHC's write (temporal augmentation and
 * Gram-Schmidt when n_convs == 3), in place on the k active rows of X. */
xhc_status xhcf_post(const xhc_config* cfg, const xhcf_weights* w, void* X, const void* out_mlp, void* ws,
                     xhc_stream_t stream);

/* ---------------------------------------------------------------------------
 * xHC-Flash-4sub: two blocks (attention, MLP, attention, MLP) sharing one
 * routing decision (xHC paper "xHC: Expanded Hyper-Connections", section
 * "xHC-Flash", paragraph "Four-sublayer extension", and Appendix E.2).
 *
 * From the group-entry state X one projection gives the router logits and
 * four separate pre-maps; the active set I and router weights p are shared by
 * the four sublayers.  The input of sublayer q is the non-active base
 * sum_{i not in I} H_pre^q_i x_i of the group-entry state plus
 * sum_j H_pre^q[I_j] x_{I_j} of the active rows as they stand before sublayer
 * q, which equals H_pre^q applied to the whole current state.  Sublayers 1-3
 * write only the active rows, without residual mixing: x_{I_j} gains
 * p_j sum_r H_post^q_jr v_r (one component after attention, the temporal
 * basis after the first MLP); each sublayer's post-map comes from RMSNorm of
 * the active rows before it.  The final MLP is full xHC's: H_res and H_post
 * from its active rows, then the k x k mix and gated write.
 *
 * Per group, on one stream and one workspace:
 *
 *   xhcf4_pre (cfg, w, X, inp, bases, ws)          inp: input of sublayer 1
 *   for q = 1..4:
 *     out = F_q(inp)
 *     xhcf4_post(cfg, w, q, X, out, bases, inp, ws)  X written; for q < 4
 *                                                   inp := input of q + 1
 *
 * bases: [3][T][C] of the state dtype (the non-active bases of sublayers
 * 2-4), caller-owned, written by xhcf4_pre and read by xhcf4_post.  cfg:
 * N, k, m, C, batch, seq, dtype, sinkhorn_iters, eps; n_convs (0 or 3) and
 * use_mgs describe both MLP sublayers.  Supported (N, k): (16, 4), (8, 4),
 * (4, 4), (1, 1).
 * ------------------------------------------------------------------------- */

/* Weights of one xHC-Flash-4sub group (host struct holding device pointers). */
typedef struct {
  /* [N*C][5N], state dtype: router W_r, then the pre-maps of sublayers 1-4 */
  const void* w_full;
  /* post-maps of sublayers 1-3, state dtype, rows j*C + c for position j:
   * [k*C][k] (attention), [k*C][k*K_r] (entry (j, r) at j*K_r + r), [k*C][k] */
  const void* w_post[3];
  /* final MLP: [k*C][k*k + k*K_r] = W_res (i*k + j), then W_post (k^2 + j*K_r + r) */
  const void* w_act_last;
  /* the two MLP sublayers' [24][C] float kernels (NULL when n_convs == 0) */
  const float* conv_w[2];
  /* float biases: pre-maps [N] each; post-maps [k], [k*K_r], [k], [k*K_r]; W_res [k*k] */
  const float* b_pre[4];
  const float* b_post[4];
  const float* b_res;
  float alpha_pre[4], alpha_post[4], alpha_res;
} xhcf4_weights;

/* Byte offsets of the public arrays of an xHC-Flash-4sub workspace. */
typedef struct {
  size_t idx;       /* [T][k] int32 */
  size_t p;         /* [T][k] */
  size_t h_pre;     /* [4][T][N], the pre-maps of sublayers 1-4 */
  size_t h_post;    /* [T][k][K_q]: the post-map of the next sublayer to write */
  size_t h_res;     /* [T][k][k], the final MLP's (after xhcf4_post with q = 3) */
  size_t z_router;  /* [T][N] */
  size_t total;
} xhcf4_ws_layout;

size_t xhcf4_workspace_bytes(const xhc_config* cfg);
xhc_status xhcf4_workspace_layout(const xhc_config* cfg, xhcf4_ws_layout* out);

/* Group entry: routing, the four pre-maps, the first sublayer's input (dense
 * read of X) and post-map, and the non-active bases of sublayers 2-4. */
xhc_status xhcf4_pre(const xhc_config* cfg, const xhcf4_weights* w, const void* X, void* inp, void* bases,
                     void* ws, xhc_stream_t stream);

/* After sublayer q (1..4) with output out: its write to the active rows of X
 * (in place); for q < 4 also the input of sublayer q + 1 into inp and that
 * sublayer's active maps into ws. */
xhc_status xhcf4_post(const xhc_config* cfg, const xhcf4_weights* w, int32_t q, void* X, const void* out,
                      const void* bases, void* inp, void* ws, xhc_stream_t stream);

/* ---------------------------------------------------------------------------
 * Backward of one xHC sublayer: the gradients of xhc_pre followed by
 * xhc_post (xHC paper "xHC: Expanded Hyper-Connections", paragraphs
 * "Mapping generation" and "Mapping application", differentiated; summary
 * "小红书xHC：时序特征增强 + 稀疏写回", sections 3.3 and 3.4).  The active set
 * is a selection: it is held fixed, and the router receives gradient only
 * through the router weights p of the selected routed streams.  The Sinkhorn
 * iterations are recomputed and differentiated through.
 *
 * Two calls, run in this order with the same backward workspace bws:
 *   xhc_post_backward  the application half (maps held fixed), and
 *   xhc_pre_backward   the generation half (through the maps).
 * Both read what the forward left in ws for the same cfg and X: the maps,
 * and per token the raw pre-map logits and the sums of x and x^2 (kept there
 * by xhc_pre, and by the chained calls in the workspace of the sublayer
 * whose routing they finish).
 * ------------------------------------------------------------------------- */

/* Weight gradients (host struct holding device pointers; float, written). */
typedef struct {
  float* dW_full;   /* [N*C][2N], layout of xhc_weights.w_full */
  float* dW_act;    /* [k*C][k*k + k*K_r], layout of xhc_weights.w_act */
  float* d_b_pre;   /* [N] */
  float* d_b_res;   /* [k*k] */
  float* d_b_post;  /* [k*K_r] */
  float* d_alpha;   /* [3]: alpha_pre, alpha_res, alpha_post */
} xhc_grads;

/* Byte offsets of the public arrays inside a backward workspace (float). */
typedef struct {
  size_t d_h_pre;   /* [T][N]    gradient of H_pre */
  size_t d_h_res;   /* [T][k][k] gradient of H_res (after the row clamp) */
  size_t d_h_post;  /* [T][k][K_r] gradient of H_post */
  size_t d_p;       /* [T][k]    gradient of the router weights p */
  size_t total;     /* bytes the caller must allocate (0 when T == 0) */
} xhc_bwd_ws_layout;

size_t xhc_backward_workspace_bytes(const xhc_config* cfg);
xhc_status xhc_backward_workspace_layout(const xhc_config* cfg, xhc_bwd_ws_layout* out);

/* Application half: the gradients of the maps (into bws), of out and of
 * the conv kernels, and the active rows' share of the state gradient
 * through the dense read and the mix (active row j: sum_i H_res[i][j]
 * d_X[I_i] + H_pre[I_j] d_inp), kept in float in bws for xhc_pre_backward.
 *   X:      [T][N][C] the state xhc_pre read (before xhc_post), read only
 *   out:    [T][C] the sublayer output, read only
 *   d_inp:  [T][C] gradient of the sublayer input inp, read only
 *   d_X:    [T][N][C] gradient of the new state, read only (active rows)
 *   d_out:  [T][C] written: gradient of out (through Gram-Schmidt and the
 *           causal convolutions for MLP-type sublayers)
 *   d_conv: float [24][C] written, the conv-kernel gradients in conv_w's
 *           layout (MLP-type; NULL for attention-type)
 *   ws:     the workspace xhc_pre filled;  bws: xhc_backward_workspace_bytes
 * X, out, d_inp, d_X, d_out in the state dtype, 16-byte aligned; d_out and
 * bws alias no input. */
xhc_status xhc_post_backward(const xhc_config* cfg, const xhc_weights* w, const void* X, const void* out,
                             const void* d_inp, const void* d_X, void* d_out, float* d_conv, const void* ws,
                             void* bws, xhc_stream_t stream);

/* Generation half: writes dX, the whole state gradient, and every field of
 * g.  dX is the application half's part (non-active rows d_X + H_pre[n]
 * d_inp; the active rows' part as xhc_post_backward left it in bws) plus
 * the part through the norms and the projections (full state for the
 * router and H_pre, active rows for H_res and H_post), summed in float and
 * rounded once to the state dtype (the paper's backward accumulates both
 * contributions straight into the full state's gradient, "Mapping
 * application").  X, d_inp and d_X as given to xhc_post_backward (read
 * only); dX [T][N][C] written, and may be d_X itself (in place); no other
 * buffer may alias. */
xhc_status xhc_pre_backward(const xhc_config* cfg, const xhc_weights* w, const void* X, const void* d_inp,
                            const void* d_X, void* dX, const xhc_grads* g, const void* ws, void* bws,
                            xhc_stream_t stream);

/* Measurement helper, not part of the layer: reads `bytes` bytes at `src`
 * (device memory, 16-byte aligned, bytes a multiple of 16) with 16-byte
 * vector loads spread over the whole device and writes one 32-bit word per
 * workgroup to `sink` (device memory, 4096 words) so that no load is dropped.
 * mode 0: the default cache policy; mode 1: non-temporal loads.  Timed next
 * to the layer's kernels, it gives the read rate a plain stream reaches on
 * the same GPU. */
xhc_status xhc_probe_read(const void* src, size_t bytes, uint32_t* sink, int mode, xhc_stream_t stream);

/* Message for the last non-OK status returned on this host thread. */
const char* xhc_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* XHC_H */
