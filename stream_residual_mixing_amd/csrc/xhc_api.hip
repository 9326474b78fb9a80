// libxhc host side: argument checks, workspace layout, launches, errors.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "xhc.h"
#include "xhc_internal.hpp"

#ifndef XHC_MHC_GRID
#define XHC_MHC_GRID 256   // workgroups the wide mHC projection aims for
#endif

namespace {

thread_local std::string g_err;

xhc_status fail(xhc_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool sync_mode() {
  static int v = -1;
  if (v < 0) {
    const char* e = std::getenv("XHC_SYNC");
    v = (e && e[0] && e[0] != '0') ? 1 : 0;
  }
  return v == 1;
}

bool xhc_shape_supported(int N, int K) {
  return (N == 16 && K == 4) || (N == 16 && K == 2) || (N == 8 && K == 4) || (N == 4 && K == 4) ||
         (N == 1 && K == 1);
}

// Validate the config and derive the plan (no device calls).
xhc_status make_plan(const xhc_config* cfg, bool mhc, xhc::Plan* P) {
  using xhc::Plan;
  if (!cfg) return fail(XHC_ERR_INVALID_ARG, "config is NULL");
  Plan q;
  q.mhc = mhc;
  q.N = cfg->n_streams;
  q.C = cfg->channels;
  q.B = cfg->batch;
  q.S = cfg->seq;
  q.dtype = cfg->dtype;
  q.iters = cfg->sinkhorn_iters;
  q.use_mgs = cfg->use_mgs ? 1 : 0;
  q.eps_norm = cfg->eps_norm;
  q.eps_mgs = cfg->eps_mgs;
  if (q.dtype != XHC_F32 && q.dtype != XHC_BF16) return fail(XHC_ERR_UNSUPPORTED, "dtype %d not supported", q.dtype);
  if (q.N < 1 || q.N > 16) return fail(XHC_ERR_INVALID_ARG, "n_streams=%d outside 1..16", q.N);
  if (q.C <= 0 || q.C % 32 != 0) return fail(XHC_ERR_INVALID_ARG, "channels=%d must be a positive multiple of 32", q.C);
  if (q.C > 65536) return fail(XHC_ERR_UNSUPPORTED, "channels=%d above 65536", q.C);
  if (q.B < 0 || q.S < 0) return fail(XHC_ERR_INVALID_ARG, "batch=%d, seq=%d must be >= 0", q.B, q.S);
  q.T = (long)q.B * (long)q.S;
  if (q.T > (1L << 30)) return fail(XHC_ERR_UNSUPPORTED, "batch*seq=%ld too large", q.T);
  if ((double)q.T * q.N * q.C > 9.0e15) return fail(XHC_ERR_UNSUPPORTED, "state too large");
  if (q.iters < 0 || q.iters > 1000) return fail(XHC_ERR_INVALID_ARG, "sinkhorn_iters=%d outside 0..1000", q.iters);
  if (!(std::isfinite(q.eps_norm) && q.eps_norm >= 0.f))
    return fail(XHC_ERR_INVALID_ARG, "eps_norm must be finite and >= 0");
  if (!(std::isfinite(q.eps_mgs) && q.eps_mgs >= 0.f))
    return fail(XHC_ERR_INVALID_ARG, "eps_mgs must be finite and >= 0");
  const int KB = q.dtype == XHC_BF16 ? 32 : 16;
  q.nslices = (q.C + xhc::PSLICE - 1) / xhc::PSLICE;
  if (mhc) {
    if (q.N != 1 && q.N != 2 && q.N != 4 && q.N != 8 && q.N != 16)
      return fail(XHC_ERR_UNSUPPORTED, "mHC supports N in {1,2,4,8,16}, got %d", q.N);
    q.K = q.N;
    q.ncol_full = 2 * q.N + q.N * q.N;
  } else {
    q.K = cfg->k_active;
    q.m = cfg->m_fixed;
    if (q.K < 1 || q.K > q.N) return fail(XHC_ERR_INVALID_ARG, "k_active=%d outside 1..N=%d", q.K, q.N);
    if (q.m < 0 || q.m > q.K) return fail(XHC_ERR_INVALID_ARG, "m_fixed=%d outside 0..k=%d", q.m, q.K);
    if (!xhc_shape_supported(q.N, q.K))
      return fail(XHC_ERR_UNSUPPORTED, "xHC (N=%d, k=%d) not built; supported: (16,4) (16,2) (8,4) (4,4) (1,1)",
                  q.N, q.K);
    if (cfg->n_convs == 0) {
      q.KR = 1;
    } else if (cfg->n_convs == 3) {
      if (cfg->conv_kernel[0] != 4 || cfg->conv_kernel[1] != 8 || cfg->conv_kernel[2] != 12)
        return fail(XHC_ERR_UNSUPPORTED, "conv kernel sizes {%d,%d,%d} not built; supported: {4,8,12}",
                    cfg->conv_kernel[0], cfg->conv_kernel[1], cfg->conv_kernel[2]);
      q.KR = 4;
    } else {
      return fail(XHC_ERR_INVALID_ARG, "n_convs=%d must be 0 or 3", cfg->n_convs);
    }
    if (q.C > 32768) return fail(XHC_ERR_UNSUPPORTED, "xHC channels=%d above 32768", q.C);
    q.ncol_full = 2 * q.N;
    q.ncol_act = q.K * q.K + q.K * q.KR;
    q.NTA = (q.ncol_act + 15) / 16;
    q.nkb_act = (long)q.K * q.C / KB;
  }
  q.NTF = (q.ncol_full + 15) / 16;
  q.nkb_full = (long)q.N * q.C / KB;
  const long nblk_t = (q.T + 63) / 64;
  long ks = nblk_t > 0 ? (1024 + nblk_t - 1) / nblk_t : 1;
  if (ks > 8) ks = 8;
  if (ks > q.nkb_full) ks = q.nkb_full;
  if (ks < 1) ks = 1;
  q.KS = (int)ks;

  // workspace layout: public arrays first, then internal scratch
  const size_t T = (size_t)q.T, N = q.N, K = q.K;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  if (mhc) {
    // Wide maps (N >= 8, bf16): the projection [T x NC] . [NC x (2N + N^2)] is a
    // real GEMM (N = 16: 618 GFLOP at T = 16384), done by a kernel that keeps
    // 256 tokens per workgroup against weights staged in LDS; its contraction
    // is split so that the grid covers the device (about 256 workgroups), each
    // range at least 16 contraction blocks long.
    q.mhc_wide = q.N >= 8 && q.dtype == XHC_BF16;
    if (q.mhc_wide) {
      const long ntile = (q.T + 255) / 256;
      long ks = ntile > 0 ? (XHC_MHC_GRID + ntile - 1) / ntile : 1;
      if (ks > 8) ks = 8;
      while (ks > 1 && q.nkb_full / ks < 16) --ks;
      q.KS = (int)(ks < 1 ? 1 : ks);
    }
    q.o_hpre = take(T * N * 4);
    q.o_hres = take(T * N * N * 4);
    q.o_hpost = take(T * N * 4);
    q.o_wfull = take((size_t)q.nkb_full * q.NTF * 64 * 16);
    q.o_part = take((size_t)q.KS * T * q.NTF * 16 * 4);
    q.o_stats = take((size_t)q.KS * T * 2 * 4);
  } else {
    // one-pass pre: 16-token tiles, G channel slices of PRE_WV * PRE_NKW blocks
    const long nkbC = q.C / KB;
    constexpr int SB = xhc::PRE_WV * xhc::PRE_NKW;
    q.G = (int)((nkbC + SB - 1) / SB);
    // persistent chained kernels: slices of 4 blocks (their routing weights fit in LDS)
    q.Gp = (int)((nkbC + 3) / 4);
    const size_t GM = (size_t)(q.G > q.Gp ? q.G : q.Gp);
    q.ntiles = (q.T + 15) / 16;
    const size_t P1 = 16 * (size_t)q.NTF * 16 + 2 * 16 + 16;
    const size_t P2 = 16 * (size_t)q.NTA * 16 + 16;
    q.o_sync = take((2 + 3 * (size_t)q.ntiles) * 4);
    q.o_idx = take(T * K * 4);
    q.o_p = take(T * K * 4);
    q.o_hpre = take(T * N * 4);
    q.o_hres = take(T * K * K * 4);
    q.o_hpost = take(T * K * q.KR * 4);
    q.o_z = take(T * N * 4);
    q.o_gstat = take(T * (N + 2) * 4);
    q.o_wfull = take((size_t)q.nkb_full * q.NTF * 64 * 16);
    q.o_wact = take((size_t)q.nkb_act * q.NTA * 64 * 16);
    q.o_part = take((size_t)q.ntiles * GM * P1 * 4);
    q.o_part2 = take((size_t)q.ntiles * GM * P2 * 4);
    q.o_gram = take((size_t)q.nslices * T * 10 * 8);
    q.o_corr = take((size_t)q.ntiles * GM * P1 * 4);
    q.o_wcoef = take(T * K * 4 * 4);
  }
  q.total = q.T == 0 ? 0 : off;
  *P = q;
  return XHC_OK;
}

// xHC-Flash block plan: the xHC checks, then the block's own workspace.
xhc_status make_flash_plan(const xhc_config* cfg, xhc::Plan* P) {
  xhc::Plan q;
  xhc_status s = make_plan(cfg, false, &q);
  if (s != XHC_OK) return s;
  if (!((q.N == 16 && q.K == 4) || (q.N == 8 && q.K == 4) || (q.N == 4 && q.K == 4) || (q.N == 1 && q.K == 1)))
    return fail(XHC_ERR_UNSUPPORTED, "xHC-Flash (N=%d, k=%d) not built; supported: (16,4) (8,4) (4,4) (1,1)", q.N,
                q.K);
  q.flash = true;
  const int KB = q.dtype == XHC_BF16 ? 32 : 16;
  q.ncol_full = 3 * q.N;
  q.NTF = (q.ncol_full + 15) / 16;
  q.nkb_full = (long)q.N * q.C / KB;
  q.ncol_act = q.K * q.K + q.K * q.KR;
  q.NTA = (q.ncol_act + 15) / 16;
  q.nkb_act = (long)q.K * q.C / KB;
  q.ntiles = (q.T + 15) / 16;
  // split-K of the full-state projection: about 1024 workgroups of 64 tokens
  const long nblk_t = (q.T + 63) / 64;
  long ks = nblk_t > 0 ? (1024 + nblk_t - 1) / nblk_t : 1;
  q.KS = (int)(ks > 8 ? 8 : ks < 1 ? 1 : ks);
  // splits of the active-row projections: about 1024 workgroups of 4 tiles
  const long nblk_a = (q.ntiles + 3) / 4;
  long g2 = nblk_a > 0 ? (1024 + nblk_a - 1) / nblk_a : 1;
  if (g2 > 8) g2 = 8;
  if (g2 > q.nkb_act) g2 = q.nkb_act;
  q.G2 = (int)(g2 < 1 ? 1 : g2);

  const size_t T = (size_t)q.T, N = q.N, K = q.K;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  q.o_sync = SIZE_MAX; q.o_corr = SIZE_MAX;
  q.o_idx = take(T * K * 4);
  q.o_p = take(T * K * 4);
  q.o_hpre = take(T * N * 4);
  q.o_hpre_m = take(T * N * 4);
  q.o_hpost_a = take(T * K * 4);
  q.o_hres = take(T * K * K * 4);
  q.o_hpost = take(T * K * q.KR * 4);
  q.o_z = take(T * N * 4);
  q.o_colsum = take((1 + 256) * N * 4);   // column sums, then the per-row-block partials
  q.o_wfull = take((size_t)q.nkb_full * q.NTF * 64 * 16);
  q.o_wact_a = take((size_t)q.nkb_act * 1 * 64 * 16);
  q.o_wact = take((size_t)q.nkb_act * q.NTA * 64 * 16);
  // projection partials: split-K [KS][T][NTF*16], or per (16-token tile,
  // slice) of the persistent N = 16 kernel (48 columns + sums + column sums)
  const size_t part_splitk = (size_t)q.KS * T * q.NTF * 16;
  const size_t part_tiles = (size_t)q.ntiles * q.Gp * (16 * 48 + 32 + 16);
  q.o_part = take((part_splitk > part_tiles ? part_splitk : part_tiles) * 4);
  q.o_stats = take((size_t)q.KS * T * 2 * 4);
  const size_t P2 = 16 * (size_t)(q.NTA > 1 ? q.NTA : 1) * 16 + 16;
  q.o_part2 = take((size_t)q.ntiles * q.G2 * P2 * 4);
  q.o_gram = take((size_t)q.nslices * T * 10 * 8);
  q.total = q.T == 0 ? 0 : off;
  *P = q;
  return XHC_OK;
}

// xHC-Flash-4sub group plan: the block plan with 5N full-state columns, four
// pre-maps and the packed post-maps of sublayers 1-3.
xhc_status make_flash4_plan(const xhc_config* cfg, xhc::Plan* P) {
  xhc::Plan q;
  xhc_status s = make_flash_plan(cfg, &q);
  if (s != XHC_OK) return s;
  q.ncol_full = 5 * q.N;
  q.NTF = (q.ncol_full + 15) / 16;
  const size_t T = (size_t)q.T, N = q.N, K = q.K;
  const int ntq[3] = {1, (q.K * q.KR + 15) / 16, 1};
  const int ntmax = q.NTA > ntq[1] ? q.NTA : ntq[1];
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  q.o_idx = take(T * K * 4);
  q.o_p = take(T * K * 4);
  q.o_hpre = take(4 * T * N * 4);
  q.o_hpost = take(T * K * q.KR * 4);
  q.o_hres = take(T * K * K * 4);
  q.o_z = take(T * N * 4);
  q.o_hpre_m = SIZE_MAX; q.o_hpost_a = SIZE_MAX; q.o_wact_a = SIZE_MAX;
  q.o_colsum = take((1 + 256) * N * 4);
  q.o_wfull = take((size_t)q.nkb_full * q.NTF * 64 * 16);
  for (int i = 0; i < 3; ++i) q.o_wq[i] = take((size_t)q.nkb_act * ntq[i] * 64 * 16);
  q.o_wact = take((size_t)q.nkb_act * q.NTA * 64 * 16);
  // projection partials: split-K [KS][T][NTF*16], or per (16-token tile,
  // slice) of the staged persistent N = 16 kernel
  const size_t part_splitk = (size_t)q.KS * T * q.NTF * 16;
  const size_t part_tiles = xhc::flash4_route_p_applies(q) ? (size_t)q.ntiles * q.Gp * xhc::FLASH4_P1 : 0;
  q.o_part = take((part_splitk > part_tiles ? part_splitk : part_tiles) * 4);
  q.o_stats = take((size_t)q.KS * T * 2 * 4);
  q.o_part2 = take((size_t)q.ntiles * q.G2 * (16 * (size_t)ntmax * 16 + 16) * 4);
  q.o_gram = take((size_t)q.nslices * T * 10 * 8);
  q.total = q.T == 0 ? 0 : off;
  *P = q;
  return XHC_OK;
}

xhc_status check_flash_weights(const xhc::Plan& P, const xhcf_weights* w, int stage) {
  if (!w) return fail(XHC_ERR_INVALID_ARG, "weights is NULL");
  if (stage == 0) {
    if (!w->w_full || !aligned16(w->w_full) || !w->w_post_attn || !aligned16(w->w_post_attn) || !w->w_act_mlp ||
        !aligned16(w->w_act_mlp))
      return fail(XHC_ERR_INVALID_ARG, "w_full, w_post_attn and w_act_mlp must be 16-byte aligned pointers");
    if (!w->b_pre_attn || !w->b_pre_mlp || !w->b_post_attn)
      return fail(XHC_ERR_INVALID_ARG, "b_pre_attn, b_pre_mlp and b_post_attn must not be NULL");
    if (!std::isfinite(w->alpha_pre_attn) || !std::isfinite(w->alpha_pre_mlp) || !std::isfinite(w->alpha_post_attn))
      return fail(XHC_ERR_INVALID_ARG, "alpha scales must be finite");
  } else if (stage == 1) {
    if (!w->b_res || !w->b_post_mlp) return fail(XHC_ERR_INVALID_ARG, "b_res and b_post_mlp must not be NULL");
    if (!std::isfinite(w->alpha_res) || !std::isfinite(w->alpha_post_mlp))
      return fail(XHC_ERR_INVALID_ARG, "alpha scales must be finite");
  } else if (P.KR == 4 && (!w->conv_w || !aligned16(w->conv_w))) {
    return fail(XHC_ERR_INVALID_ARG, "conv_w must be a 16-byte aligned pointer when n_convs == 3");
  }
  return XHC_OK;
}

xhc_status check_weights(const xhc::Plan& P, const xhc_weights* w, bool need_pre) {
  if (!w) return fail(XHC_ERR_INVALID_ARG, "weights is NULL");
  if (!std::isfinite(w->alpha_pre) || !std::isfinite(w->alpha_res) || !std::isfinite(w->alpha_post))
    return fail(XHC_ERR_INVALID_ARG, "alpha scales must be finite");
  if (need_pre) {
    if (!w->w_full || !aligned16(w->w_full)) return fail(XHC_ERR_INVALID_ARG, "w_full must be a 16-byte aligned pointer");
    if (!P.mhc && (!w->w_act || !aligned16(w->w_act)))
      return fail(XHC_ERR_INVALID_ARG, "w_act must be a 16-byte aligned pointer");
    if (!w->b_pre || !w->b_res || !w->b_post) return fail(XHC_ERR_INVALID_ARG, "bias pointers must not be NULL");
  }
  if (!need_pre && !P.mhc && P.KR == 4 && (!w->conv_w || !aligned16(w->conv_w)))
    return fail(XHC_ERR_INVALID_ARG, "conv_w must be a 16-byte aligned pointer for MLP-type configs");
  return XHC_OK;
}

xhc_status finish(hipStream_t st) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(XHC_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  if (sync_mode()) {
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(XHC_ERR_HIP, "stream synchronize failed: %s", hipGetErrorString(e));
    e = hipGetLastError();
    if (e != hipSuccess) return fail(XHC_ERR_HIP, "kernel failed: %s", hipGetErrorString(e));
  }
  return XHC_OK;
}

xhc_status fill_layout(const xhc::Plan& P, xhc_ws_layout* out) {
  if (!out) return fail(XHC_ERR_INVALID_ARG, "layout output is NULL");
  out->idx = P.o_idx;
  out->p = P.o_p;
  out->h_pre = P.o_hpre;
  out->h_res = P.o_hres;
  out->h_post = P.o_hpost;
  out->z_router = P.o_z;
  out->status = P.o_sync == SIZE_MAX ? SIZE_MAX : P.o_sync + 4;
  out->total = P.total;
  return XHC_OK;
}

xhc_status pre_common(const xhc_config* cfg, const xhc_weights* w, const void* X, void* inp, void* ws,
                      xhc_stream_t stream, bool mhc) {
  xhc::Plan P;
  xhc_status s = make_plan(cfg, mhc, &P);
  if (s != XHC_OK) return s;
  if ((s = check_weights(P, w, true)) != XHC_OK) return s;
  if (P.T == 0) return XHC_OK;
  if (!X || !inp || !ws) return fail(XHC_ERR_INVALID_ARG, "X, inp and ws must not be NULL");
  if (!aligned16(X) || !aligned16(inp) || !aligned16(ws))
    return fail(XHC_ERR_INVALID_ARG, "X, inp and ws must be 16-byte aligned");
  if (X == inp || X == ws || inp == ws) return fail(XHC_ERR_INVALID_ARG, "X, inp and ws must not alias");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool ok = mhc ? xhc::launch_mhc_pre(P, X, inp, w, static_cast<char*>(ws), st)
                      : xhc::launch_xhc_pre(P, X, inp, w, static_cast<char*>(ws), st);
  if (!ok) return fail(XHC_ERR_UNSUPPORTED, "no kernel built for this shape");
  return finish(st);
}

xhc_status post_common(const xhc_config* cfg, const xhc_weights* w, void* X, const void* out, void* ws,
                       xhc_stream_t stream, bool mhc) {
  xhc::Plan P;
  xhc_status s = make_plan(cfg, mhc, &P);
  if (s != XHC_OK) return s;
  if (!mhc && (s = check_weights(P, w, false)) != XHC_OK) return s;
  if (P.T == 0) return XHC_OK;
  if (!X || !out || !ws) return fail(XHC_ERR_INVALID_ARG, "X, out and ws must not be NULL");
  if (!aligned16(X) || !aligned16(out) || !aligned16(ws))
    return fail(XHC_ERR_INVALID_ARG, "X, out and ws must be 16-byte aligned");
  if (X == out || X == ws || out == ws) return fail(XHC_ERR_INVALID_ARG, "X, out and ws must not alias");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool ok = mhc ? xhc::launch_mhc_post(P, X, out, static_cast<char*>(ws), st)
                      : xhc::launch_xhc_post(P, X, out, w, static_cast<char*>(ws), st);
  if (!ok) return fail(XHC_ERR_UNSUPPORTED, "no kernel built for this shape");
  return finish(st);
}

// Plan of the next sublayer of a chain, checked against this one.
xhc_status next_plan(const xhc::Plan& P, const xhc_config* cfg_next, xhc::Plan* Pn) {
  xhc_status s = make_plan(cfg_next, false, Pn);
  if (s != XHC_OK) return s;
  if (Pn->N != P.N || Pn->K != P.K || Pn->m != P.m || Pn->C != P.C || Pn->B != P.B || Pn->S != P.S ||
      Pn->dtype != P.dtype)
    return fail(XHC_ERR_INVALID_ARG, "next sublayer must agree in n_streams, k_active, m_fixed, channels, batch, "
                                     "seq and dtype");
  return XHC_OK;
}

xhc_status check_state_ws(const void* X, const void* io, const void* ws, const void* ws_next, bool chained) {
  if (!X || !io || !ws) return fail(XHC_ERR_INVALID_ARG, "X, inp/out and ws must not be NULL");
  if (!aligned16(X) || !aligned16(io) || !aligned16(ws) || (ws_next && !aligned16(ws_next)))
    return fail(XHC_ERR_INVALID_ARG, "X, inp/out and workspaces must be 16-byte aligned");
  if (X == io || X == ws || io == ws) return fail(XHC_ERR_INVALID_ARG, "X, inp/out and ws must not alias");
  if (chained && (ws_next == ws || ws_next == X || ws_next == io))
    return fail(XHC_ERR_INVALID_ARG, "ws_next must be a workspace of its own");
  return XHC_OK;
}

}  // namespace

extern "C" {

size_t xhc_workspace_bytes(const xhc_config* cfg) {
  xhc::Plan P;
  return make_plan(cfg, false, &P) == XHC_OK ? P.total : 0;
}

size_t mhc_workspace_bytes(const xhc_config* cfg) {
  xhc::Plan P;
  return make_plan(cfg, true, &P) == XHC_OK ? P.total : 0;
}

xhc_status xhc_workspace_layout(const xhc_config* cfg, xhc_ws_layout* out) {
  xhc::Plan P;
  xhc_status s = make_plan(cfg, false, &P);
  return s != XHC_OK ? s : fill_layout(P, out);
}

xhc_status mhc_workspace_layout(const xhc_config* cfg, xhc_ws_layout* out) {
  xhc::Plan P;
  xhc_status s = make_plan(cfg, true, &P);
  return s != XHC_OK ? s : fill_layout(P, out);
}

xhc_status xhc_pre(const xhc_config* cfg, const xhc_weights* w, const void* X, void* inp, void* ws,
                   xhc_stream_t stream) {
  return pre_common(cfg, w, X, inp, ws, stream, false);
}

xhc_status xhc_post(const xhc_config* cfg, const xhc_weights* w, void* X, const void* out, void* ws,
                    xhc_stream_t stream) {
  return post_common(cfg, w, X, out, ws, stream, false);
}

xhc_status xhc_post_noalloc(const xhc_config* cfg, const xhc_weights* w, void* X, const void* out, const void* ws,
                            xhc_stream_t stream) {
  xhc::Plan P;
  xhc_status s = make_plan(cfg, false, &P);
  if (s != XHC_OK) return s;
  if ((s = check_weights(P, w, false)) != XHC_OK) return s;
  const size_t need = xhc::post_scratch_bytes(P);
  if (need > XHC_NOALLOC_SCRATCH_BYTES)
    return fail(XHC_ERR_INVALID_ARG,
                "xhc_post_noalloc: this write needs %zu bytes of scratch (T=%ld, C=%d), more than the library's %zu",
                need, P.T, P.C, (size_t)XHC_NOALLOC_SCRATCH_BYTES);
  if (P.T == 0) return XHC_OK;
  if (!X || !out || !ws) return fail(XHC_ERR_INVALID_ARG, "X, out and ws must not be NULL");
  if (!aligned16(X) || !aligned16(out) || !aligned16(ws))
    return fail(XHC_ERR_INVALID_ARG, "X, out and ws must be 16-byte aligned");
  if (X == out || X == ws || out == ws) return fail(XHC_ERR_INVALID_ARG, "X, out and ws must not alias");
  double* sp = nullptr;
  const hipError_t e = xhc::noalloc_scratch(&sp);
  if (e != hipSuccess) return fail(XHC_ERR_HIP, "scratch address lookup failed: %s", hipGetErrorString(e));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!xhc::launch_xhc_post_noalloc(P, X, out, w, static_cast<const char*>(ws), sp, st))
    return fail(XHC_ERR_UNSUPPORTED, "no kernel built for this shape");
  return finish(st);
}

xhc_status xhc_probe_read(const void* src, size_t bytes, uint32_t* sink, int mode, xhc_stream_t stream) {
  if (!src || !sink) return fail(XHC_ERR_INVALID_ARG, "src and sink must not be NULL");
  if (!aligned16(src) || bytes % 16 != 0) return fail(XHC_ERR_INVALID_ARG, "src must be 16-byte aligned, bytes a multiple of 16");
  if (mode != 0 && mode != 1) return fail(XHC_ERR_INVALID_ARG, "mode must be 0 or 1");
  if (bytes == 0) return XHC_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  xhc::launch_probe_read(src, bytes, sink, mode, st);
  return finish(st);
}

xhc_status mhc_pre(const xhc_config* cfg, const xhc_weights* w, const void* X, void* inp, void* ws,
                   xhc_stream_t stream) {
  return pre_common(cfg, w, X, inp, ws, stream, true);
}

xhc_status mhc_post(const xhc_config* cfg, const xhc_weights* w, void* X, const void* out, void* ws,
                    xhc_stream_t stream) {
  return post_common(cfg, w, X, out, ws, stream, true);
}

xhc_status xhc_route(const xhc_config* cfg, const xhc_weights* w, const void* X, void* ws, xhc_stream_t stream) {
  xhc::Plan P;
  xhc_status s = make_plan(cfg, false, &P);
  if (s != XHC_OK) return s;
  if (!w) return fail(XHC_ERR_INVALID_ARG, "weights is NULL");
  if (!w->w_full || !aligned16(w->w_full)) return fail(XHC_ERR_INVALID_ARG, "w_full must be a 16-byte aligned pointer");
  if (!w->b_pre) return fail(XHC_ERR_INVALID_ARG, "b_pre must not be NULL");
  if (!std::isfinite(w->alpha_pre)) return fail(XHC_ERR_INVALID_ARG, "alpha scales must be finite");
  if (P.T == 0) return XHC_OK;
  if (!X || !ws) return fail(XHC_ERR_INVALID_ARG, "X and ws must not be NULL");
  if (!aligned16(X) || !aligned16(ws)) return fail(XHC_ERR_INVALID_ARG, "X and ws must be 16-byte aligned");
  if (X == ws) return fail(XHC_ERR_INVALID_ARG, "X and ws must not alias");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!xhc::launch_xhc_route(P, X, w, static_cast<char*>(ws), st))
    return fail(XHC_ERR_UNSUPPORTED, "no kernel built for this shape");
  return finish(st);
}

xhc_status xhc_pre_chained(const xhc_config* cfg, const xhc_weights* w, const xhc_config* cfg_next,
                           const xhc_weights* w_next, const void* X, void* inp, void* ws, void* ws_next,
                           xhc_stream_t stream) {
  xhc::Plan P, Pn;
  xhc_status s = make_plan(cfg, false, &P);
  if (s != XHC_OK) return s;
  if ((s = check_weights(P, w, true)) != XHC_OK) return s;
  const bool chained = cfg_next != nullptr;
  if (chained) {
    if ((s = next_plan(P, cfg_next, &Pn)) != XHC_OK) return s;
    if (!w_next || !w_next->w_full || !aligned16(w_next->w_full))
      return fail(XHC_ERR_INVALID_ARG, "w_next->w_full must be a 16-byte aligned pointer");
    if (!ws_next) return fail(XHC_ERR_INVALID_ARG, "ws_next must not be NULL with a next sublayer");
  }
  if (P.T == 0) return XHC_OK;
  if ((s = check_state_ws(X, inp, ws, chained ? ws_next : nullptr, chained)) != XHC_OK) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!xhc::launch_xhc_pre_chained(P, w, chained ? &Pn : nullptr, w_next, X, inp, static_cast<char*>(ws),
                                   static_cast<char*>(ws_next), st))
    return fail(XHC_ERR_UNSUPPORTED, "no kernel built for this shape");
  return finish(st);
}

xhc_status xhc_post_chained(const xhc_config* cfg, const xhc_weights* w, const xhc_config* cfg_next,
                            const xhc_weights* w_next, void* X, const void* out, void* ws, void* ws_next,
                            xhc_stream_t stream) {
  xhc::Plan P, Pn;
  xhc_status s = make_plan(cfg, false, &P);
  if (s != XHC_OK) return s;
  if ((s = check_weights(P, w, false)) != XHC_OK) return s;
  const bool chained = cfg_next != nullptr;
  if (chained) {
    if ((s = next_plan(P, cfg_next, &Pn)) != XHC_OK) return s;
    if (!w_next || !w_next->b_pre || !std::isfinite(w_next->alpha_pre))
      return fail(XHC_ERR_INVALID_ARG, "w_next needs b_pre and a finite alpha_pre");
    if (!ws_next) return fail(XHC_ERR_INVALID_ARG, "ws_next must not be NULL with a next sublayer");
  }
  if (P.T == 0) return XHC_OK;
  if ((s = check_state_ws(X, out, ws, chained ? ws_next : nullptr, chained)) != XHC_OK) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // attention-type with a next sublayer: the write and the next routing's
  // correction in one pass
  const bool fuse = chained && xhc::chain_post_fused(P);
  if (!fuse && !xhc::launch_xhc_post(P, X, out, w, static_cast<char*>(ws), st))
    return fail(XHC_ERR_UNSUPPORTED, "no kernel built for this shape");
  if (chained && !xhc::launch_xhc_chain_tail(P, Pn, w, w_next, X, out, static_cast<char*>(ws),
                                             static_cast<char*>(ws_next), fuse, st))
    return fail(XHC_ERR_UNSUPPORTED, "no kernel built for this shape");
  return finish(st);
}

xhc_status xhc_post_decode(const xhc_config* cfg, const xhc_weights* w, void* X, const void* out, void* conv_state,
                           const int32_t* steps, void* ws, xhc_stream_t stream) {
  xhc::Plan P;
  xhc_status s = make_plan(cfg, false, &P);
  if (s != XHC_OK) return s;
  if (cfg->seq != 1) return fail(XHC_ERR_INVALID_ARG, "decode takes one new token per sequence: seq must be 1");
  if (P.KR != 4)
    return fail(XHC_ERR_UNSUPPORTED, "decode of an attention-type sublayer needs no history: use xhc_post");
  if ((s = check_weights(P, w, false)) != XHC_OK) return s;
  if (P.T == 0) return XHC_OK;
  if ((s = check_state_ws(X, out, ws, nullptr, false)) != XHC_OK) return s;
  if (!conv_state || !aligned16(conv_state)) return fail(XHC_ERR_INVALID_ARG, "conv_state must be 16-byte aligned");
  if (!steps || (reinterpret_cast<uintptr_t>(steps) & 3u)) return fail(XHC_ERR_INVALID_ARG, "steps must be an aligned int32 pointer");
  if (conv_state == X || conv_state == out || conv_state == ws)
    return fail(XHC_ERR_INVALID_ARG, "conv_state must not alias X, out or ws");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!xhc::launch_xhc_post_decode(P, X, out, conv_state, steps, w, static_cast<char*>(ws), st))
    return fail(XHC_ERR_UNSUPPORTED, "no kernel built for this shape");
  return finish(st);
}

size_t xhcf_workspace_bytes(const xhc_config* cfg) {
  xhc::Plan P;
  return make_flash_plan(cfg, &P) == XHC_OK ? P.total : 0;
}

xhc_status xhcf_workspace_layout(const xhc_config* cfg, xhcf_ws_layout* out) {
  xhc::Plan P;
  xhc_status s = make_flash_plan(cfg, &P);
  if (s != XHC_OK) return s;
  if (!out) return fail(XHC_ERR_INVALID_ARG, "layout output is NULL");
  out->idx = P.o_idx;
  out->p = P.o_p;
  out->h_pre_attn = P.o_hpre;
  out->h_pre_mlp = P.o_hpre_m;
  out->h_post_attn = P.o_hpost_a;
  out->h_res = P.o_hres;
  out->h_post_mlp = P.o_hpost;
  out->z_router = P.o_z;
  out->total = P.total;
  return XHC_OK;
}

xhc_status xhcf_pre(const xhc_config* cfg, const xhcf_weights* w, const void* X, void* inp_attn, void* inp_mlp,
                    void* ws, xhc_stream_t stream) {
  xhc::Plan P;
  xhc_status s = make_flash_plan(cfg, &P);
  if (s != XHC_OK) return s;
  if ((s = check_flash_weights(P, w, 0)) != XHC_OK) return s;
  if (P.T == 0) return XHC_OK;
  if ((s = check_state_ws(X, inp_attn, ws, nullptr, false)) != XHC_OK) return s;
  if (!inp_mlp || !aligned16(inp_mlp)) return fail(XHC_ERR_INVALID_ARG, "inp_mlp must be a 16-byte aligned pointer");
  if (inp_mlp == X || inp_mlp == ws || inp_mlp == inp_attn)
    return fail(XHC_ERR_INVALID_ARG, "inp_mlp must not alias X, ws or inp_attn");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!xhc::launch_xhcf_pre(P, w, X, inp_attn, inp_mlp, static_cast<char*>(ws), st))
    return fail(XHC_ERR_UNSUPPORTED, "no kernel built for this shape");
  return finish(st);
}

xhc_status xhcf_mid(const xhc_config* cfg, const xhcf_weights* w, void* X, const void* out_attn, void* inp_mlp,
                    void* ws, xhc_stream_t stream) {
  xhc::Plan P;
  xhc_status s = make_flash_plan(cfg, &P);
  if (s != XHC_OK) return s;
  if ((s = check_flash_weights(P, w, 1)) != XHC_OK) return s;
  if (P.T == 0) return XHC_OK;
  if ((s = check_state_ws(X, out_attn, ws, nullptr, false)) != XHC_OK) return s;
  if (!inp_mlp || !aligned16(inp_mlp)) return fail(XHC_ERR_INVALID_ARG, "inp_mlp must be a 16-byte aligned pointer");
  if (inp_mlp == X || inp_mlp == ws || inp_mlp == out_attn)
    return fail(XHC_ERR_INVALID_ARG, "inp_mlp must not alias X, ws or out_attn");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!xhc::launch_xhcf_mid(P, w, X, out_attn, inp_mlp, static_cast<char*>(ws), st))
    return fail(XHC_ERR_UNSUPPORTED, "no kernel built for this shape");
  return finish(st);
}

xhc_status xhcf_post(const xhc_config* cfg, const xhcf_weights* w, void* X, const void* out_mlp, void* ws,
                     xhc_stream_t stream) {
  xhc::Plan P;
  xhc_status s = make_flash_plan(cfg, &P);
  if (s != XHC_OK) return s;
  if ((s = check_flash_weights(P, w, 2)) != XHC_OK) return s;
  if (P.T == 0) return XHC_OK;
  if ((s = check_state_ws(X, out_mlp, ws, nullptr, false)) != XHC_OK) return s;
  xhc_weights wx{};
  wx.conv_w = w->conv_w;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!xhc::launch_xhc_post(P, X, out_mlp, &wx, static_cast<char*>(ws), st))
    return fail(XHC_ERR_UNSUPPORTED, "no kernel built for this shape");
  return finish(st);
}

size_t xhcf4_workspace_bytes(const xhc_config* cfg) {
  xhc::Plan P;
  return make_flash4_plan(cfg, &P) == XHC_OK ? P.total : 0;
}

xhc_status xhcf4_workspace_layout(const xhc_config* cfg, xhcf4_ws_layout* out) {
  xhc::Plan P;
  xhc_status s = make_flash4_plan(cfg, &P);
  if (s != XHC_OK) return s;
  if (!out) return fail(XHC_ERR_INVALID_ARG, "layout output is NULL");
  out->idx = P.o_idx;
  out->p = P.o_p;
  out->h_pre = P.o_hpre;
  out->h_post = P.o_hpost;
  out->h_res = P.o_hres;
  out->z_router = P.o_z;
  out->total = P.total;
  return XHC_OK;
}

xhc_status xhcf4_pre(const xhc_config* cfg, const xhcf4_weights* w, const void* X, void* inp, void* bases, void* ws,
                     xhc_stream_t stream) {
  xhc::Plan P;
  xhc_status s = make_flash4_plan(cfg, &P);
  if (s != XHC_OK) return s;
  if (!w) return fail(XHC_ERR_INVALID_ARG, "weights is NULL");
  bool ok = w->w_full && aligned16(w->w_full);
  for (int q = 0; q < 3; ++q) ok = ok && w->w_post[q] && aligned16(w->w_post[q]);
  ok = ok && w->w_act_last && aligned16(w->w_act_last);
  if (!ok) return fail(XHC_ERR_INVALID_ARG, "w_full, w_post[0..2] and w_act_last must be 16-byte aligned pointers");
  for (int q = 0; q < 4; ++q) {
    if (!w->b_pre[q]) return fail(XHC_ERR_INVALID_ARG, "b_pre[%d] must not be NULL", q);
    if (!std::isfinite(w->alpha_pre[q])) return fail(XHC_ERR_INVALID_ARG, "alpha scales must be finite");
  }
  if (!w->b_post[0] || !std::isfinite(w->alpha_post[0]))
    return fail(XHC_ERR_INVALID_ARG, "b_post[0] must not be NULL and alpha_post[0] finite");
  if (P.T == 0) return XHC_OK;
  if ((s = check_state_ws(X, inp, ws, nullptr, false)) != XHC_OK) return s;
  if (!bases || !aligned16(bases)) return fail(XHC_ERR_INVALID_ARG, "bases must be a 16-byte aligned pointer");
  if (bases == X || bases == inp || bases == ws) return fail(XHC_ERR_INVALID_ARG, "bases must not alias X, inp or ws");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!xhc::launch_xhcf4_pre(P, w, X, inp, bases, static_cast<char*>(ws), st))
    return fail(XHC_ERR_UNSUPPORTED, "no kernel built for this shape");
  return finish(st);
}

xhc_status xhcf4_post(const xhc_config* cfg, const xhcf4_weights* w, int32_t q, void* X, const void* out,
                      const void* bases, void* inp, void* ws, xhc_stream_t stream) {
  xhc::Plan P;
  xhc_status s = make_flash4_plan(cfg, &P);
  if (s != XHC_OK) return s;
  if (!w) return fail(XHC_ERR_INVALID_ARG, "weights is NULL");
  if (q < 1 || q > 4) return fail(XHC_ERR_INVALID_ARG, "sublayer q=%d outside 1..4", q);
  if ((q == 2 || q == 4) && P.KR == 4 && (!w->conv_w[q / 2 - 1] || !aligned16(w->conv_w[q / 2 - 1])))
    return fail(XHC_ERR_INVALID_ARG, "conv_w[%d] must be a 16-byte aligned pointer when n_convs == 3", q / 2 - 1);
  if (q < 4) {
    if (!w->b_post[q] || !std::isfinite(w->alpha_post[q]))
      return fail(XHC_ERR_INVALID_ARG, "b_post[%d] must not be NULL and alpha_post[%d] finite", q, q);
    if (q == 3 && (!w->b_res || !std::isfinite(w->alpha_res)))
      return fail(XHC_ERR_INVALID_ARG, "b_res must not be NULL and alpha_res finite");
  }
  if (P.T == 0) return XHC_OK;
  if ((s = check_state_ws(X, out, ws, nullptr, false)) != XHC_OK) return s;
  if (q < 4) {
    if (!bases || !aligned16(bases) || !inp || !aligned16(inp))
      return fail(XHC_ERR_INVALID_ARG, "bases and inp must be 16-byte aligned pointers");
    if (inp == X || inp == ws || inp == out || inp == bases || bases == X || bases == ws)
      return fail(XHC_ERR_INVALID_ARG, "inp and bases must not alias X, out, ws or each other");
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!xhc::launch_xhcf4_post(P, w, q, X, out, bases, inp, static_cast<char*>(ws), st))
    return fail(XHC_ERR_UNSUPPORTED, "no kernel built for this shape");
  return finish(st);
}

size_t xhc_backward_workspace_bytes(const xhc_config* cfg) {
  xhc::Plan P;
  if (make_plan(cfg, false, &P) != XHC_OK) return 0;
  xhc::BwdPlan B;
  xhc::make_bwd_plan(P, &B);
  return B.total;
}

xhc_status xhc_backward_workspace_layout(const xhc_config* cfg, xhc_bwd_ws_layout* out) {
  xhc::Plan P;
  xhc_status s = make_plan(cfg, false, &P);
  if (s != XHC_OK) return s;
  if (!out) return fail(XHC_ERR_INVALID_ARG, "layout output is NULL");
  xhc::BwdPlan B;
  xhc::make_bwd_plan(P, &B);
  out->d_h_pre = B.o_dhpre;
  out->d_h_res = B.o_dhres;
  out->d_h_post = B.o_dhpost;
  out->d_p = B.o_dp;
  out->total = B.total;
  return XHC_OK;
}

xhc_status xhc_post_backward(const xhc_config* cfg, const xhc_weights* w, const void* X, const void* out,
                             const void* d_inp, const void* d_X, void* d_out, float* d_conv, const void* ws, void* bws,
                             xhc_stream_t stream) {
  xhc::Plan P;
  xhc_status s = make_plan(cfg, false, &P);
  if (s != XHC_OK) return s;
  if ((s = check_weights(P, w, false)) != XHC_OK) return s;
  if (P.T == 0) return XHC_OK;
  const void* ptrs[] = {X, out, d_inp, d_X, d_out, ws, bws};
  for (const void* q : ptrs)
    if (!q || !aligned16(q))
      return fail(XHC_ERR_INVALID_ARG, "X, out, d_inp, d_X, d_out, ws and bws must be 16-byte aligned, non-NULL");
  if (P.KR == 4 && !d_conv) return fail(XHC_ERR_INVALID_ARG, "d_conv must not be NULL for MLP-type configs");
  const void* outs[] = {d_out, bws};
  const void* ins[] = {X, out, d_inp, d_X, ws};
  for (const void* o : outs)
    for (const void* i : ins)
      if (o == i) return fail(XHC_ERR_INVALID_ARG, "outputs d_out and bws must not alias X, out, d_inp, d_X or ws");
  if (d_out == bws) return fail(XHC_ERR_INVALID_ARG, "d_out and bws must be distinct");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!xhc::launch_xhc_post_backward(P, w, X, out, d_inp, d_X, d_out, d_conv, static_cast<const char*>(ws),
                                     static_cast<char*>(bws), st))
    return fail(XHC_ERR_UNSUPPORTED, "no kernel built for this shape");
  return finish(st);
}

xhc_status xhc_pre_backward(const xhc_config* cfg, const xhc_weights* w, const void* X, const void* d_inp,
                            const void* d_X, void* dX, const xhc_grads* g, const void* ws, void* bws,
                            xhc_stream_t stream) {
  xhc::Plan P;
  xhc_status s = make_plan(cfg, false, &P);
  if (s != XHC_OK) return s;
  if ((s = check_weights(P, w, true)) != XHC_OK) return s;
  if (!g || !g->dW_full || !g->dW_act || !g->d_b_pre || !g->d_b_res || !g->d_b_post || !g->d_alpha)
    return fail(XHC_ERR_INVALID_ARG, "every gradient pointer must be set");
  if (P.T == 0) return XHC_OK;
  const void* ptrs[] = {X, d_inp, d_X, dX, ws, bws};
  for (const void* q : ptrs)
    if (!q || !aligned16(q))
      return fail(XHC_ERR_INVALID_ARG, "X, d_inp, d_X, dX, ws and bws must be 16-byte aligned, non-NULL");
  // dX may be d_X; no other pair may alias
  if (dX == X || dX == d_inp || dX == ws || dX == bws || bws == X || bws == d_inp || bws == d_X || bws == ws)
    return fail(XHC_ERR_INVALID_ARG, "dX and bws must not alias X, d_inp, ws or each other (only dX may be d_X)");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (!xhc::launch_xhc_pre_backward(P, w, X, d_inp, d_X, dX, g, static_cast<const char*>(ws),
                                    static_cast<char*>(bws), st))
    return fail(XHC_ERR_UNSUPPORTED, "no kernel built for this shape");
  return finish(st);
}

const char* xhc_last_error(void) { return g_err.c_str(); }

}  // extern "C"
