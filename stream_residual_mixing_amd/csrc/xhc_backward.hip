// libxhc: backward of one xHC sublayer, the gradients of xhc_pre + xhc_post.
//
// The forward is differentiated in two halves that meet at the maps
// (xHC paper "xHC: Expanded Hyper-Connections", paragraphs "Mapping
// generation" and "Mapping application"; summary "小红书xHC：时序特征增强 +
// 稀疏写回", sections 3.3 and 3.4):
//
//  * application: with the maps fixed, the dense read inp = sum_n H_pre[n] X_n
//    and the active rewrite X_I' = H_res X_I + diag(p) H_post V give the state
//    gradient through the read and the mix, the write basis' gradient (then
//    the Gram-Schmidt and the causal convolutions, transposed) and the maps'
//    gradients;
//  * generation: the maps' gradients go back through the sigmoids, the
//    Sinkhorn iterations (recomputed) and the row clamp, the router weights of
//    the selected streams, the RMSNorm / LayerNorm and the projections, giving
//    the state gradient through the norms and every weight gradient.
//
// Two small scalar programs are differentiated in forward mode, one tangent
// per input direction, recomputed from their inputs instead of stored: the
// Gram-Schmidt coefficients as a function of the K_r x K_r Gram matrix (10
// symmetric directions) and the Sinkhorn map as a function of its k x k logits
// (k^2 directions, one lane each).
//
// Kernels, in order:
//  application:  bwd_apply (per token: dot products, scalar stage, dX rows and
//                the basis gradient), bwd_conv (MLP-type: transposed convs
//                into d_out, conv-weight partials), bwd_reduce;
//  generation:   packing + split-K MFMA projection of the gathered active rows
//                (recomputing their raw logits and sums; the full state's were
//                kept by xhc_pre),
//                bwd_wcolsum, bwd_token (per-token scalars), bwd_sum_rows
//                (bias / scale gradients), bwd_rows twice (full state, active
//                rows: dX += W G + c x, weight-gradient partials), bwd_reduce.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "xhc.h"
#include "xhc_device.hpp"
#include "xhc_internal.hpp"

namespace xhc {

namespace {

constexpr int BT = 256;      // threads per workgroup
constexpr int NCONV = 24;    // conv weight rows: kernels 4, 8, 12
constexpr int NCOLB = 128;   // workgroups of the first stage of the W_r column sums

__device__ __forceinline__ float ld1(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ __forceinline__ float ld1(const float* p) { return *p; }
__device__ __forceinline__ void st1(uint16_t* p, float v) { *p = (uint16_t)f32_to_bf16(v); }
__device__ __forceinline__ void st1(float* p, float v) { *p = v; }

// Sum of v over the workgroup (BT threads); every thread receives it.
__device__ __forceinline__ float block_sum(float v, float* s_tmp) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) s_tmp[wave] = v;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int w = 0; w < BT / WAVE; ++w) r += s_tmp[w];
  return r;
}

// Write basis of token t at channels c..c+VEC: the output itself and, for
// MLP-type sublayers, its causal depthwise convolutions with kernels 4, 8, 12
// (weight rows 0, 4, 12; row off + i multiplies lag i), lags that reach
// before the sequence start left out.
template <class E, int KR>
__device__ __forceinline__ void write_basis(const typename E::T* out_t, int s, int C, int c, const float* conv_w,
                                            float (&g)[KR][E::VEC]) {
  constexpr int V = E::VEC;
  E::unpack(ld16(out_t + c), g[0]);
  if constexpr (KR == 4) {
#pragma unroll
    for (int q = 1; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < V; ++e) g[q][e] = 0.f;
    const int L = s < 11 ? s : 11;
    for (int tau = 0; tau <= L; ++tau) {
      float o[V];
      E::unpack(ld16(out_t - (long)tau * C + c), o);
#pragma unroll
      for (int q = 1; q < 4; ++q) {
        if (tau >= 4 * q) continue;
        const int row = (q == 1 ? 0 : q == 2 ? 4 : 12) + tau;
        const float* w = conv_w + (size_t)row * C + c;
#pragma unroll
        for (int e = 0; e < V; ++e) g[q][e] = fmaf(w[e], o[e], g[q][e]);
      }
    }
  }
}

// Gram-Schmidt coefficients from the Gram matrix M of the raw components:
// v_r = sum_q A[r][q] g_q, with u <- u - <u, v> / (<v, v> + eps) v taken over
// the earlier v's in order.  With a tangent direction: M's entries (a, b)
// and (b, a) moved together (one entry when a == b); returns
// sum_{r,q} D[r][q] dA[r][q].
template <int R>
__device__ float mgs_coef(const float (&M)[R][R], float eps, float (&A)[R][R], int a, int b, const float (&D)[R][R]) {
  float dA[R][R];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int q = 0; q < R; ++q) { A[r][q] = (r == q && r == 0) ? 1.f : 0.f; dA[r][q] = 0.f; }
#pragma unroll
  for (int r = 1; r < R; ++r) {
    float u[R], du[R];
#pragma unroll
    for (int i = 0; i < R; ++i) { u[i] = i == r ? 1.f : 0.f; du[i] = 0.f; }
#pragma unroll
    for (int v = 0; v < R; ++v) {
      if (v >= r) break;
      float MAv[R], dMAv[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        float s = 0.f, ds = 0.f;
#pragma unroll
        for (int j = 0; j < R; ++j) {
          s = fmaf(M[i][j], A[v][j], s);
          const float dm = ((i == a && j == b) || (i == b && j == a)) ? 1.f : 0.f;
          ds = fmaf(dm, A[v][j], fmaf(M[i][j], dA[v][j], ds));
        }
        MAv[i] = s;
        dMAv[i] = ds;
      }
      float num = 0.f, dnum = 0.f, den = eps, dden = 0.f;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        num = fmaf(u[i], MAv[i], num);
        dnum = fmaf(du[i], MAv[i], fmaf(u[i], dMAv[i], dnum));
        den = fmaf(A[v][i], MAv[i], den);
        dden = fmaf(dA[v][i], MAv[i], fmaf(A[v][i], dMAv[i], dden));
      }
      const float cf = num / den;
      const float dc = (dnum - cf * dden) / den;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        du[i] = du[i] - dc * A[v][i] - cf * dA[v][i];
        u[i] = u[i] - cf * A[v][i];
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) { A[r][i] = u[i]; dA[r][i] = du[i]; }
  }
  float f = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int q = 0; q < R; ++q) f = fmaf(D[r][q], dA[r][q], f);
  return f;
}

struct BwdApplyArgs {
  const void *X, *out, *d_inp, *d_X;
  void *d_out, *xa;
  float* dxa;         // [T][K][C]: the active rows' state gradient so far (float)
  float* dg;
  const float* conv_w;
  const int* idx;
  const float *p, *h_pre, *h_res, *h_post;
  float *d_hpre, *d_hres, *d_hpost, *d_p;
  int T, S, C, use_mgs;
  float eps_mgs;
};

// Application half, one workgroup per token.  Pass 1 takes the dot products
// <d_inp, X_n> (H_pre gradient), <dY_i, X_{I_j}> (H_res gradient),
// <dY_i, g_q> and the Gram <g_a, g_b> of the raw write components, with dY_i
// the new state's gradient on active row i; and stores the gathered active
// rows for the generation half.  The scalar stage gives the H_post and p
// gradients and the basis gradient as a combination of the dY_i and the g_q.
// Pass 2 writes the basis gradient and the active rows' share of the state
// gradient through the read and the mix (active row j: sum_i H_res[i][j] dY_i
// + H_pre[I_j] d_inp) in float to the backward workspace.  A non-active row's
// share, d_X + H_pre[n] d_inp, is formed by the generation half's full-state
// pass together with its own terms (this pass reads no non-active row of
// d_X).  Each element of the state gradient is rounded to the state dtype
// once, by the last pass that adds to it.
//
// MLP-type: workgroups are dispatched to the 8 XCDs in turn; workgroup b
// takes token (b mod 8) * ceil(T / 8) + b / 8, so that each XCD walks a
// contiguous run of tokens and the 11-row output windows of neighbouring
// tokens hit its own L2 (attention-type: token b, which measured faster).
template <class E, int N, int K, int KR>
__global__ __launch_bounds__(BT) void bwd_apply_kernel(BwdApplyArgs a) {
  using T = typename E::T;
  constexpr int V = E::VEC;
  constexpr int NG = KR * (KR + 1) / 2;
  constexpr int O_H = N, O_E = N + K * K, O_G = O_E + K * KR, NACC = O_G + NG;
  const int per_xcd = (a.T + 7) / 8;
  const int t = KR == 4 ? (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  if (t >= a.T) return;   // the whole workgroup: before any barrier
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int C = a.C;
  const int s = t % a.S;
  const T* X = reinterpret_cast<const T*>(a.X) + (size_t)t * N * C;
  const T* dXn = reinterpret_cast<const T*>(a.d_X) + (size_t)t * N * C;
  const T* di = reinterpret_cast<const T*>(a.d_inp) + (size_t)t * C;
  const T* ot = reinterpret_cast<const T*>(a.out) + (size_t)t * C;
  T* xa = reinterpret_cast<T*>(a.xa) + (size_t)t * K * C;
  __shared__ int s_idx[K], s_pos[N];
  __shared__ float s_hpre[N], s_mix[K][K];
  __shared__ float s_red[BT / WAVE][NACC], s_acc[NACC];
  __shared__ float s_al[KR][K], s_be[KR][KR];
  if (tid < N) {
    s_hpre[tid] = a.h_pre[(size_t)t * N + tid];
    s_pos[tid] = -1;
  }
  if (tid < K * K) s_mix[tid / K][tid % K] = a.h_res[(size_t)t * K * K + tid];
  __syncthreads();
  if (tid < K) {
    const int n = a.idx[(size_t)t * K + tid];
    s_idx[tid] = n;
    s_pos[n] = tid;
  }
  __syncthreads();

  float acc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i) acc[i] = 0.f;
  const int ngrp = C / V;
  for (int cg = tid; cg < ngrp; cg += BT) {
    const int c = cg * V;
    float fi[V], y[K][V], xr[K][V], g[KR][V];
    uint4 raw[K];
    E::unpack(ld16(di + c), fi);
#pragma unroll
    for (int i = 0; i < K; ++i) {
      E::unpack(ld16(dXn + (size_t)s_idx[i] * C + c), y[i]);
      raw[i] = ld16(X + (size_t)s_idx[i] * C + c);
      E::unpack(raw[i], xr[i]);
    }
    write_basis<E, KR>(ot, s, C, c, a.conv_w, g);
#pragma unroll
    for (int n = 0; n < N; ++n) {
      float x[V];
      E::unpack(ld16(X + (size_t)n * C + c), x);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[n] = fmaf(fi[e], x[e], acc[n]);
    }
#pragma unroll
    for (int i = 0; i < K; ++i) {
#pragma unroll
      for (int j = 0; j < K; ++j)
#pragma unroll
        for (int e = 0; e < V; ++e) acc[O_H + i * K + j] = fmaf(y[i][e], xr[j][e], acc[O_H + i * K + j]);
#pragma unroll
      for (int q = 0; q < KR; ++q)
#pragma unroll
        for (int e = 0; e < V; ++e) acc[O_E + i * KR + q] = fmaf(y[i][e], g[q][e], acc[O_E + i * KR + q]);
    }
    int gi = 0;
#pragma unroll
    for (int qa = 0; qa < KR; ++qa)
#pragma unroll
      for (int qb = qa; qb < KR; ++qb, ++gi)
#pragma unroll
        for (int e = 0; e < V; ++e) acc[O_G + gi] = fmaf(g[qa][e], g[qb][e], acc[O_G + gi]);
    // the gathered active rows for the generation half, stored after every
    // load of the step (a store in between would keep the later loads, which
    // the compiler cannot prove apart from it, from going out early)
#pragma unroll
    for (int i = 0; i < K; ++i) st16(xa + (size_t)i * C + c, raw[i]);
  }
#pragma unroll
  for (int i = 0; i < NACC; ++i) {
    const float v = wave_sum(acc[i]);
    if (lane == 0) s_red[wave][i] = v;
  }
  __syncthreads();
  if (tid < NACC) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < BT / WAVE; ++w) v += s_red[w][tid];
    s_acc[tid] = v;
  }
  __syncthreads();

  // scalar stage on wave 0: lane l < NG differentiates the Gram-Schmidt
  // coefficients along the l-th symmetric Gram direction; lane 0 also forms
  // the H_post / p gradients and the basis-gradient combination.
  __shared__ float s_F[NG];
  const bool mgs = KR > 1 && a.use_mgs;
  if (tid < WAVE) {
    float Gm[KR][KR], Ec[K][KR], A[KR][KR], D[KR][KR], gam[KR][K], hp[K][KR], pp[K];
    int gi = 0;
#pragma unroll
    for (int qa = 0; qa < KR; ++qa)
#pragma unroll
      for (int qb = qa; qb < KR; ++qb, ++gi) Gm[qa][qb] = Gm[qb][qa] = s_acc[O_G + gi];
#pragma unroll
    for (int i = 0; i < K; ++i) {
      pp[i] = a.p[(size_t)t * K + i];
#pragma unroll
      for (int q = 0; q < KR; ++q) {
        Ec[i][q] = s_acc[O_E + i * KR + q];
        hp[i][q] = a.h_post[((size_t)t * K + i) * KR + q];
      }
    }
#pragma unroll
    for (int r = 0; r < KR; ++r)
#pragma unroll
      for (int i = 0; i < K; ++i) gam[r][i] = pp[i] * hp[i][r];
#pragma unroll
    for (int r = 0; r < KR; ++r)
#pragma unroll
      for (int q = 0; q < KR; ++q) {
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < K; ++i) d = fmaf(gam[r][i], Ec[i][q], d);
        D[r][q] = d;
      }
    if (mgs && tid < NG) {
      int qa = 0, qb = 0, l = 0;
      for (int x = 0; x < KR; ++x)
        for (int y = x; y < KR; ++y, ++l)
          if (l == tid) { qa = x; qb = y; }
      float Ad[KR][KR];
      s_F[tid] = mgs_coef<KR>(Gm, a.eps_mgs, Ad, qa, qb, D);
    }
    if (tid == 0) {
      if (mgs) {
        mgs_coef<KR>(Gm, a.eps_mgs, A, -1, -1, D);
      } else {
#pragma unroll
        for (int r = 0; r < KR; ++r)
#pragma unroll
          for (int q = 0; q < KR; ++q) A[r][q] = r == q ? 1.f : 0.f;
      }
#pragma unroll
      for (int i = 0; i < K; ++i) {
        float dpv = 0.f;
#pragma unroll
        for (int r = 0; r < KR; ++r) {
          float dq = 0.f;
#pragma unroll
          for (int q = 0; q < KR; ++q) dq = fmaf(A[r][q], Ec[i][q], dq);
          a.d_hpost[((size_t)t * K + i) * KR + r] = pp[i] * dq;
          dpv = fmaf(hp[i][r], dq, dpv);
        }
        a.d_p[(size_t)t * K + i] = dpv;
      }
#pragma unroll
      for (int q = 0; q < KR; ++q)
#pragma unroll
        for (int i = 0; i < K; ++i) {
          float al = 0.f;
#pragma unroll
          for (int r = 0; r < KR; ++r) al = fmaf(A[r][q], gam[r][i], al);
          s_al[q][i] = al;
        }
    }
  }
  __syncthreads();
  if (tid < KR * KR) {
    const int qa = tid / KR, qb = tid % KR;
    float be = 0.f;
    if (mgs) {
      const int x = qa < qb ? qa : qb, y = qa < qb ? qb : qa;
      const int l = x * KR - x * (x - 1) / 2 + (y - x);   // index of (x, y) in the upper-triangle order
      be = x == y ? 2.f * s_F[l] : s_F[l];
    }
    s_be[qa][qb] = be;
  }
  if (tid < N) a.d_hpre[(size_t)t * N + tid] = s_acc[tid];
  if (tid < K * K) a.d_hres[(size_t)t * K * K + tid] = s_acc[O_H + tid];
  __syncthreads();

  for (int cg = tid; cg < ngrp; cg += BT) {
    const int c = cg * V;
    float fi[V], y[K][V], g[KR][V];
    E::unpack(ld16(di + c), fi);
#pragma unroll
    for (int i = 0; i < K; ++i) E::unpack(ld16(dXn + (size_t)s_idx[i] * C + c), y[i]);
    if constexpr (KR == 4) write_basis<E, KR>(ot, s, C, c, a.conv_w, g);
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const int j = s_pos[n];
      if (j >= 0) {
        // active position j: sum_i H_res[i][j] dY_i + H_pre[I_j] d_inp, in float
        float o[V];
#pragma unroll
        for (int e = 0; e < V; ++e) {
          float v = s_hpre[n] * fi[e];
#pragma unroll
          for (int i = 0; i < K; ++i) v = fmaf(s_mix[i][j], y[i][e], v);
          o[e] = v;
        }
        float* pa = a.dxa + ((size_t)t * K + j) * C + c;
#pragma unroll
        for (int e = 0; e < V; e += 4) *reinterpret_cast<float4*>(pa + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
      }
    }
#pragma unroll
    for (int q = 0; q < KR; ++q) {
      float o[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < K; ++i) v = fmaf(s_al[q][i], y[i][e], v);
        if constexpr (KR == 4) {
#pragma unroll
          for (int b = 0; b < KR; ++b) v = fmaf(s_be[q][b], g[b][e], v);
        }
        o[e] = v;
      }
      if constexpr (KR == 4) {
        float* dst = a.dg + ((size_t)t * KR + q) * C + c;
#pragma unroll
        for (int e = 0; e < V; e += 4)
          *reinterpret_cast<f32x4_t*>(dst + e) = f32x4_t{o[e], o[e + 1], o[e + 2], o[e + 3]};
      } else {
        st16(reinterpret_cast<T*>(a.d_out) + (size_t)t * C + c, E::pack(o));
      }
    }
  }
}

struct BwdConvArgs {
  const float* dg;
  const void* out;
  const float* conv_w;
  void* d_out;
  float* part;
  int T, S, C, TC;
};

// MLP-type: d_out[t] = dg_0[t] + sum over kernels q and lags i of
// w_q[i] dg_q[t + i] (same sequence), and the conv-weight gradient partials
// sum_t dg_q[t] out[t - i] over this workgroup's token range.  One thread per
// channel; two sweeps over the range, each carrying a window of 11 tokens in
// registers: downwards the later basis gradients (for d_out), upwards the
// earlier outputs (for the weight gradient).  A window is emptied where a
// sequence ends, so nothing crosses from one sequence to the next.
template <class E>
__global__ __launch_bounds__(BT) void bwd_conv_kernel(BwdConvArgs a) {
  using T = typename E::T;
  constexpr int L = 11;
  const int c = blockIdx.x * BT + threadIdx.x;
  if (c >= a.C) return;
  const int C = a.C, S = a.S;
  const int t0 = blockIdx.y * a.TC;
  const int t1 = t0 + a.TC < a.T ? t0 + a.TC : a.T;
  if (t0 >= t1) {
#pragma unroll
    for (int r = 0; r < NCONV; ++r) a.part[((size_t)blockIdx.y * NCONV + r) * C + c] = 0.f;
    return;
  }
  const T* out = reinterpret_cast<const T*>(a.out);
  T* d_out = reinterpret_cast<T*>(a.d_out);
  const float* dg = a.dg + c;
  float w[NCONV];
#pragma unroll
  for (int r = 0; r < NCONV; ++r) w[r] = a.conv_w[(size_t)r * C + c];
  // downward sweep: F[q][i] = dg_q[t + 1 + i] within the sequence, else 0
  float F[3][L];
  {
    const int tl = t1 - 1, sl = tl % S;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const bool in = sl + 1 + i < S;
#pragma unroll
      for (int q = 0; q < 3; ++q) F[q][i] = in ? dg[((size_t)(tl + 1 + i) * 4 + q + 1) * C] : 0.f;
    }
  }
  for (int t = t1 - 1; t >= t0; --t) {
    float g[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) g[q] = dg[((size_t)t * 4 + q) * C];
    float d = g[0];
#pragma unroll
    for (int q = 1; q < 4; ++q) {
      const int off = q == 1 ? 0 : q == 2 ? 4 : 12;
      d = fmaf(w[off], g[q], d);
#pragma unroll
      for (int i = 1; i < 4 * q; ++i) d = fmaf(w[off + i], F[q - 1][i - 1], d);
    }
    st1(d_out + (size_t)t * C + c, d);
    const bool start = t % S == 0;   // t - 1 belongs to the previous sequence
#pragma unroll
    for (int q = 0; q < 3; ++q) {
#pragma unroll
      for (int i = L - 1; i > 0; --i) F[q][i] = start ? 0.f : F[q][i - 1];
      F[q][0] = start ? 0.f : g[q + 1];
    }
  }
  // upward sweep: P[i] = out[t - 1 - i] within the sequence, else 0
  float P[L], acc[NCONV];
#pragma unroll
  for (int r = 0; r < NCONV; ++r) acc[r] = 0.f;
  {
    const int s0 = t0 % S;
#pragma unroll
    for (int i = 0; i < L; ++i) P[i] = s0 - 1 - i >= 0 ? ld1(out + (size_t)(t0 - 1 - i) * C + c) : 0.f;
  }
  for (int t = t0; t < t1; ++t) {
    const float o = ld1(out + (size_t)t * C + c);
#pragma unroll
    for (int q = 1; q < 4; ++q) {
      const int off = q == 1 ? 0 : q == 2 ? 4 : 12;
      const float gq = dg[((size_t)t * 4 + q) * C];
      acc[off] = fmaf(gq, o, acc[off]);
#pragma unroll
      for (int i = 1; i < 4 * q; ++i) acc[off + i] = fmaf(gq, P[i - 1], acc[off + i]);
    }
    const bool last = (t + 1) % S == 0;   // t + 1 starts a new sequence
#pragma unroll
    for (int i = L - 1; i > 0; --i) P[i] = last ? 0.f : P[i - 1];
    P[0] = last ? 0.f : o;
  }
#pragma unroll
  for (int r = 0; r < NCONV; ++r) a.part[((size_t)blockIdx.y * NCONV + r) * C + c] = acc[r];
}

// out[i] = sum over nch partial arrays of part[ch][i], minus corr[i % ncol]
// for the first ncorr columns.
__global__ __launch_bounds__(BT) void bwd_reduce_kernel(const float* __restrict__ part, int nch, long n,
                                                       float* __restrict__ out, const float* __restrict__ corr,
                                                       int ncol, int ncorr) {
  const long i = (long)blockIdx.x * BT + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int ch = 0; ch < nch; ++ch) s += part[(size_t)ch * n + i];
  if (ncorr > 0) {
    const int col = (int)(i % ncol);
    if (col < ncorr) s -= corr[col];
  }
  out[i] = s;
}

// Column sums of W_full's router columns, first stage: workgroup b sums the
// rows b, b + nblk, ... of columns 0..N-1 into part[b][n] (the second stage is
// bwd_reduce_kernel over the nblk partials).
template <class E>
__global__ __launch_bounds__(BT) void bwd_wcolsum_kernel(const typename E::T* __restrict__ W, long R, int ncol,
                                                         int N, float* __restrict__ part) {
  __shared__ float s_tmp[BT / WAVE][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float acc[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) acc[n] = 0.f;
  for (long row = (long)blockIdx.x * BT + threadIdx.x; row < R; row += (long)gridDim.x * BT) {
#pragma unroll
    for (int n = 0; n < 16; ++n)
      if (n < N) acc[n] += ld1(W + (size_t)row * ncol + n);
  }
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    const float v = wave_sum(acc[n]);
    if (lane == 0) s_tmp[wave][n] = v;
  }
  __syncthreads();
  if (threadIdx.x < N) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < BT / WAVE; ++w) v += s_tmp[w][threadIdx.x];
    part[(size_t)blockIdx.x * N + threadIdx.x] = v;
  }
}

// Column sums of the per-token rows [T][ncols]: column col of the bias / scale
// block goes to its destination (d_b_pre, d_b_res, d_b_post, d_alpha; the
// router correction sums stay in sums).
struct BwdSumArgs {
  const float* rows;
  long T;
  int ncols, N, KK, KKR;
  float *d_b_pre, *d_b_res, *d_b_post, *d_alpha, *sums;
};
__global__ __launch_bounds__(BT) void bwd_sum_rows_kernel(BwdSumArgs a) {
  __shared__ float s_tmp[BT / WAVE];
  const int col = blockIdx.x;
  float v = 0.f;
  for (long t = threadIdx.x; t < a.T; t += BT) v += a.rows[(size_t)t * a.ncols + col];
  v = block_sum(v, s_tmp);
  if (threadIdx.x != 0) return;
  a.sums[col] = v;
  int c = col;
  if (c < a.N) { a.d_b_pre[c] = v; return; }
  c -= a.N;
  if (c < a.KK) { a.d_b_res[c] = v; return; }
  c -= a.KK;
  if (c < a.KKR) { a.d_b_post[c] = v; return; }
  c -= a.KKR;
  if (c < 3) a.d_alpha[c] = v;
}

struct BwdTokArgs {
  const float* gstat;             // from xhc_pre, per token: raw pre-map logits [N], sum x, sum x^2
  const float *part_a, *stats_a;  // active-row raw logits [KSa][T][NPA], sums [KSa][T][2]
  int KSa, NPA;
  const int* idx;
  const float *p, *h_pre, *h_post, *z;
  const float *d_hpre, *d_hres, *d_hpost, *d_p;
  const float *b_res, *colsum;
  float a_pre, a_res, a_post, eps;
  int iters, m, T, C;
  float *Gt, *Ga, *sc, *brow;
  float* rsel;                    // [T][N]: H_pre[n] for a stream outside the active list, -1 - (its position) for one in it
};

// Generation half, per-token scalars.  16 lanes per token: lane (a, b) < k^2
// carries the tangent of the Sinkhorn map along its logit (a, b) and returns
// that logit's gradient; the token's lanes then form the coefficient rows
//   Gt = [dz / (sigma + eps) | alpha_pre g_pre / rho]   (router | pre-map),
//   Ga = [alpha_res dL | alpha_post g_post] / rho_a      (active maps),
// the per-token scalars cx, c0 (full state) and cxa (active rows) of the norm
// backward, dx = W Gt + cx x + c0, dx_a = W_act Ga + cxa x_a, and its share
// of the bias / scale gradients and of the router's mean correction.
template <int N, int K, int KR>
__global__ __launch_bounds__(BT) void bwd_token_kernel(BwdTokArgs a) {
  constexpr int KK = K * K, NA = KK + K * KR, NBT = 2 * N + KK + K * KR + 3;
  const int tl = threadIdx.x >> 4, l = threadIdx.x & 15;
  const int t = blockIdx.x * 16 + tl;
  const bool valid = t < a.T;
  const int tt = valid ? t : 0;
  __shared__ float s_la[16][32], s_dL[16][16];
  const float KC = (float)K * (float)a.C;
  float s2a = 0.f;
  for (int ks = 0; ks < a.KSa; ++ks) s2a += a.stats_a[((size_t)ks * a.T + tt) * 2 + 1];
  const float rhoa = sqrtf(s2a / KC + a.eps);
  for (int col = l; col < NA; col += 16) {
    float v = 0.f;
    for (int ks = 0; ks < a.KSa; ++ks) v += a.part_a[((size_t)ks * a.T + tt) * a.NPA + col];
    s_la[tl][col] = v / rhoa;
  }
  __syncthreads();
  if (l < KK) {
    const int ra = l / K, rb = l % K;
    float M[K][K], dM[K][K], mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < K; ++i)
#pragma unroll
      for (int j = 0; j < K; ++j) {
        M[i][j] = fmaf(a.a_res, s_la[tl][i * K + j], a.b_res[i * K + j]);
        mx = fmaxf(mx, M[i][j]);
      }
#pragma unroll
    for (int i = 0; i < K; ++i)
#pragma unroll
      for (int j = 0; j < K; ++j) {
        M[i][j] = expf(M[i][j] - mx);
        dM[i][j] = (i == ra && j == rb) ? M[i][j] : 0.f;
      }
    for (int it = 0; it < a.iters; ++it) {
#pragma unroll
      for (int j = 0; j < K; ++j) {
        float cs = 0.f, dcs = 0.f;
#pragma unroll
        for (int i = 0; i < K; ++i) { cs += M[i][j]; dcs += dM[i][j]; }
#pragma unroll
        for (int i = 0; i < K; ++i) {
          const float mv = M[i][j] / cs;
          dM[i][j] = (dM[i][j] - mv * dcs) / cs;
          M[i][j] = mv;
        }
      }
#pragma unroll
      for (int i = 0; i < K; ++i) {
        float rs = 0.f, drs = 0.f;
#pragma unroll
        for (int j = 0; j < K; ++j) { rs += M[i][j]; drs += dM[i][j]; }
#pragma unroll
        for (int j = 0; j < K; ++j) {
          const float mv = M[i][j] / rs;
          dM[i][j] = (dM[i][j] - mv * drs) / rs;
          M[i][j] = mv;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < K; ++i) {
      float rs = 0.f, drs = 0.f;
#pragma unroll
      for (int j = 0; j < K; ++j) { rs += M[i][j]; drs += dM[i][j]; }
      if (rs > 1.f) {
#pragma unroll
        for (int j = 0; j < K; ++j) {
          const float mv = M[i][j] / rs;
          dM[i][j] = (dM[i][j] - mv * drs) / rs;
          M[i][j] = mv;
        }
      }
    }
    float dl = 0.f;
#pragma unroll
    for (int i = 0; i < K; ++i)
#pragma unroll
      for (int j = 0; j < K; ++j) dl = fmaf(a.d_hres[(size_t)tt * KK + i * K + j], dM[i][j], dl);
    s_dL[tl][l] = dl;
  }
  __syncthreads();
  // the rest with the token's 16 lanes: lane l takes stream l (N <= 16) and
  // active-map entries l (k^2 <= 16, k K_r <= 16); sums over lanes by the
  // group butterfly, so every lane holds the same scalars
  const float NC = (float)N * (float)a.C;
  const float* gs = a.gstat + (size_t)tt * (N + 2);
  const float s1 = gs[N], s2 = gs[N + 1];
  const float mu = s1 / NC, ms = s2 / NC;
  const float rho = sqrtf(ms + a.eps);
  const float sig = sqrtf(fmaxf(ms - mu * mu, 0.f));
  const float sh = sig + a.eps;
  float* gt = a.Gt + (size_t)tt * 2 * N;
  float* br = a.brow + (size_t)tt * NBT;
  float* ga = a.Ga + (size_t)tt * NA;
  // pre-map: H_pre = sigmoid(alpha_pre y + b_pre), y = (x W_pre) / rho;
  // router: p_i = sigmoid(z_{I_i}) for the routed positions i >= m
  float sdy = 0.f, apre = 0.f, sdz = 0.f, cs = 0.f;
  if (l < N) {
    const int n = l;
    const float y = gs[n] / rho;
    const float h = a.h_pre[(size_t)tt * N + n];
    const float gp = a.d_hpre[(size_t)tt * N + n] * h * (1.f - h);
    const float dy = a.a_pre * gp;
    sdy = dy * y;
    apre = gp * y;
    float dz = 0.f;
    for (int i = a.m; i < K; ++i)
      if (a.idx[(size_t)tt * K + i] == n) {
        const float pv = a.p[(size_t)tt * K + i];
        dz += a.d_p[(size_t)tt * K + i] * pv * (1.f - pv);
      }
    sdz = dz * a.z[(size_t)tt * N + n];
    const float gr = dz / sh;
    cs = gr * a.colsum[n];
    int pos = -1;
    for (int i = 0; i < K; ++i)
      if (a.idx[(size_t)tt * K + i] == n) pos = i;
    if (valid) {
      a.rsel[(size_t)tt * N + n] = pos >= 0 ? -1.f - (float)pos : h;
      gt[N + n] = dy / rho;
      br[n] = gp;
      gt[n] = gr;
      br[NBT - N + n] = mu * gr;
    }
  }
  // active maps: H_res = rowclamp(SK(alpha_res la_res + b_res)),
  // H_post = 2 sigmoid(alpha_post la_post + b_post), la = (x_a W_act) / rho_a
  float sdl = 0.f, ares = 0.f, apost = 0.f;
  if (l < KK) {
    const float dL = s_dL[tl][l];
    const float dla = a.a_res * dL;
    sdl = dla * s_la[tl][l];
    ares = dL * s_la[tl][l];
    if (valid) {
      ga[l] = dla / rhoa;
      br[N + l] = dL;
    }
  }
  if (l < K * KR) {
    const float sg = 0.5f * a.h_post[(size_t)tt * K * KR + l];
    const float gpo = a.d_hpost[(size_t)tt * K * KR + l] * 2.f * sg * (1.f - sg);
    const float dla = a.a_post * gpo;
    sdl = fmaf(dla, s_la[tl][KK + l], sdl);
    apost = gpo * s_la[tl][KK + l];
    if (valid) {
      ga[KK + l] = dla / rhoa;
      br[N + KK + l] = gpo;
    }
  }
  sdy = group_sum<16>(sdy);
  apre = group_sum<16>(apre);
  sdz = group_sum<16>(sdz);
  cs = group_sum<16>(cs);
  sdl = group_sum<16>(sdl);
  ares = group_sum<16>(ares);
  apost = group_sum<16>(apost);
  if (l != 0 || !valid) return;
  const float cxr = sig > 0.f ? -sdz / (sh * NC * sig) : 0.f;
  const float cx = -sdy / (rho * rho * NC) + cxr;
  const float c0 = -cxr * mu - cs / NC;
  br[N + NA] = apre;
  br[N + NA + 1] = ares;
  br[N + NA + 2] = apost;
  const float cxa = -sdl / (rhoa * rhoa * KC);
  a.sc[(size_t)t * 4 + 0] = cx;
  a.sc[(size_t)t * 4 + 1] = c0;
  a.sc[(size_t)t * 4 + 2] = cxa;
  a.sc[(size_t)t * 4 + 3] = mu;
}

struct BwdRowArgs {
  const void* X;      // rows source [T][R]: the state (full) or the gathered active rows
  const void* W;      // [R][ncol] state dtype
  const float* G;     // [T][ncol]
  const float* sc;    // [T][4]
  void* dX;           // [T][N][C] written (full mode: rows outside the active list; active mode: the active rows)
  const void* d_X;    // [T][N][C] the new state's gradient (full mode; may be dX)
  const int* idx;     // active lists
  const float* rsel;  // [T][N]: H_pre[n] if stream n is outside token t's active list, else -1 - its position
  float* part;        // [nch][R][ncol]
  const void* dinp;   // [T][C] the sublayer input's gradient (full mode)
  const float* h_pre;           // [T][N] (full mode)
  float* dxa;         // [T][K][C] float: the active rows' state gradient between the two passes
  long R;
  int ncol, T, TW, N, K, C, act;
};

// dX += W G_t + c x (+ c0) row by row, and the weight-gradient partials
// sum_t x_t[row] G_t over this workgroup's token range (for the router
// columns of the full state, the centred x_t[row] - mu_t, so that no mean
// correction is subtracted afterwards).  Each thread owns two
// adjacent rows of the contraction (same stream, adjacent channels) with
// their weights in registers; the coefficient rows of 64 tokens at a time
// are staged in LDS.  Full mode: rows of the flattened state, c = cx, plus
// c0.  Active mode: rows of the gathered active state, c = cxa, scattered to
// stream I_t[j].
template <class E, int CM>
__global__ __launch_bounds__(BT) void bwd_rows_kernel(BwdRowArgs a) {
  using T = typename E::T;
  const long r0 = ((long)blockIdx.x * BT + threadIdx.x) * 2;
  const bool own = r0 < a.R;
  const int t0 = blockIdx.y * a.TW;
  const int t1 = t0 + a.TW < a.T ? t0 + a.TW : a.T;
  __shared__ float s_g[64][CM];
  __shared__ float s_c[64][3];
  const T* W = reinterpret_cast<const T*>(a.W);
  const T* X = reinterpret_cast<const T*>(a.X);
  T* dX = reinterpret_cast<T*>(a.dX);
  float w0[CM], w1[CM], acc0[CM], acc1[CM];
#pragma unroll
  for (int q = 0; q < CM; ++q) {
    w0[q] = (own && q < a.ncol) ? ld1(W + (size_t)r0 * a.ncol + q) : 0.f;
    w1[q] = (own && q < a.ncol) ? ld1(W + (size_t)(r0 + 1) * a.ncol + q) : 0.f;
    acc0[q] = acc1[q] = 0.f;
  }
  const int j = own ? (int)(r0 / a.C) : 0;
  const int c = own ? (int)(r0 % a.C) : 0;
  for (int tb = t0; tb < t1; tb += 64) {
    const int nt = t1 - tb < 64 ? t1 - tb : 64;
    __syncthreads();
    for (int u = threadIdx.x; u < 64 * CM; u += BT) {
      const int tu = u / CM, q = u % CM;
      s_g[tu][q] = (tu < nt && q < a.ncol) ? a.G[(size_t)(tb + tu) * a.ncol + q] : 0.f;
    }
    if (threadIdx.x < 64) {
      const int tu = threadIdx.x;
      s_c[tu][0] = tu < nt ? a.sc[(size_t)(tb + tu) * 4 + (a.act ? 2 : 0)] : 0.f;
      s_c[tu][1] = (tu < nt && !a.act) ? a.sc[(size_t)(tb + tu) * 4 + 1] : 0.f;
      s_c[tu][2] = (tu < nt && !a.act) ? a.sc[(size_t)(tb + tu) * 4 + 3] : 0.f;
    }
    __syncthreads();
    if (!own) continue;
    const int ncen = a.act ? 0 : a.N;   // centred (router) columns
    for (int u = 0; u < nt; ++u) {
      const int t = tb + u;
      const T* xr = X + (size_t)t * a.R + r0;
      const float x0 = ld1(xr), x1 = ld1(xr + 1);
      float d0 = fmaf(s_c[u][0], x0, s_c[u][1]), d1 = fmaf(s_c[u][0], x1, s_c[u][1]);
      const float m0 = x0 - s_c[u][2], m1 = x1 - s_c[u][2];
#pragma unroll
      for (int q = 0; q < CM; ++q) {
        const float g = s_g[u][q];
        d0 = fmaf(g, w0[q], d0);
        d1 = fmaf(g, w1[q], d1);
        acc0[q] = fmaf(q < ncen ? m0 : x0, g, acc0[q]);
        acc1[q] = fmaf(q < ncen ? m1 : x1, g, acc1[q]);
      }
      if (a.act) {
        // the active row's gradient so far (float), plus this pass's terms, stored once
        const float* pa = a.dxa + ((size_t)t * a.K + j) * a.C + c;
        T* dr = dX + ((size_t)t * a.N + a.idx[(size_t)t * a.K + j]) * a.C + c;
        st1(dr, pa[0] + d0);
        st1(dr + 1, pa[1] + d1);
      } else {
        // plus the application half's share: for a row outside the active
        // list d_X + H_pre[n] d_inp, stored once; an active row's share is
        // already in float in the backward workspace (kept there for the
        // active-row pass)
        const float h = a.rsel[(size_t)t * a.N + j];
        if (h >= 0.f) {
          const T* di = reinterpret_cast<const T*>(a.dinp) + (size_t)t * a.C + c;
          const T* dy = reinterpret_cast<const T*>(a.d_X) + (size_t)t * a.R + r0;
          T* dr = dX + (size_t)t * a.R + r0;
          st1(dr, ld1(dy) + fmaf(h, ld1(di), d0));
          st1(dr + 1, ld1(dy + 1) + fmaf(h, ld1(di + 1), d1));
        } else {
          float* pa = a.dxa + ((size_t)t * a.K + (int)(-1.f - h)) * a.C + c;
          pa[0] += d0;
          pa[1] += d1;
        }
      }
    }
  }
  if (!own) return;
  float* pp = a.part + ((size_t)blockIdx.y * a.R + r0) * a.ncol;
  for (int q = 0; q < a.ncol; ++q) {
    pp[q] = acc0[q];
    pp[a.ncol + q] = acc1[q];
  }
}

// bf16 form of the pass above on MFMA 16x16x32 tiles.  Workgroup: 4 waves x
// 64 rows (four 16-row tiles per wave), tokens in blocks of 32.  Per block,
// the coefficient rows are staged in LDS as bf16 hi + lo pairs (G = hi + lo to
// about 2^-17 relative; both halves go through the MFMA, so the products
// keep float accuracy), in token-major and column-major copies, and the
// state rows of the workgroup transposed to [row][token]:
//   dX tile (16 tokens x 16 rows) = G (16 x 32 columns) . W^T, A = G rows,
//       B = the wave's W rows (registers for the whole launch), then
//       + c x + c0 and the read-modify-write of dX;
//   dW^T tile (16 columns x 16 rows) += G^T (16 x 32 tokens) . X (32 x 16),
//       accumulated in registers over the token range.
template <int NR>
__global__ __launch_bounds__(BT) void bwd_rows_mfma_kernel(BwdRowArgs a) {
  constexpr int TB = 32;            // tokens per block
  constexpr int RW = 16 * NR;       // rows per wave
  constexpr int XS = 4 * RW + 8;    // LDS row stride (elements) of the state tile [token][row]
  constexpr int DS = 4 * RW + 4;    // LDS row stride of the product tile [token][row]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  const long rwg = (long)blockIdx.x * 4 * RW;   // first row of the workgroup
  const int t0 = blockIdx.y * a.TW;
  const int t1 = t0 + a.TW < a.T ? t0 + a.TW : a.T;
  __shared__ __align__(16) uint16_t s_x[TB][XS];
  __shared__ __align__(16) uint16_t s_g[2][TB][32];    // [hi/lo][token][column]
  __shared__ __align__(16) uint16_t s_gt[2][32][TB];   // [hi/lo][column][token]
  __shared__ float s_c[TB][2];
  __shared__ __align__(16) float s_d[16][DS];          // W G for 16 tokens
  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.W);
  const uint16_t* X = reinterpret_cast<const uint16_t*>(a.X);
  uint16_t* dX = reinterpret_cast<uint16_t*>(a.dX);
  const int ncol = a.ncol;
  // B fragments of the wave's W rows: lane (g, r) of tile j holds W[row][8g .. 8g + 7]
  uint4 bw[NR];
  bool tile_in[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const long row = rwg + (long)wave * RW + 16 * j + r;
    tile_in[j] = rwg + (long)wave * RW + 16 * j < a.R;   // R is a multiple of 32: tiles are whole
    union { uint16_t h[8]; uint4 u; } f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int col = 8 * g + e;
      f.h[e] = (tile_in[j] && col < ncol) ? W[(size_t)row * ncol + col] : (uint16_t)0;
    }
    bw[j] = f.u;
  }
  f32x4_t accw[NR][2];
#pragma unroll
  for (int j = 0; j < NR; ++j) accw[j][0] = accw[j][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Each thread moves 4 chunks of 8 rows of one token per block: chunk k is
  // token (tid + 256 k) / 32, rows 8 ((tid + 256 k) % 32); chunks 0-1 fall in
  // the block's first 16 tokens, 2-3 in the second.  The next block's state
  // chunks and this block's dX chunks are loaded ahead of the compute.
  constexpr int NCH = TB * (4 * RW / 8) / BT;   // 4
  static_assert(NCH == 4, "chunk mapping assumes 4 chunks per thread");
  // Full mode also takes each chunk's H_pre or position in the active list
  // one block ahead, so that the gradient loads need not wait for it.
  // The block's coefficient rows (thread u: token u / 8, columns 4 (u % 8)
  // .. + 3) and per-token scalars come with its state chunks, a block ahead.
  uint4 xn[NCH];
  float hn[NCH];
  float gn[4], scn[2] = {0.f, 0.f};
  auto load_x = [&](int tb, int nt) {
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int u = threadIdx.x + BT * k;
      const int tu = u / (4 * RW / 8), rc = (u % (4 * RW / 8)) * 8;
      const long row = rwg + rc;
      const bool in = tu < nt && row < a.R;
      xn[k] = in ? ld16(X + (size_t)(tb + tu) * a.R + row) : make_uint4(0, 0, 0, 0);
      if (!a.act) hn[k] = in ? a.rsel[(tb + tu) * a.N + (int)(row / a.C)] : 0.f;
    }
    const int tu = threadIdx.x >> 3, c4 = (threadIdx.x & 7) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      gn[e] = (tu < nt && c4 + e < ncol) ? a.G[(size_t)(tb + tu) * ncol + c4 + e] : 0.f;
    if (threadIdx.x < TB) {
      const int t = threadIdx.x;
      scn[0] = t < nt ? a.sc[(size_t)(tb + t) * 4 + (a.act ? 2 : 0)] : 0.f;
      scn[1] = (t < nt && !a.act) ? a.sc[(size_t)(tb + t) * 4 + 1] : 0.f;
    }
  };
  if (t0 < t1) load_x(t0, t1 - t0 < TB ? t1 - t0 : TB);
  for (int tb = t0; tb < t1; tb += TB) {
    const int nt = t1 - tb < TB ? t1 - tb : TB;
    __syncthreads();
    // this block's gradient chunks first, so that their latency runs under
    // the staging and the products below.  Full mode: d_X and d_inp for a row
    // outside the active list, the float gradient so far for one in it.
    // Active mode: the active row's float gradient so far.
    uint16_t* dr[NCH];
    uint4 dv[NCH], fv[NCH];
    int pos[NCH];
    float hp[NCH];
    bool own[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int u = threadIdx.x + BT * k;
      const int tu = u / (4 * RW / 8), rc = (u % (4 * RW / 8)) * 8;
      const long row = rwg + rc;
      own[k] = tu < nt && row < a.R;
      const int t = tb + (own[k] ? tu : 0);
      const long rr = own[k] ? row : 0;
      const int rj = (int)(rr / a.C), rcol = (int)(rr % a.C);
      if (a.act) {
        dr[k] = dX + ((size_t)t * a.N + a.idx[(size_t)t * a.K + rj]) * a.C + rcol;
        pos[k] = rj;
      } else {
        dr[k] = dX + (size_t)t * a.R + rr;
        hp[k] = hn[k];
        pos[k] = (own[k] && hp[k] < 0.f) ? (int)(-1.f - hp[k]) : -1;
      }
      if (pos[k] >= 0) {
        // an active row: its float gradient so far
        const float* pa = a.dxa + ((size_t)t * a.K + pos[k]) * a.C + rcol;
        dv[k] = own[k] ? ld16(pa) : make_uint4(0, 0, 0, 0);
        fv[k] = own[k] ? ld16(pa + 4) : make_uint4(0, 0, 0, 0);
      } else {
        // a row outside the active list: d_X and d_inp
        dv[k] = own[k] ? ld16(reinterpret_cast<const uint16_t*>(a.d_X) + (size_t)t * a.R + rr)
                       : make_uint4(0, 0, 0, 0);
        fv[k] = own[k] ? ld16(reinterpret_cast<const uint16_t*>(a.dinp) + (size_t)t * a.C + rcol)
                       : make_uint4(0, 0, 0, 0);
      }
    }
    // state rows as they are in memory (loaded during the previous block)
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int u = threadIdx.x + BT * k;
      *reinterpret_cast<uint4*>(&s_x[u / (4 * RW / 8)][(u % (4 * RW / 8)) * 8]) = xn[k];
    }
    // coefficients (loaded during the previous block)
    {
      const int tu = threadIdx.x >> 3, c4 = (threadIdx.x & 7) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int col = c4 + e;
        const float v = gn[e];
        const uint32_t hi = f32_to_bf16(v);
        const uint32_t lo = f32_to_bf16(v - __uint_as_float(hi << 16));
        s_g[0][tu][col] = (uint16_t)hi;
        s_g[1][tu][col] = (uint16_t)lo;
        s_gt[0][col][tu] = (uint16_t)hi;
        s_gt[1][col][tu] = (uint16_t)lo;
      }
      if (threadIdx.x < TB) {
        s_c[threadIdx.x][0] = scn[0];
        s_c[threadIdx.x][1] = scn[1];
      }
    }
    // then the next block's state chunks and coefficients
    if (tb + TB < t1) load_x(tb + TB, t1 - tb - TB < TB ? t1 - tb - TB : TB);
    __syncthreads();
    // weight gradient: dW^T[col][row] += sum over the block's tokens; the B
    // fragment (8 tokens of one row) is gathered from the token-major tile
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      if (!tile_in[j]) continue;
      union { uint16_t h[8]; uint4 u; } f;
      const int rl = wave * RW + 16 * j + r;
#pragma unroll
      for (int e = 0; e < 8; ++e) f.h[e] = s_x[8 * g + e][rl];
#pragma unroll
      for (int m = 0; m < 2; ++m) {   // both column tiles: columns past ncol are zero in LDS
        const uint4 ah = *reinterpret_cast<const uint4*>(&s_gt[0][16 * m + r][8 * g]);
        const uint4 al = *reinterpret_cast<const uint4*>(&s_gt[1][16 * m + r][8 * g]);
        accw[j][m] = Bf16::mma(Bf16::mma(accw[j][m], ah, f.u), al, f.u);
      }
    }
    // state gradient, 16 tokens at a time: products into LDS, then the
    // 16-byte read-modify-writes, dX += W G + c x + c0
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (16 * h >= nt) break;   // uniform over the workgroup
      const uint4 ah = *reinterpret_cast<const uint4*>(&s_g[0][16 * h + r][8 * g]);
      const uint4 al = *reinterpret_cast<const uint4*>(&s_g[1][16 * h + r][8 * g]);
      if (h) __syncthreads();    // the previous half's products have been read
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const f32x4_t acc = Bf16::mma(Bf16::mma(f32x4_t{0.f, 0.f, 0.f, 0.f}, ah, bw[j]), al, bw[j]);
#pragma unroll
        for (int i = 0; i < 4; ++i) s_d[4 * g + i][wave * RW + 16 * j + r] = acc[i];
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int k = 2 * h + kk;
        if (!own[k]) continue;
        const int u = threadIdx.x + BT * k;
        const int tl = u / (4 * RW / 8), rc = (u % (4 * RW / 8)) * 8;
        float v[8], x[8];
        Bf16::unpack(*reinterpret_cast<const uint4*>(&s_x[tl][rc]), x);
        const float cx = s_c[tl][0], c0 = s_c[tl][1];
        const int t = tb + tl;
        if (pos[k] >= 0) {
          // an active row: its float gradient so far plus this pass's terms;
          // the active-row pass rounds it once, after adding its own
          v[0] = __uint_as_float(dv[k].x); v[1] = __uint_as_float(dv[k].y);
          v[2] = __uint_as_float(dv[k].z); v[3] = __uint_as_float(dv[k].w);
          v[4] = __uint_as_float(fv[k].x); v[5] = __uint_as_float(fv[k].y);
          v[6] = __uint_as_float(fv[k].z); v[7] = __uint_as_float(fv[k].w);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] += s_d[tl - 16 * h][rc + e] + fmaf(cx, x[e], c0);
          if (a.act) {
            st16(dr[k], Bf16::pack(v));
          } else {
            const long rr = rwg + rc;
            float* pa = a.dxa + ((size_t)t * a.K + pos[k]) * a.C + rr % a.C;
            *reinterpret_cast<float4*>(pa) = make_float4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<float4*>(pa + 4) = make_float4(v[4], v[5], v[6], v[7]);
          }
        } else {
          // a row outside the active list: d_X + H_pre d_inp + this pass's terms, rounded once
          float fi[8];
          Bf16::unpack(fv[k], fi);
          Bf16::unpack(dv[k], v);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] += fmaf(hp[k], fi[e], s_d[tl - 16 * h][rc + e] + fmaf(cx, x[e], c0));
          st16(dr[k], Bf16::pack(v));
        }
      }
    }
  }
  // partial weight gradients: lane (g, r) of tile (j, m) holds columns 16m + 4g + i of row 16j + r
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    if (!tile_in[j]) continue;
    const long row = rwg + (long)wave * RW + 16 * j + r;
    float* pp = a.part + ((size_t)blockIdx.y * a.R + row) * ncol;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = 16 * m + 4 * g + i;
        if (col < ncol) pp[col] = accw[j][m][i];
      }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

int clampi(long v, int lo, int hi) { return (int)(v < lo ? lo : v > hi ? hi : v); }

}  // namespace

bool make_bwd_plan(const Plan& P, BwdPlan* B) {
  BwdPlan q;
  const size_t T = (size_t)P.T, N = P.N, K = P.K, C = P.C, KR = P.KR;
  const size_t es = P.dtype == XHC_BF16 ? 2 : 4;
  const int KB = P.dtype == XHC_BF16 ? 32 : 16;
  q.NC = (long)N * (long)C;
  q.KC = (long)K * (long)C;
  q.ncol_f = 2 * P.N;
  q.ncol_a = P.K * P.K + P.K * P.KR;
  q.NTF = (q.ncol_f + 15) / 16;
  q.NTA = (q.ncol_a + 15) / 16;
  q.nkb_f = q.NC / KB;
  q.nkb_a = q.KC / KB;
  const long nblk_t = (P.T + 63) / 64;
  const long ks = nblk_t > 0 ? (1024 + nblk_t - 1) / nblk_t : 1;
  q.KSa = clampi(ks, 1, 8);
  if (q.KSa > q.nkb_a) q.KSa = (int)q.nkb_a;
  q.NBT = 2 * P.N + P.K * P.K + P.K * P.KR + 3;
  // token chunks of the row kernels: about 2048 workgroups, at least 64 tokens each
  const long maxch = (P.T + 63) / 64 > 0 ? (P.T + 63) / 64 : 1;
  // rows per workgroup: 256 for the bf16 MFMA pass, 512 for the float one
  const long rpw = P.dtype == XHC_BF16 ? 256 : 2 * BT;
  const long xf = (q.NC + rpw - 1) / rpw, xa = (q.KC + rpw - 1) / rpw;
  q.nch_f = clampi((2048 + xf - 1) / xf, 1, 64);
  if (q.nch_f > maxch) q.nch_f = (int)maxch;
  q.nch_a = clampi((2048 + xa - 1) / xa, 1, 64);
  if (q.nch_a > maxch) q.nch_a = (int)maxch;
  q.TW_f = (int)((P.T + q.nch_f - 1) / q.nch_f);
  q.TW_a = (int)((P.T + q.nch_a - 1) / q.nch_a);
  // conv-transpose token chunks: about 128 tokens each, at most 1024 chunks
  // (grid.y and the [chunk][24][C] partials stay bounded for any T)
  q.nch_c = clampi((P.T + 127) / 128, 1, 1024);
  q.TC = (int)((P.T + q.nch_c - 1) / q.nch_c);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = al256(off + bytes);
    return o;
  };
  q.o_dhpre = take(T * N * 4);
  q.o_dhres = take(T * K * K * 4);
  q.o_dhpost = take(T * K * KR * 4);
  q.o_dp = take(T * K * 4);
  q.o_xa = take(T * K * C * es);
  q.o_dxa = take(T * K * C * 4);
  q.o_dg = KR == 4 ? take(T * 4 * C * 4) : SIZE_MAX;
  q.o_cpart = KR == 4 ? take((size_t)q.nch_c * NCONV * C * 4) : SIZE_MAX;
  q.o_wpa = take((size_t)q.nkb_a * q.NTA * 64 * 16);
  q.o_parta = take((size_t)q.KSa * T * q.NTA * 16 * 4);
  q.o_statsa = take((size_t)q.KSa * T * 2 * 4);
  q.o_gt = take(T * q.ncol_f * 4);
  q.o_ga = take(T * q.ncol_a * 4);
  q.o_sc = take(T * 4 * 4);
  q.o_rsel = take(T * N * 4);
  q.o_brow = take(T * q.NBT * 4);
  q.o_bsum = take((size_t)q.NBT * 4);
  q.o_colsum = take(N * 4);
  q.o_colpart = take((size_t)NCOLB * N * 4);
  q.o_wpartf = take((size_t)q.nch_f * q.NC * q.ncol_f * 4);
  q.o_wparta = take((size_t)q.nch_a * q.KC * q.ncol_a * 4);
  q.total = T == 0 ? 0 : off;
  *B = q;
  return true;
}

namespace {

template <class E, int N, int K, int KR>
void apply_launch(const Plan& P, const BwdPlan& Bp, const xhc_weights* w, const void* X, const void* out,
                  const void* d_inp, const void* d_X, void* d_out, float* d_conv, const char* ws, char* bws,
                  hipStream_t st) {
  BwdApplyArgs a{};
  a.X = X;
  a.out = out;
  a.d_inp = d_inp;
  a.d_X = d_X;
  a.d_out = d_out;
  a.xa = bws + Bp.o_xa;
  a.dxa = reinterpret_cast<float*>(bws + Bp.o_dxa);
  a.dg = KR == 4 ? reinterpret_cast<float*>(bws + Bp.o_dg) : nullptr;
  a.conv_w = w->conv_w;
  a.idx = reinterpret_cast<const int*>(ws + P.o_idx);
  a.p = reinterpret_cast<const float*>(ws + P.o_p);
  a.h_pre = reinterpret_cast<const float*>(ws + P.o_hpre);
  a.h_res = reinterpret_cast<const float*>(ws + P.o_hres);
  a.h_post = reinterpret_cast<const float*>(ws + P.o_hpost);
  a.d_hpre = reinterpret_cast<float*>(bws + Bp.o_dhpre);
  a.d_hres = reinterpret_cast<float*>(bws + Bp.o_dhres);
  a.d_hpost = reinterpret_cast<float*>(bws + Bp.o_dhpost);
  a.d_p = reinterpret_cast<float*>(bws + Bp.o_dp);
  a.T = (int)P.T;
  a.S = P.S;
  a.C = P.C;
  a.use_mgs = P.use_mgs;
  a.eps_mgs = P.eps_mgs;
  bwd_apply_kernel<E, N, K, KR><<<(unsigned)(KR == 4 ? 8 * ((P.T + 7) / 8) : P.T), BT, 0, st>>>(a);
  if constexpr (KR == 4) {
    BwdConvArgs c{};
    c.dg = a.dg;
    c.out = out;
    c.conv_w = w->conv_w;
    c.d_out = d_out;
    c.part = reinterpret_cast<float*>(bws + Bp.o_cpart);
    c.T = (int)P.T;
    c.S = P.S;
    c.C = P.C;
    c.TC = Bp.TC;
    dim3 grid((P.C + BT - 1) / BT, Bp.nch_c);
    bwd_conv_kernel<E><<<grid, BT, 0, st>>>(c);
    const long n = (long)NCONV * P.C;
    bwd_reduce_kernel<<<(unsigned)((n + BT - 1) / BT), BT, 0, st>>>(c.part, Bp.nch_c, n, d_conv, nullptr, 1, 0);
  }
}

template <class E, int CM>
void rows_launch(const BwdRowArgs& a, int nch, hipStream_t st) {
  dim3 grid((unsigned)((a.R / 2 + BT - 1) / BT), nch);
  bwd_rows_kernel<E, CM><<<grid, BT, 0, st>>>(a);
}

template <class E>
void rows_dispatch(const BwdRowArgs& a, int nch, hipStream_t st) {
  if constexpr (std::is_same<E, Bf16>::value) {
    dim3 grid((unsigned)((a.R + 4 * 64 - 1) / (4 * 64)), nch);
    bwd_rows_mfma_kernel<4><<<grid, BT, 0, st>>>(a);
    return;
  }
  if (a.ncol <= 8) rows_launch<E, 8>(a, nch, st);
  else if (a.ncol <= 16) rows_launch<E, 16>(a, nch, st);
  else rows_launch<E, 32>(a, nch, st);
}

template <class E, int N, int K, int KR>
void gen_launch(const Plan& P, const BwdPlan& Bp, const xhc_weights* w, const void* X, const void* d_inp,
                const void* d_X, void* dX, const xhc_grads* g, const char* ws, char* bws, hipStream_t st) {
  const int dt = P.dtype;
  const int T = (int)P.T;
  float* parta = reinterpret_cast<float*>(bws + Bp.o_parta);
  float* statsa = reinterpret_cast<float*>(bws + Bp.o_statsa);
  const void* xa = bws + Bp.o_xa;
  // the full-state projection and sums were kept by xhc_pre; the active rows' are recomputed
  launch_pack_b(dt, w->w_act, Bp.nkb_a, Bp.ncol_a, Bp.NTA, bws + Bp.o_wpa, st);
  launch_projection(dt, Bp.NTA, xa, T, Bp.KC, bws + Bp.o_wpa, Bp.nkb_a, Bp.KSa, parta, statsa, st);
  float* colsum = reinterpret_cast<float*>(bws + Bp.o_colsum);
  float* cpart = reinterpret_cast<float*>(bws + Bp.o_colpart);
  bwd_wcolsum_kernel<E><<<NCOLB, BT, 0, st>>>(reinterpret_cast<const typename E::T*>(w->w_full), Bp.NC, Bp.ncol_f,
                                              N, cpart);
  bwd_reduce_kernel<<<1, BT, 0, st>>>(cpart, NCOLB, N, colsum, nullptr, 1, 0);
  BwdTokArgs a{};
  a.gstat = reinterpret_cast<const float*>(ws + P.o_gstat);
  a.part_a = parta;
  a.stats_a = statsa;
  a.KSa = Bp.KSa;
  a.NPA = Bp.NTA * 16;
  a.idx = reinterpret_cast<const int*>(ws + P.o_idx);
  a.p = reinterpret_cast<const float*>(ws + P.o_p);
  a.h_pre = reinterpret_cast<const float*>(ws + P.o_hpre);
  a.h_post = reinterpret_cast<const float*>(ws + P.o_hpost);
  a.z = reinterpret_cast<const float*>(ws + P.o_z);
  a.d_hpre = reinterpret_cast<const float*>(bws + Bp.o_dhpre);
  a.d_hres = reinterpret_cast<const float*>(bws + Bp.o_dhres);
  a.d_hpost = reinterpret_cast<const float*>(bws + Bp.o_dhpost);
  a.d_p = reinterpret_cast<const float*>(bws + Bp.o_dp);
  a.b_res = w->b_res;
  a.colsum = colsum;
  a.a_pre = w->alpha_pre;
  a.a_res = w->alpha_res;
  a.a_post = w->alpha_post;
  a.eps = P.eps_norm;
  a.iters = P.iters;
  a.m = P.m;
  a.T = T;
  a.C = P.C;
  a.Gt = reinterpret_cast<float*>(bws + Bp.o_gt);
  a.Ga = reinterpret_cast<float*>(bws + Bp.o_ga);
  a.sc = reinterpret_cast<float*>(bws + Bp.o_sc);
  a.brow = reinterpret_cast<float*>(bws + Bp.o_brow);
  a.rsel = reinterpret_cast<float*>(bws + Bp.o_rsel);
  bwd_token_kernel<N, K, KR><<<(T + 15) / 16, BT, 0, st>>>(a);
  BwdSumArgs s{};
  s.rows = a.brow;
  s.T = T;
  s.ncols = Bp.NBT;
  s.N = N;
  s.KK = K * K;
  s.KKR = K * KR;
  s.d_b_pre = g->d_b_pre;
  s.d_b_res = g->d_b_res;
  s.d_b_post = g->d_b_post;
  s.d_alpha = g->d_alpha;
  s.sums = reinterpret_cast<float*>(bws + Bp.o_bsum);
  bwd_sum_rows_kernel<<<Bp.NBT, BT, 0, st>>>(s);
  // full state
  BwdRowArgs r{};
  r.X = X;
  r.W = w->w_full;
  r.G = a.Gt;
  r.sc = a.sc;
  r.dX = dX;
  r.d_X = d_X;
  r.idx = a.idx;
  r.part = reinterpret_cast<float*>(bws + Bp.o_wpartf);
  r.R = Bp.NC;
  r.ncol = Bp.ncol_f;
  r.T = T;
  r.TW = Bp.TW_f;
  r.N = N;
  r.K = K;
  r.C = P.C;
  r.act = 0;
  r.dinp = d_inp;
  r.h_pre = reinterpret_cast<const float*>(ws + P.o_hpre);
  r.dxa = reinterpret_cast<float*>(bws + Bp.o_dxa);
  r.rsel = a.rsel;
  rows_dispatch<E>(r, Bp.nch_f, st);
  const long nf = Bp.NC * Bp.ncol_f;
  // the bf16 pass accumulates uncentred rows: subtract sum_t mu_t G_t from the router columns
  const int ncorr = std::is_same<E, Bf16>::value ? N : 0;
  bwd_reduce_kernel<<<(unsigned)((nf + BT - 1) / BT), BT, 0, st>>>(r.part, Bp.nch_f, nf, g->dW_full,
                                                                   s.sums + Bp.NBT - N, Bp.ncol_f, ncorr);
  // active rows
  BwdRowArgs ra = r;
  ra.X = xa;
  ra.W = w->w_act;
  ra.G = a.Ga;
  ra.part = reinterpret_cast<float*>(bws + Bp.o_wparta);
  ra.R = Bp.KC;
  ra.ncol = Bp.ncol_a;
  ra.TW = Bp.TW_a;
  ra.act = 1;
  rows_dispatch<E>(ra, Bp.nch_a, st);
  const long na = Bp.KC * Bp.ncol_a;
  bwd_reduce_kernel<<<(unsigned)((na + BT - 1) / BT), BT, 0, st>>>(ra.part, Bp.nch_a, na, g->dW_act, nullptr, 1, 0);
}

template <class E, int KR>
bool apply_shape(const Plan& P, const BwdPlan& Bp, const xhc_weights* w, const void* X, const void* out,
                 const void* d_inp, const void* d_X, void* d_out, float* d_conv, const char* ws, char* bws,
                 hipStream_t st) {
#define XHC_BWD_APPLY(n, k) \
  if (P.N == n && P.K == k) { \
    apply_launch<E, n, k, KR>(P, Bp, w, X, out, d_inp, d_X, d_out, d_conv, ws, bws, st); \
    return true; \
  }
  XHC_BWD_APPLY(16, 4)
  XHC_BWD_APPLY(16, 2)
  XHC_BWD_APPLY(8, 4)
  XHC_BWD_APPLY(4, 4)
  XHC_BWD_APPLY(1, 1)
#undef XHC_BWD_APPLY
  return false;
}

template <class E, int KR>
bool gen_shape(const Plan& P, const BwdPlan& Bp, const xhc_weights* w, const void* X, const void* d_inp,
               const void* d_X, void* dX, const xhc_grads* g, const char* ws, char* bws, hipStream_t st) {
#define XHC_BWD_GEN(n, k) \
  if (P.N == n && P.K == k) { \
    gen_launch<E, n, k, KR>(P, Bp, w, X, d_inp, d_X, dX, g, ws, bws, st); \
    return true; \
  }
  XHC_BWD_GEN(16, 4)
  XHC_BWD_GEN(16, 2)
  XHC_BWD_GEN(8, 4)
  XHC_BWD_GEN(4, 4)
  XHC_BWD_GEN(1, 1)
#undef XHC_BWD_GEN
  return false;
}

}  // namespace

bool launch_xhc_post_backward(const Plan& P, const xhc_weights* w, const void* X, const void* out, const void* d_inp,
                              const void* d_X, void* d_out, float* d_conv, const char* ws, char* bws, hipStream_t st) {
  BwdPlan Bp;
  make_bwd_plan(P, &Bp);
  if (P.dtype == XHC_BF16)
    return P.KR == 4 ? apply_shape<Bf16, 4>(P, Bp, w, X, out, d_inp, d_X, d_out, d_conv, ws, bws, st)
                     : apply_shape<Bf16, 1>(P, Bp, w, X, out, d_inp, d_X, d_out, d_conv, ws, bws, st);
  return P.KR == 4 ? apply_shape<F32, 4>(P, Bp, w, X, out, d_inp, d_X, d_out, d_conv, ws, bws, st)
                   : apply_shape<F32, 1>(P, Bp, w, X, out, d_inp, d_X, d_out, d_conv, ws, bws, st);
}

bool launch_xhc_pre_backward(const Plan& P, const xhc_weights* w, const void* X, const void* d_inp, const void* d_X,
                             void* dX, const xhc_grads* g, const char* ws, char* bws, hipStream_t st) {
  BwdPlan Bp;
  make_bwd_plan(P, &Bp);
  if (P.dtype == XHC_BF16)
    return P.KR == 4 ? gen_shape<Bf16, 4>(P, Bp, w, X, d_inp, d_X, dX, g, ws, bws, st)
                     : gen_shape<Bf16, 1>(P, Bp, w, X, d_inp, d_X, dX, g, ws, bws, st);
  return P.KR == 4 ? gen_shape<F32, 4>(P, Bp, w, X, d_inp, d_X, dX, g, ws, bws, st)
                   : gen_shape<F32, 1>(P, Bp, w, X, d_inp, d_X, dX, g, ws, bws, st);
}

}  // namespace xhc
