// xHC after the sublayer (gfx950): write basis, Gram-Schmidt, mix and the
// gated write of the k active rows, in place.
//
// After an MLP-type sublayer the write basis of a token is F's output plus
// three causal depthwise convolutions of it along the sequence (kernel sizes
// 4, 8, 12), made mutually orthogonal along C by modified Gram-Schmidt
// (explainer "xHC: sixteen residual streams, four written at a time",
// section "What xHC changes"; summary "小红书xHC：时序特征增强 + 稀疏写回",
// section 3.3).  Gram-Schmidt needs inner products over all C channels of a
// token before any channel can be written, so the work is done in two passes
// over the same tiling (a block = PT consecutive tokens x 1024 channels, a
// thread = 4 channels):
//
//   xhc_gram   the Gram matrix of [out, g1, g2, g3] per token, partial over
//              the block's channels (10 numbers per token and slice);
//   xhc_apply  Gram-Schmidt coefficients from the summed Gram matrix (the same
//              sequence of projections, carried out on coefficient vectors),
//              then for each of the k active rows
//                x_j <- sum_i H_res[j][i] x_i + p_j sum_r H_post[j][r] v_r,
//              written in place; the other N - k rows are never touched
//              (xHC paper "xHC: Expanded Hyper-Connections", paragraph
//              "Mapping application"; summary 3.4.3).
//
// Each thread keeps its conv weights and the last 11 rows of `out` for its
// channels in registers and slides along the tokens of its block, so `out`
// is read once per pass (plus an 11-row history at the start of a block).
// Attention-type sublayers (K_r = 1) skip the first pass.
#include <mutex>
#include <type_traits>

#include "xhc_device.hpp"
#include "xhc_internal.hpp"
#include "xhc_tile.hpp"

namespace xhc {

namespace {

template <class E>
__device__ __forceinline__ typename Quad<E>::V ldq(const typename E::T* p) {
  return *reinterpret_cast<const typename Quad<E>::V*>(p);
}
// The same through a buffer resource (a byte offset past its range reads zeros).
template <class E>
__device__ __forceinline__ typename Quad<E>::V ldq_rs(__amdgpu_buffer_rsrc_t rs, uint32_t off);
template <>
__device__ __forceinline__ Quad<Bf16>::V ldq_rs<Bf16>(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(Quad<Bf16>::V, ld_b64(rs, off));
}
template <>
__device__ __forceinline__ Quad<F32>::V ldq_rs<F32>(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(Quad<F32>::V, ld_b128(rs, off, 0));
}

__device__ __forceinline__ void load_conv_weights(const float* __restrict__ cw, int C, int c, bool act,
                                                  float (&w1)[4][4], float (&w2)[8][4], float (&w3)[12][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 v = act ? *reinterpret_cast<const float4*>(cw + (size_t)i * C + c) : make_float4(0, 0, 0, 0);
    w1[i][0] = v.x; w1[i][1] = v.y; w1[i][2] = v.z; w1[i][3] = v.w;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 v = act ? *reinterpret_cast<const float4*>(cw + (size_t)(4 + i) * C + c) : make_float4(0, 0, 0, 0);
    w2[i][0] = v.x; w2[i][1] = v.y; w2[i][2] = v.z; w2[i][3] = v.w;
  }
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    const float4 v = act ? *reinterpret_cast<const float4*>(cw + (size_t)(12 + i) * C + c) : make_float4(0, 0, 0, 0);
    w3[i][0] = v.x; w3[i][1] = v.y; w3[i][2] = v.z; w3[i][3] = v.w;
  }
}

// The history of `out` is a ring of HL = 12 rows (the longest conv kernel).
// Tokens are taken in periods of HL, unrolled, so every index below is a
// constant: the token at position q of a period writes its row to slot q,
// and its lag-i row sits in slot (q - i) mod HL.  Nothing is shifted.
constexpr int HL = 12;

// Start of a block, before its first token t0 (position s0 in its sequence):
// lag-(i+1) rows out[t0 - 1 - i] inside that sequence go to slot HL - 1 - i,
// zero before its start.
template <class E>
__device__ __forceinline__ void load_history(const typename E::T* __restrict__ out, int t0, int s0, int C, int c,
                                             bool act, float (&h)[HL][4]) {
  typename Quad<E>::V v[HL - 1];
#pragma unroll
  for (int i = 0; i < HL - 1; ++i) {
    if (act && i + 1 <= s0) v[i] = ldq<E>(out + (size_t)(t0 - 1 - i) * C + c);
    else v[i] = typename Quad<E>::V{};
  }
#pragma unroll
  for (int i = 0; i < HL - 1; ++i) Quad<E>::unpack(v[i], h[HL - 1 - i]);
#pragma unroll
  for (int e = 0; e < 4; ++e) h[0][e] = 0.f;
}

// Token at position Q of a period (position s in its sequence): a sequence
// start clears the history (block-uniform branch), then its row takes slot Q.
template <int Q>
__device__ __forceinline__ void push_history(float (&h)[HL][4], const float (&row)[4], int s) {
  if (s == 0) {
    asm volatile("");   // keeps this a (rare, uniform) branch rather than 48 selects per token
#pragma unroll
    for (int i = 0; i < HL; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) h[i][e] = 0.f;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) h[Q][e] = row[e];
}

// Basis [out, g1, g2, g3] for this thread's 4 channels, token at position Q:
// g_j = sum_{i < kappa_j} w_j[i] * out[t - i] (lag i; kappa = 4, 8, 12).
template <int Q>
__device__ __forceinline__ void conv_basis(const float (&h)[HL][4], const float (&w1)[4][4],
                                           const float (&w2)[8][4], const float (&w3)[12][4], float (&b)[4][4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    b[0][e] = h[Q][e];
    float g1 = 0.f, g2 = 0.f, g3 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) g1 = fmaf(w1[i][e], h[(Q - i + HL) % HL][e], g1);
#pragma unroll
    for (int i = 0; i < 8; ++i) g2 = fmaf(w2[i][e], h[(Q - i + HL) % HL][e], g2);
#pragma unroll
    for (int i = 0; i < 12; ++i) g3 = fmaf(w3[i][e], h[(Q - i + HL) % HL][e], g3);
    b[1][e] = g1;
    b[2][e] = g2;
    b[3][e] = g3;
  }
}

// Calls f(std::integral_constant<int, Q>) for Q = 0 .. HL - 1.
template <int Q = 0, class F>
__device__ __forceinline__ void for_period(F&& f) {
  if constexpr (Q < HL) {
    f(std::integral_constant<int, Q>{});
    for_period<Q + 1>(f);
  }
}

// Sum of the 10 Gram entries over the 64 lanes of a wave, as a reduce-scatter
// in doubles: each step halves the values a lane keeps and adds its
// partner's copy of them, so the work falls with every step.  On return a
// group of 4 lanes holds one total (wave_sum10_index says which).  Every
// exchange is a VALU lane operation on the two 32-bit halves of a double:
//   bit 5: v_permlane32_swap of value i (kept by lanes 0-31) and value 5 + i
//          (kept by lanes 32-63), i < 5, so one add finishes each pair;
//   bit 4: v_permlane16_swap, even rows keep one value, odd rows another:
//          pairs (0, 3), (1, 4) of the five, and value 2 with itself (both
//          rows keep it);
//   bit 3: DPP row shifts by 8: lanes 0-7 of a row keep the first pair's
//          value, lanes 8-15 the second's; value 2 goes to lanes 0-7;
//   bit 2: DPP row shifts by 4: lanes 0-3 of an 8-lane group keep the value
//          from bit 3, lanes 4-7 value 2 (meaningful where bit 3 is 0);
//   bits 1, 0: DPP quad permutations (all 4 lanes end with the total).
// The DPP moves write every lane (lanes whose source lies outside the row
// read zero and are never selected), so no register has to be cleared first.
constexpr int DPP_ROW_SHL8 = 0x108, DPP_ROW_SHR8 = 0x118, DPP_ROW_SHL4 = 0x104, DPP_ROW_SHR4 = 0x114;
constexpr int DPP_QUAD_XOR2 = 0x4e, DPP_QUAD_XOR1 = 0xb1;   // quad_perm [2,3,0,1], [1,0,3,2]
__device__ __forceinline__ uint32_t lo32(double x) { return (uint32_t)__double2loint(x); }
__device__ __forceinline__ uint32_t hi32(double x) { return (uint32_t)__double2hiint(x); }
__device__ __forceinline__ double mk_d(uint32_t lo, uint32_t hi) { return __hiloint2double((int)hi, (int)lo); }
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
  const uint32_t l = (uint32_t)__builtin_amdgcn_mov_dpp((int)lo32(x), CTRL, 0xf, 0xf, true);
  const uint32_t h = (uint32_t)__builtin_amdgcn_mov_dpp((int)hi32(x), CTRL, 0xf, 0xf, true);
  return mk_d(l, h);
}
// x (kept where lane bit 5 is 0) and y (kept where it is 1), each plus its copy in the other half
__device__ __forceinline__ double swap32_add(double x, double y) {
  const auto rl = __builtin_amdgcn_permlane32_swap(lo32(x), lo32(y), false, false);
  const auto rh = __builtin_amdgcn_permlane32_swap(hi32(x), hi32(y), false, false);
  return mk_d(rl[0], rh[0]) + mk_d(rl[1], rh[1]);
}
// the same for lane bit 4 (even and odd rows of 16 lanes)
__device__ __forceinline__ double swap16_add(double x, double y) {
  const auto rl = __builtin_amdgcn_permlane16_swap(lo32(x), lo32(y), false, false);
  const auto rh = __builtin_amdgcn_permlane16_swap(hi32(x), hi32(y), false, false);
  return mk_d(rl[0], rh[0]) + mk_d(rl[1], rh[1]);
}

__device__ __forceinline__ double wave_sum10_d(const double (&v)[10], int lane) {
  double a[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) a[i] = swap32_add(v[i], v[5 + i]);
  const double b0 = swap16_add(a[0], a[3]), b1 = swap16_add(a[1], a[4]), b2 = swap16_add(a[2], a[2]);
  const bool u8 = (lane & 8) != 0, u4 = (lane & 4) != 0;
  const double c0lo = b0 + dpp_d<DPP_ROW_SHL8>(b0);
  const double c0hi = b1 + dpp_d<DPP_ROW_SHR8>(b1);
  const double c1 = b2 + dpp_d<DPP_ROW_SHL8>(b2);
  const double c0 = u8 ? c0hi : c0lo;
  const double dlo = c0 + dpp_d<DPP_ROW_SHL4>(c0);
  const double dhi = c1 + dpp_d<DPP_ROW_SHR4>(c1);
  double x = u4 ? dhi : dlo;
  x += dpp_d<DPP_QUAD_XOR2>(x);
  x += dpp_d<DPP_QUAD_XOR1>(x);
  return x;
}

// Index of the total wave_sum10_d leaves in this lane, or -1 (no total, or a
// copy of one another lane group holds).
__device__ __forceinline__ int wave_sum10_index(int lane) {
  const int h5 = (lane >> 5) & 1, h4 = (lane >> 4) & 1, h3 = (lane >> 3) & 1, h2 = (lane >> 2) & 1;
  if (h2 == 0) return (h3 ? (h4 ? 4 : 1) : (h4 ? 3 : 0)) + 5 * h5;
  return (h3 == 0 && h4 == 0) ? 2 + 5 * h5 : -1;
}

// Modified Gram-Schmidt on coefficient vectors: v_j = sum_a Tm[j][a] basis_a,
// with <x, y> = x^T G y (G = Gram matrix of the basis).  The same sequence
// of projections and the same eps as on the vectors themselves (summary
// 3.3), so the result is exact in real arithmetic.  Done in double, on a
// Gram matrix accumulated in double from exact products of the float basis:
// with nearly parallel branches the coefficients are large and cancel, and
// float Gram entries would lose the residuals.
__device__ __forceinline__ void mgs_from_gram(const double (&G)[4][4], double eps, double (&Tm)[4][4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int b = 0; b < 4; ++b) Tm[j][b] = (j == b) ? 1.0 : 0.0;
#pragma unroll
  for (int j = 1; j < 4; ++j) {
    double u[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) u[b] = (j == b) ? 1.0 : 0.0;
#pragma unroll
    for (int i = 0; i < j; ++i) {
      double Gt[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        double s = 0.0;
#pragma unroll
        for (int y = 0; y < 4; ++y) s = fma(G[x][y], Tm[i][y], s);
        Gt[x] = s;
      }
      double num = 0.0, den = 0.0;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        num = fma(u[x], Gt[x], num);
        den = fma(Tm[i][x], Gt[x], den);
      }
      const double cf = num / (den + eps);
#pragma unroll
      for (int x = 0; x < 4; ++x) u[x] = fma(-cf, Tm[i][x], u[x]);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) Tm[j][b] = u[b];
  }
}

// The per-token write coefficients Q[j][b] = p_j sum_r H_post[j][r] Tm[r][b]
// (Tm the Gram-Schmidt map, identity without it), in double, rounded once.
template <int KR>
__device__ __forceinline__ void write_coeffs(const double (&Tm)[4][4], const float* hpo, float pj, float* q) {
#pragma unroll
  for (int b = 0; b < KR; ++b) {
    double s = 0.0;
#pragma unroll
    for (int r = 0; r < KR; ++r) s = fma((double)hpo[r], Tm[r][b], s);
    q[b] = (float)((double)pj * s);
  }
}

#ifndef XHC_GRAM_GB
#define XHC_GRAM_GB 4
#endif
constexpr int GB = XHC_GRAM_GB;   // tokens per load batch in the Gram pass (HL is a multiple)
static_assert(HL % GB == 0, "load batches tile a history period");

}  // namespace

// Gram matrix of [out, g1, g2, g3] per token over this block's channels.
template <class E>
__global__ __launch_bounds__(256) void xhc_gram_kernel(XhcPostArgs a) {
  using T = typename E::T;
  using Qd = Quad<E>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slice = blockIdx.y;
  const int c = slice * PSLICE + tid * PCH;
  const bool act = c < a.C;
  const int cc = act ? c : 0;
  const int t0 = blockIdx.x * PT;
  const int t1 = min(t0 + PT, a.T);
  const T* __restrict__ out = reinterpret_cast<const T*>(a.out);
  __shared__ double s_g[PT][4][10];

  float w1[4][4], w2[8][4], w3[12][4];
  load_conv_weights(a.conv_w, a.C, cc, act, w1, w2, w3);
  float h[HL][4];
  load_history<E>(out, t0, t0 % a.S, a.C, cc, act, h);
  const int myidx = wave_sum10_index(lane);

  // The block's rows of out through a resource that ends at its last token,
  // so that the batch loaded ahead past it reads zeros (as does a lane past
  // C).  Batches of GB rows are loaded one batch ahead of their use.
  const __amdgpu_buffer_rsrc_t ro =
      make_rsrc(out + (size_t)t0 * a.C, (uint32_t)((size_t)(t1 - t0) * a.C * sizeof(T)));
  const uint32_t lo = act ? (uint32_t)(cc * sizeof(T)) : OUT_OF_RANGE;
  const uint32_t rowb = (uint32_t)(a.C * sizeof(T));
  typename Qd::V cur[GB], nxt[GB];
#pragma unroll
  for (int u = 0; u < GB; ++u) nxt[u] = ldq_rs<E>(ro, lo + (uint32_t)u * rowb);

  // sequence position of the next token, kept in a scalar register so that
  // the clearing at a sequence start is a branch, not per-element selects
  int s = __builtin_amdgcn_readfirstlane(t0 % a.S);
  for (int tp = t0; tp < t1; tp += HL) {
    for_period([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      const int t = tp + q;
      if constexpr (q % GB == 0) {
#pragma unroll
        for (int u = 0; u < GB; ++u) {
          cur[u] = nxt[u];
          nxt[u] = ldq_rs<E>(ro, lo + (uint32_t)(t - t0 + GB + u) * rowb);
        }
      }
      if (t < t1) {
        float r[4];
        Qd::unpack(cur[q % GB], r);
        push_history<q>(h, r, s);
        s = s + 1 == a.S ? 0 : s + 1;
        float b[4][4];
        conv_basis<q>(h, w1, w2, w3, b);
        // products of floats are exact in double
        double pr[10];
        int k = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = u; v < 4; ++v) {
            double d = 0.0;
#pragma unroll
            for (int e = 0; e < 4; ++e) d = fma((double)b[u][e], (double)b[v][e], d);
            pr[k++] = d;
          }
        const double tot = wave_sum10_d(pr, lane);
        if ((lane & 3) == 0 && myidx >= 0) s_g[t - t0][wave][myidx] = tot;
      }
    });
  }
  __syncthreads();
  for (int u = tid; u < (t1 - t0) * 10; u += 256) {
    const int tau = u / 10, j = u % 10;
    a.gram[((size_t)slice * a.T + t0 + tau) * 10 + j] =
        (s_g[tau][0][j] + s_g[tau][1][j]) + (s_g[tau][2][j] + s_g[tau][3][j]);
  }
}

// Mix + gated write of the k active rows, in place.  PB tokens per load batch.
// MODE 0: full xHC's write.  MODE 2: no residual mix (H_res = I), the
// unmixed writes of xHC-Flash (xHC paper, "xHC-Flash", Eq. 18, and the
// "Four-sublayer extension").  MODE 1 (xHC-Flash attention write, K_r = 1):
// MODE 2, and the MLP base readout inp_m gains a out with
// a = sum_j H_pre^MLP[I_j] p_j H_post_j (Eq. 19), read and rewritten in the
// same pass over out.
template <class E, int K, int KR, int PB, int MODE = 0>
__global__ __launch_bounds__(256) void xhc_apply_kernel(XhcPostArgs a) {
  using T = typename E::T;
  using Qd = Quad<E>;
  const int tid = threadIdx.x;
  const int slice = blockIdx.y;
  const int c = slice * PSLICE + tid * PCH;
  const bool act = c < a.C;
  const int cc = act ? c : 0;
  const int t0 = blockIdx.x * PT;
  const int t1 = min(t0 + PT, a.T);
  T* __restrict__ X = reinterpret_cast<T*>(a.X);
  const T* __restrict__ out = reinterpret_cast<const T*>(a.out);
  __shared__ float s_Q[PT][K][KR];
  __shared__ float s_H[PT][K][K];
  __shared__ int s_I[PT][K];
  constexpr bool FL = MODE == 1, IDM = MODE != 0;
  __shared__ float s_A[FL ? PT : 1];
  static_assert(!FL || KR == 1, "the Flash attention write has one write component");

  // per-token coefficients: Q = diag(p) H_post Tm (Tm = Gram-Schmidt map)
  for (int tau = tid; tau < t1 - t0; tau += 256) {
    const int t = t0 + tau;
    double Tm[4][4];
    if (KR == 4 && a.use_mgs) {
      double pg[10];
#pragma unroll
      for (int j = 0; j < 10; ++j) pg[j] = 0.0;
      for (int sl = 0; sl < a.nslices; ++sl)
#pragma unroll
        for (int j = 0; j < 10; ++j) pg[j] += a.gram[((size_t)sl * a.T + t) * 10 + j];
      double G[4][4];
      int q = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = u; v < 4; ++v) { G[u][v] = pg[q]; G[v][u] = pg[q]; ++q; }
      mgs_from_gram(G, (double)a.eps_mgs, Tm);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b) Tm[j][b] = (j == b) ? 1.0 : 0.0;
    }
    float acorr = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      int ij = a.idx[(size_t)t * K + j];
      ij = ij < 0 ? 0 : (ij >= a.N ? a.N - 1 : ij);
      s_I[tau][j] = ij;
      const float pj = a.p[(size_t)t * K + j];
#pragma unroll
      for (int i = 0; i < K; ++i) s_H[tau][j][i] = IDM ? (i == j ? 1.f : 0.f) : a.h_res[((size_t)t * K + j) * K + i];
      float hpo[KR];
#pragma unroll
      for (int r = 0; r < KR; ++r) hpo[r] = a.h_post[((size_t)t * K + j) * KR + r];
      if constexpr (FL) acorr = fmaf(a.h_pre_m[(size_t)t * a.N + ij] * pj, hpo[0], acorr);
      write_coeffs<KR>(Tm, hpo, pj, &s_Q[tau][j][0]);
    }
    if constexpr (FL) s_A[tau] = acorr;
  }
  __syncthreads();
  if (!act) return;

  // the k new rows of token t from its unpacked active rows and basis
  auto mix_store = [&](int t, const typename Qd::V (&xq)[K], const float (&b)[KR][4]) {
    const int tau = t - t0;
    float xa[K][4];
#pragma unroll
    for (int j = 0; j < K; ++j) Qd::unpack(xq[j], xa[j]);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      float nv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < K; ++i) sum = fmaf(s_H[tau][j][i], xa[i][e], sum);
#pragma unroll
        for (int v = 0; v < KR; ++v) sum = fmaf(s_Q[tau][j][v], b[v][e], sum);
        nv[e] = sum;
      }
      // streaming store: nothing reads the rewritten rows again in this pass
      __builtin_nontemporal_store(Qd::pack(nv),
                                  reinterpret_cast<typename Qd::V*>(X + ((size_t)t * a.N + s_I[tau][j]) * a.C + c));
    }
  };
  auto load_batch = [&](int tb, typename Qd::V (&orow)[PB], typename Qd::V (&xr)[PB][K]) {
#pragma unroll
    for (int q = 0; q < PB; ++q) {
      const int t = tb + q;
      const bool ok = t < t1;
      orow[q] = ok ? ldq<E>(out + (size_t)t * a.C + c) : typename Qd::V{};
#pragma unroll
      for (int j = 0; j < K; ++j)
        xr[q][j] = ok ? ldq<E>(X + ((size_t)t * a.N + s_I[t - t0][j]) * a.C + c) : typename Qd::V{};
    }
  };

  if constexpr (KR == 4) {
    // MLP-type: the basis needs the conv history; tokens in periods of HL
    static_assert(HL % PB == 0, "load batches tile a history period");
    float w1[4][4], w2[8][4], w3[12][4];
    float h[HL][4];
    load_conv_weights(a.conv_w, a.C, c, true, w1, w2, w3);
    load_history<E>(out, t0, t0 % a.S, a.C, c, true, h);
    // sequence position of the next token, kept in a scalar register so that
  // the clearing at a sequence start is a branch, not per-element selects
  int s = __builtin_amdgcn_readfirstlane(t0 % a.S);
    for (int tp = t0; tp < t1; tp += HL) {
      typename Qd::V orow[PB];
      typename Qd::V xr[PB][K];
      for_period([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        const int t = tp + q;
        if constexpr (q % PB == 0) load_batch(t, orow, xr);
        if (t < t1) {
          float r[4];
          Qd::unpack(orow[q % PB], r);
          push_history<q>(h, r, s);
          s = s + 1 == a.S ? 0 : s + 1;
          float b[KR][4];
          conv_basis<q>(h, w1, w2, w3, b);
          mix_store(t, xr[q % PB], b);
        }
      });
    }
  } else {
    T* __restrict__ inp_m = reinterpret_cast<T*>(a.inp_m);
    for (int tb = t0; tb < t1; tb += PB) {
      typename Qd::V orow[PB];
      typename Qd::V xr[PB][K];
      typename Qd::V mrow[FL ? PB : 1];
      load_batch(tb, orow, xr);
      if constexpr (FL) {
#pragma unroll
        for (int q = 0; q < PB; ++q) mrow[q] = tb + q < t1 ? ldq<E>(inp_m + (size_t)(tb + q) * a.C + c) : typename Qd::V{};
      }
#pragma unroll
      for (int q = 0; q < PB; ++q) {
        const int t = tb + q;
        if (t >= t1) break;
        float b[KR][4];
        Qd::unpack(orow[q], b[0]);
        mix_store(t, xr[q], b);
        if constexpr (FL) {
          float mv[4];
          Qd::unpack(mrow[q], mv);
          const float al = s_A[t - t0];
#pragma unroll
          for (int e = 0; e < 4; ++e) mv[e] = fmaf(al, b[0][e], mv[e]);
          __builtin_nontemporal_store(Qd::pack(mv), reinterpret_cast<typename Qd::V*>(inp_m + (size_t)t * a.C + c));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Single-token decode of the MLP-type write: one workgroup per sequence, whose
// new token's lag-i outputs (i = 1..11) come from a ring of 12 slots (slot
// s mod 12 holds the output of position s; positions before the sequence
// start are zero history).  The Gram matrix of the token's basis is reduced
// over all C channels inside the workgroup, so the write needs one launch;
// the new output then goes to slot step mod 12, which no lag of this token
// reads.
// ---------------------------------------------------------------------------
constexpr int DRING = 12;

struct DecodeArgs {
  void* X;
  const void* out;
  void* ring;
  const int* steps;
  int B, C, N;
  const int* idx;
  const float *p, *h_res, *h_post;
  const float* conv_w;
  int use_mgs;
  float eps_mgs;
};

// KR = 1 (attention-type, no history): the same per-token write without the
// ring, used for any batch too small to fill the device with 64-token blocks.
template <class E, int K, int KR>
__global__ __launch_bounds__(256) void xhc_decode_post_kernel(DecodeArgs a) {
  using T = typename E::T;
  using Qd = Quad<E>;
  static_assert(KR == 1 || KR == 4, "write components");
  __shared__ double s_g[4][10];
  __shared__ float s_Q[K][KR];
  __shared__ float s_H[K][K];
  __shared__ int s_I[K];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x, C = a.C;
  int step = KR == 4 ? a.steps[t] : 0;
  step = step < 0 ? 0 : step;
  T* __restrict__ X = reinterpret_cast<T*>(a.X);
  const T* __restrict__ out = reinterpret_cast<const T*>(a.out) + (size_t)t * C;
  T* __restrict__ ring = KR == 4 ? reinterpret_cast<T*>(a.ring) + (size_t)t * DRING * C : nullptr;

  // basis [out, g1, g2, g3] of channels c..c+3 of this token
  auto basis = [&](int c, float (&b)[KR][4]) {
    if constexpr (KR == 1) {
      Qd::unpack(ldq<E>(out + c), b[0]);
      return;
    }
    float w1[4][4], w2[8][4], w3[12][4];
    load_conv_weights(a.conv_w, C, c, true, w1, w2, w3);
    typename Qd::V v[DRING];
    v[0] = ldq<E>(out + c);
#pragma unroll
    for (int i = 1; i < DRING; ++i)
      v[i] = i <= step ? ldq<E>(ring + (size_t)((step - i) % DRING) * C + c) : typename Qd::V{};
    float h[DRING][4];
#pragma unroll
    for (int i = 0; i < DRING; ++i) Qd::unpack(v[i], h[i]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float g1 = 0.f, g2 = 0.f, g3 = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) g1 = fmaf(w1[i][e], h[i][e], g1);
#pragma unroll
      for (int i = 0; i < 8; ++i) g2 = fmaf(w2[i][e], h[i][e], g2);
#pragma unroll
      for (int i = 0; i < 12; ++i) g3 = fmaf(w3[i][e], h[i][e], g3);
      b[0][e] = h[0][e];
      b[KR > 1 ? 1 : 0][e] = g1;
      b[KR > 2 ? 2 : 0][e] = g2;
      b[KR > 3 ? 3 : 0][e] = g3;
    }
  };

  // pass 1: Gram matrix of the basis over all channels (fixed-order sums)
  if (KR == 4 && a.use_mgs) {
    double gr[10];
#pragma unroll
    for (int j = 0; j < 10; ++j) gr[j] = 0.0;
    for (int c = tid * PCH; c < C; c += 256 * PCH) {
      float b[KR][4];
      basis(c, b);
      int q = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = u; w < 4; ++w) {
          double d = 0.0;
#pragma unroll
          for (int e = 0; e < 4; ++e) d = fma((double)b[u][e], (double)b[w][e], d);   // exact products
          gr[q++] += d;
        }
    }
#pragma unroll
    for (int j = 0; j < 10; ++j) {
      double v = gr[j];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
      if (lane == 0) s_g[wave][j] = v;
    }
  }
  __syncthreads();
  if (tid == 0) {
    double Tm[4][4];
    if (KR == 4 && a.use_mgs) {
      double G[4][4];
      int q = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int w = u; w < 4; ++w) {
          const double v = (s_g[0][q] + s_g[1][q]) + (s_g[2][q] + s_g[3][q]);
          G[u][w] = v;
          G[w][u] = v;
          ++q;
        }
      mgs_from_gram(G, (double)a.eps_mgs, Tm);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b) Tm[j][b] = (j == b) ? 1.0 : 0.0;
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
      int ij = a.idx[(size_t)t * K + j];
      s_I[j] = ij < 0 ? 0 : (ij >= a.N ? a.N - 1 : ij);
      const float pj = a.p[(size_t)t * K + j];
#pragma unroll
      for (int i = 0; i < K; ++i) s_H[j][i] = a.h_res[((size_t)t * K + j) * K + i];
      float hpo[KR];
#pragma unroll
      for (int r = 0; r < KR; ++r) hpo[r] = a.h_post[((size_t)t * K + j) * KR + r];
      write_coeffs<KR>(Tm, hpo, pj, &s_Q[j][0]);
    }
  }
  __syncthreads();

  // pass 2: mix and gated write of the k active rows, then the ring slot
  for (int c = tid * PCH; c < C; c += 256 * PCH) {
    float b[KR][4];
    basis(c, b);
    typename Qd::V xq[K];
#pragma unroll
    for (int j = 0; j < K; ++j) xq[j] = ldq<E>(X + ((size_t)t * a.N + s_I[j]) * C + c);
    float xa[K][4];
#pragma unroll
    for (int j = 0; j < K; ++j) Qd::unpack(xq[j], xa[j]);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      float nv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < K; ++i) sum = fmaf(s_H[j][i], xa[i][e], sum);
#pragma unroll
        for (int v = 0; v < KR; ++v) sum = fmaf(s_Q[j][v], b[v][e], sum);
        nv[e] = sum;
      }
      *reinterpret_cast<typename Qd::V*>(X + ((size_t)t * a.N + s_I[j]) * C + c) = Qd::pack(nv);
    }
    if constexpr (KR == 4) *reinterpret_cast<typename Qd::V*>(ring + (size_t)(step % DRING) * C + c) = ldq<E>(out + c);
  }
}

template <class E, int KR>
static bool decode_launch(const DecodeArgs& a, int K, hipStream_t st) {
  switch (K) {
    case 4: xhc_decode_post_kernel<E, 4, KR><<<a.B, 256, 0, st>>>(a); return true;
    case 2: xhc_decode_post_kernel<E, 2, KR><<<a.B, 256, 0, st>>>(a); return true;
    case 1: xhc_decode_post_kernel<E, 1, KR><<<a.B, 256, 0, st>>>(a); return true;
    default: return false;
  }
}

template <class E, int K, int KR, int MODE = 0>
static void launch_apply(const XhcPostArgs& a, hipStream_t st) {
  dim3 grid((a.T + PT - 1) / PT, a.nslices);
  // tokens per load batch: measured best of 2, 3, 4, 6 for MLP-type bf16
  // (the batch divides the 12-token history period; fp32 rows are twice as
  // wide, so 4), and of 4, 8, 16 for attention-type
  constexpr int PB = KR == 4 ? (sizeof(typename E::T) == 2 ? 6 : 4) : 8;
  xhc_apply_kernel<E, K, KR, PB, MODE><<<grid, 256, 0, st>>>(a);
}

template <class E>
static bool xhc_post_launch(const Plan& P, void* X, const void* out, const xhc_weights* w, const char* ws,
                            double* gram, hipStream_t st) {
  XhcPostArgs a;
  a.X = X; a.out = out; a.T = (int)P.T; a.S = P.S; a.C = P.C; a.N = P.N; a.nslices = P.nslices;
  a.idx = reinterpret_cast<const int*>(ws + P.o_idx);
  a.p = reinterpret_cast<const float*>(ws + P.o_p);
  a.h_res = reinterpret_cast<const float*>(ws + P.o_hres);
  a.h_post = reinterpret_cast<const float*>(ws + P.o_hpost);
  a.conv_w = w->conv_w; a.use_mgs = P.use_mgs; a.eps_mgs = P.eps_mgs;
  a.gram = gram;
  if (P.KR == 1 && ((P.T + PT - 1) / PT) * P.nslices < 512) {
    // too few 64-token blocks to fill the device: one workgroup per token
    DecodeArgs d;
    d.X = X; d.out = out; d.ring = nullptr; d.steps = nullptr;
    d.B = (int)P.T; d.C = P.C; d.N = P.N;
    d.idx = a.idx; d.p = a.p; d.h_res = a.h_res; d.h_post = a.h_post;
    d.conv_w = nullptr; d.use_mgs = 0; d.eps_mgs = P.eps_mgs;
    return decode_launch<E, 1>(d, P.K, st);
  }
  if (P.KR == 4 && P.use_mgs) {
    dim3 grid((a.T + PT - 1) / PT, a.nslices);
    xhc_gram_kernel<E><<<grid, 256, 0, st>>>(a);
  }
  switch (P.K * 10 + P.KR) {
    case 41: launch_apply<E, 4, 1>(a, st); return true;
    case 44: launch_apply<E, 4, 4>(a, st); return true;
    case 21: launch_apply<E, 2, 1>(a, st); return true;
    case 24: launch_apply<E, 2, 4>(a, st); return true;
    case 11: launch_apply<E, 1, 1>(a, st); return true;
    case 14: launch_apply<E, 1, 4>(a, st); return true;
    default: return false;
  }
}

bool launch_xhc_post_decode(const Plan& P, void* X, const void* out, void* ring, const int* steps,
                            const xhc_weights* w, const char* ws, hipStream_t st) {
  DecodeArgs a;
  a.X = X; a.out = out; a.ring = ring; a.steps = steps;
  a.B = (int)P.T; a.C = P.C; a.N = P.N;
  a.idx = reinterpret_cast<const int*>(ws + P.o_idx);
  a.p = reinterpret_cast<const float*>(ws + P.o_p);
  a.h_res = reinterpret_cast<const float*>(ws + P.o_hres);
  a.h_post = reinterpret_cast<const float*>(ws + P.o_hpost);
  a.conv_w = w->conv_w; a.use_mgs = P.use_mgs; a.eps_mgs = P.eps_mgs;
  return P.dtype == XHC_BF16 ? decode_launch<Bf16, 4>(a, P.K, st) : decode_launch<F32, 4>(a, P.K, st);
}

// xHC-Flash attention write (Eq. 18) fused with the MLP input correction
// (Eq. 19); a.h_post holds H_post^Attn [T][K], a.h_pre_m H_pre^MLP [T][N].
template <class E>
static bool flash_attn_launch(const XhcPostArgs& a, int K, hipStream_t st) {
  dim3 grid((a.T + PT - 1) / PT, a.nslices);
  switch (K) {
    case 4: xhc_apply_kernel<E, 4, 1, 8, 1><<<grid, 256, 0, st>>>(a); return true;
    case 1: xhc_apply_kernel<E, 1, 1, 8, 1><<<grid, 256, 0, st>>>(a); return true;
    default: return false;
  }
}

bool launch_flash_attn_write(const Plan& P, void* X, const void* out, void* inp_m, const char* ws, hipStream_t st) {
  XhcPostArgs a{};
  a.X = X; a.out = out; a.T = (int)P.T; a.S = P.S; a.C = P.C; a.N = P.N; a.nslices = P.nslices;
  a.idx = reinterpret_cast<const int*>(ws + P.o_idx);
  a.p = reinterpret_cast<const float*>(ws + P.o_p);
  a.h_res = nullptr;
  a.h_post = reinterpret_cast<const float*>(ws + P.o_hpost_a);
  a.h_pre_m = reinterpret_cast<const float*>(ws + P.o_hpre_m);
  a.inp_m = inp_m;
  a.use_mgs = 0;
  return P.dtype == XHC_BF16 ? flash_attn_launch<Bf16>(a, P.K, st) : flash_attn_launch<F32>(a, P.K, st);
}

// The unmixed write of an intermediate xHC-Flash-4sub sublayer (H_res = I):
// K_r = 1 after attention, the temporal basis after the first MLP.
template <class E>
static bool unmixed_launch(const Plan& P, int KR, void* X, const void* out, const float* conv_w, char* ws,
                           hipStream_t st) {
  XhcPostArgs a{};
  a.X = X; a.out = out; a.T = (int)P.T; a.S = P.S; a.C = P.C; a.N = P.N; a.nslices = P.nslices;
  a.idx = reinterpret_cast<const int*>(ws + P.o_idx);
  a.p = reinterpret_cast<const float*>(ws + P.o_p);
  a.h_res = nullptr;
  a.h_post = reinterpret_cast<const float*>(ws + P.o_hpost);
  a.conv_w = conv_w; a.use_mgs = P.use_mgs; a.eps_mgs = P.eps_mgs;
  a.gram = reinterpret_cast<double*>(ws + P.o_gram);
  if (KR == 4 && P.use_mgs) {
    dim3 grid((a.T + PT - 1) / PT, a.nslices);
    xhc_gram_kernel<E><<<grid, 256, 0, st>>>(a);
  }
  switch (P.K * 10 + KR) {
    case 41: launch_apply<E, 4, 1, 2>(a, st); return true;
    case 44: launch_apply<E, 4, 4, 2>(a, st); return true;
    case 11: launch_apply<E, 1, 1, 2>(a, st); return true;
    case 14: launch_apply<E, 1, 4, 2>(a, st); return true;
    default: return false;
  }
}

bool launch_unmixed_write(const Plan& P, int KR, void* X, const void* out, const float* conv_w, char* ws,
                          hipStream_t st) {
  return P.dtype == XHC_BF16 ? unmixed_launch<Bf16>(P, KR, X, out, conv_w, ws, st)
                             : unmixed_launch<F32>(P, KR, X, out, conv_w, ws, st);
}

// Per-token write coefficients of an MLP-type sublayer for the persistent
// post pass: Q[j][b] = p_j sum_r H_post[j][r] Tm[r][b], Tm the Gram-Schmidt
// map from the summed Gram partials (identity without Gram-Schmidt), with
// the apply kernel's arithmetic (the same sums in the same order, the same
// double-precision map, rounded once), so that both writes give the same
// bits.  One thread per token.
struct WcoefArgs {
  int T, nslices, use_mgs;
  float eps_mgs;
  const double* gram;
  const float *p, *h_post;
  float* wq;   // [T][K][4]
};

template <int K>
__global__ __launch_bounds__(256) void xhc_wcoef_kernel(WcoefArgs a) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= a.T) return;
  double Tm[4][4];
  if (a.use_mgs) {
    double pg[10];
#pragma unroll
    for (int j = 0; j < 10; ++j) pg[j] = 0.0;
    for (int sl = 0; sl < a.nslices; ++sl)
#pragma unroll
      for (int j = 0; j < 10; ++j) pg[j] += a.gram[((size_t)sl * a.T + t) * 10 + j];
    double G[4][4];
    int q = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = u; v < 4; ++v) { G[u][v] = pg[q]; G[v][u] = pg[q]; ++q; }
    mgs_from_gram(G, (double)a.eps_mgs, Tm);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) Tm[j][b] = (j == b) ? 1.0 : 0.0;
  }
#pragma unroll
  for (int j = 0; j < K; ++j) {
    float hpo[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) hpo[r] = a.h_post[((size_t)t * K + j) * 4 + r];
    write_coeffs<4>(Tm, hpo, a.p[(size_t)t * K + j], a.wq + ((size_t)t * K + j) * 4);
  }
}

template <class E>
static void wcoef_launch(const Plan& P, const void* out, const xhc_weights* w, char* ws, hipStream_t st) {
  XhcPostArgs g{};
  g.out = out; g.T = (int)P.T; g.S = P.S; g.C = P.C; g.N = P.N; g.nslices = P.nslices;
  g.conv_w = w->conv_w; g.use_mgs = P.use_mgs; g.eps_mgs = P.eps_mgs;
  g.gram = reinterpret_cast<double*>(ws + P.o_gram);
  if (P.use_mgs) {
    dim3 grid((g.T + PT - 1) / PT, g.nslices);
    xhc_gram_kernel<E><<<grid, 256, 0, st>>>(g);
  }
  WcoefArgs a;
  a.T = (int)P.T; a.nslices = P.nslices; a.use_mgs = P.use_mgs; a.eps_mgs = P.eps_mgs;
  a.gram = g.gram;
  a.p = reinterpret_cast<const float*>(ws + P.o_p);
  a.h_post = reinterpret_cast<const float*>(ws + P.o_hpost);
  a.wq = reinterpret_cast<float*>(ws + P.o_wcoef);
  const unsigned nb = (unsigned)((P.T + 255) / 256);
  switch (P.K) {
    case 4: xhc_wcoef_kernel<4><<<nb, 256, 0, st>>>(a); break;
    case 2: xhc_wcoef_kernel<2><<<nb, 256, 0, st>>>(a); break;
    case 1: xhc_wcoef_kernel<1><<<nb, 256, 0, st>>>(a); break;
    default: break;
  }
}

void launch_xhc_wcoef(const Plan& P, const void* out, const xhc_weights* w, char* ws, hipStream_t st) {
  if (P.dtype == XHC_BF16) wcoef_launch<Bf16>(P, out, w, ws, st);
  else wcoef_launch<F32>(P, out, w, ws, st);
}

bool launch_xhc_post(const Plan& P, void* X, const void* out, const xhc_weights* w, char* ws, hipStream_t st) {
  double* gram = reinterpret_cast<double*>(ws + P.o_gram);
  return P.dtype == XHC_BF16 ? xhc_post_launch<Bf16>(P, X, out, w, ws, gram, st)
                             : xhc_post_launch<F32>(P, X, out, w, ws, gram, st);
}

size_t post_scratch_bytes(const Plan& P) {
  return (P.KR == 4 && P.use_mgs) ? (size_t)P.nslices * (size_t)P.T * 10 * sizeof(double) : 0;
}

}  // namespace xhc

// ---------------------------------------------------------------------------
// The write without allocation (xhc_post_noalloc): the Gram partials, the only
// memory the write needs beyond its inputs and outputs, live in this array,
// one copy per GPU (each device that runs the library holds its own until the
// process ends).  Calls that overlap on one GPU share it and race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) double scratch[XHC_NOALLOC_SCRATCH_BYTES / sizeof(double)];

namespace xhc {

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};
}  // namespace

// This device's address of `scratch`, looked up once per device with the
// device current.  Host code uses only this address, never the symbol itself.
hipError_t noalloc_scratch(double** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<double*>(g_scratch_ptr[dev]);
  return hipSuccess;
}

bool launch_xhc_post_noalloc(const Plan& P, void* X, const void* out, const xhc_weights* w, const char* ws,
                             double* scratch_ptr, hipStream_t st) {
  return P.dtype == XHC_BF16 ? xhc_post_launch<Bf16>(P, X, out, w, ws, scratch_ptr, st)
                             : xhc_post_launch<F32>(P, X, out, w, ws, scratch_ptr, st);
}

}  // namespace xhc
