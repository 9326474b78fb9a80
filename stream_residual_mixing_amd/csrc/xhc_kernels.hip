// libxhc kernels for gfx950.
//
// mHC pre stage (mapping generation + dense read):
//   pack_b      weights -> MFMA B fragments (once per call, a few MiB)
//   proj_gen    one pass over X: split-K bf16/f32 MFMA projection of the raw
//               (un-normalised) flattened state, plus sum x and sum x^2
//   mhc_read    per 16 tokens: RMS correction, H_pre / H_post, N x N
//               Sinkhorn, dense read -> inp
// (the xHC pre stage is the one-pass kernel of xhc_pre.hip)
// Post stage:
//   xhc_gram    MLP-type only: causal convolutions of out and the 4 x 4 Gram
//               matrix of [out, g1, g2, g3] per token (partial per C slice)
//   xhc_apply   Gram-Schmidt coefficients from the Gram matrix, then the
//               active rows' mix + gated write, in place
//   mhc_post    dense N x N mix + rank-1 write, in place
//
// Normalisations are applied after the projection, from sum x and sum x^2,
// so no normalised state is ever materialised (xHC paper "xHC: Expanded
// Hyper-Connections", paragraph "Mapping generation").
#include "xhc_device.hpp"
#include "xhc_internal.hpp"

namespace xhc {

// ---------------------------------------------------------------------------
// weight packing: fragment (kb, nt, lane = 16 g + col) holds
// W[kb*KB + VEC*g + e][nt*16 + col] for e < VEC (zero beyond ncol)
// ---------------------------------------------------------------------------
template <class E>
__global__ __launch_bounds__(256) void pack_b_kernel(const typename E::T* __restrict__ W, long nkb,
                                                     int ncol, int NT, uint4* __restrict__ out) {
  using T = typename E::T;
  const long f = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (f >= nkb * NT * WAVE) return;
  const int lane = (int)(f % WAVE);
  const long rest = f / WAVE;
  const int nt = (int)(rest % NT);
  const long kb = rest / NT;
  const int g = lane >> 4, col = nt * 16 + (lane & 15);
  union { T v[E::VEC]; uint4 u; } frag;
#pragma unroll
  for (int e = 0; e < E::VEC; ++e) {
    const long row = kb * E::KB + E::VEC * g + e;
    frag.v[e] = col < ncol ? W[row * ncol + col] : T(0);
  }
  out[f] = frag.u;
}

// ---------------------------------------------------------------------------
// proj_gen: block = 4 waves x 16 tokens, one K range (split-K over blockIdx.y).
// Lane (g, r) streams 16-byte fragments of token r's flattened row; the
// fragment is the A operand of one MFMA step and feeds the sum / sum-of-
// squares statistics.  Output: raw logits and the two sums per (split, token).
// ---------------------------------------------------------------------------
template <class E, int NT>
__global__ __launch_bounds__(256) void proj_gen_kernel(const typename E::T* __restrict__ X, int T, long K,
                                                       const uint4* __restrict__ Wp, long nkb, int KS,
                                                       float* __restrict__ part, float* __restrict__ stats) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int tok0 = blockIdx.x * 64 + wave * 16;
  const int ks = blockIdx.y;
  const long kb0 = (long)ks * nkb / KS, kb1 = (long)(ks + 1) * nkb / KS;
  const int tok = tok0 + r;
  const bool valid = tok < T;
  const typename E::T* xrow = X + (size_t)(valid ? tok : 0) * K + E::VEC * g;
  f32x4_t acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float s1 = 0.f, s2 = 0.f;
  const uint4* wp = Wp + lane;
  const uint4 zero = make_uint4(0, 0, 0, 0);

  auto step = [&](const uint4& a, long kb) {
    float f[E::VEC];
    E::unpack(a, f);
#pragma unroll
    for (int e = 0; e < E::VEC; ++e) { s1 += f[e]; s2 = fmaf(f[e], f[e], s2); }
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = E::mma(acc[n], a, wp[(kb * NT + n) * WAVE]);
  };

  constexpr int U = 4;
  long kb = kb0;
  for (; kb + U <= kb1; kb += U) {
    uint4 a[U];
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = valid ? ld16(xrow + (kb + u) * E::KB) : zero;
#pragma unroll
    for (int u = 0; u < U; ++u) step(a[u], kb + u);
  }
  for (; kb < kb1; ++kb) {
    const uint4 a = valid ? ld16(xrow + kb * E::KB) : zero;
    step(a, kb);
  }
  s1 += __shfl_xor(s1, 16, WAVE);
  s1 += __shfl_xor(s1, 32, WAVE);
  s2 += __shfl_xor(s2, 16, WAVE);
  s2 += __shfl_xor(s2, 32, WAVE);
  constexpr int NP = NT * 16;
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = tok0 + 4 * g + i;
      if (t < T) part[((size_t)ks * T + t) * NP + n * 16 + r] = acc[n][i];
    }
  if (g == 0 && valid) {
    stats[((size_t)ks * T + tok) * 2 + 0] = s1;
    stats[((size_t)ks * T + tok) * 2 + 1] = s2;
  }
}

constexpr int RT = 16;  // tokens per mHC read block

// ---------------------------------------------------------------------------
// mhc_read: block = 16 tokens.  N lanes per token (one row of H_res each)
// build the three maps; then the 4 waves split the channels for the dense read.
// ---------------------------------------------------------------------------
template <class E, int N>
__global__ __launch_bounds__(256) void mhc_read_kernel(MhcReadArgs a) {
  using T = typename E::T;
  constexpr int NTF = (2 * N + N * N + 15) / 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * RT;
  const int C = a.C;
  const T* __restrict__ X = reinterpret_cast<const T*>(a.X);
  T* __restrict__ inp = reinterpret_cast<T*>(a.inp);
  __shared__ float s_hpre[RT][N];

  constexpr int TPP = WAVE / N;
  constexpr int PASSES = (RT + TPP - 1) / TPP;
  for (int pass = wave; pass < PASSES; pass += 4) {
    const int tau = pass * TPP + lane / N;
    const int row = lane % N;
    const int t = t0 + tau;
    const bool valid = tau < RT && t < a.T;
    const int tc = valid ? t : 0;
    float pre = 0.f, post = 0.f, s2 = 0.f, L[N];
#pragma unroll
    for (int b = 0; b < N; ++b) L[b] = 0.f;
    for (int ks = 0; ks < a.KS; ++ks) {
      const float* pp = a.part + ((size_t)ks * a.T + tc) * (NTF * 16);
      pre += pp[row];
      post += pp[N + row];
#pragma unroll
      for (int b = 0; b < N; ++b) L[b] += pp[2 * N + row * N + b];
      s2 += a.stats[((size_t)ks * a.T + tc) * 2 + 1];
    }
    const float rr = 1.f / sqrtf(s2 / ((float)N * (float)C) + a.eps);
    const float hp = sigmoidf_(fmaf(a.a_pre * pre, rr, a.b_pre[row]));
    const float ho = 2.f * sigmoidf_(fmaf(a.a_post * post, rr, a.b_post[row]));
#pragma unroll
    for (int b = 0; b < N; ++b) L[b] = fmaf(a.a_res * L[b], rr, a.b_res[row * N + b]);
    sinkhorn_rows<N>(L, a.iters);
    if (valid) {
      a.h_pre[(size_t)t * N + row] = hp;
      a.h_post[(size_t)t * N + row] = ho;
#pragma unroll
      for (int b = 0; b < N; ++b) a.h_res[((size_t)t * N + row) * N + b] = L[b];
    }
    if (tau < RT) s_hpre[tau][row] = valid ? hp : 0.f;
  }
  __syncthreads();

  const int g = lane >> 4, r = lane & 15;
  const int t = t0 + r;
  const bool valid = t < a.T;
  const int tt = valid ? t : t0;
  float hp[N];
#pragma unroll
  for (int i = 0; i < N; ++i) hp[i] = s_hpre[r][i];
  const int nkbC = C / E::KB;
  const int kbA = wave * nkbC / 4, kbB = (wave + 1) * nkbC / 4;
  const T* xt = X + (size_t)tt * N * C + E::VEC * g;
  for (int kb = kbA; kb < kbB; ++kb) {
    const int c = kb * E::KB;
    float o[E::VEC];
#pragma unroll
    for (int e = 0; e < E::VEC; ++e) o[e] = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      float f[E::VEC];
      E::unpack(ld16(xt + (size_t)i * C + c), f);
#pragma unroll
      for (int e = 0; e < E::VEC; ++e) o[e] = fmaf(hp[i], f[e], o[e]);
    }
    if (valid) st16(inp + (size_t)t * C + c + E::VEC * g, E::pack(o));
  }
}

// ---------------------------------------------------------------------------
// post kernels: block = PT tokens x one slice of 256 threads x 4 channels.
// ---------------------------------------------------------------------------

// Causal depthwise convolutions of out for this thread's 4 channels at token t
// (position s in its sequence): g_j = sum_{i < kappa_j} w_j[i] * out[t - i],
// no history before the sequence start (explainer, "What xHC changes";
// summary 3.3).  Kernel sizes 4, 8, 12.
template <class E>
__device__ __forceinline__ void conv_basis(const typename E::T* __restrict__ out, int t, int s, int C, int c,
                                           const float (&w1)[4][4], const float (&w2)[8][4],
                                           const float (&w3)[12][4], float (&b)[4][4]) {
  using Qd = Quad<E>;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) b[q][e] = 0.f;
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    if (i <= s) {
      float o[4];
      Qd::unpack(*reinterpret_cast<const typename Qd::V*>(out + (size_t)(t - i) * C + c), o);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (i == 0) b[0][e] = o[e];
        if (i < 4) b[1][e] = fmaf(w1[i][e], o[e], b[1][e]);
        if (i < 8) b[2][e] = fmaf(w2[i][e], o[e], b[2][e]);
        b[3][e] = fmaf(w3[i][e], o[e], b[3][e]);
      }
    }
  }
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

// Gram matrix of [out, g1, g2, g3] per token over this block's channel slice.
template <class E>
__global__ __launch_bounds__(256) void xhc_gram_kernel(XhcPostArgs a) {
  using T = typename E::T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slice = blockIdx.y;
  const int c = slice * PSLICE + tid * PCH;
  const bool act = c < a.C;
  const int cc = act ? c : 0;
  const int t0 = blockIdx.x * PT;
  const T* __restrict__ out = reinterpret_cast<const T*>(a.out);
  float w1[4][4], w2[8][4], w3[12][4];
  load_conv_weights(a.conv_w, a.C, cc, act, w1, w2, w3);
  __shared__ float s_g[PT][4][10];
  for (int tau = 0; tau < PT; ++tau) {
    const int t = t0 + tau;
    if (t >= a.T) break;
    const int s = t % a.S;
    float b[4][4];
    conv_basis<E>(out, t, s, a.C, cc, w1, w2, w3, b);
    float pr[10];
    int q = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = u; v < 4; ++v) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) d = fmaf(b[u][e], b[v][e], d);
        pr[q++] = act ? d : 0.f;
      }
#pragma unroll
    for (int j = 0; j < 10; ++j) {
      const float sj = wave_sum(pr[j]);
      if (lane == 0) s_g[tau][wave][j] = sj;
    }
  }
  __syncthreads();
  for (int u = tid; u < PT * 10; u += 256) {
    const int tau = u / 10, j = u % 10;
    const int t = t0 + tau;
    if (t < a.T)
      a.gram[((size_t)slice * a.T + t) * 10 + j] = (s_g[tau][0][j] + s_g[tau][1][j]) + (s_g[tau][2][j] + s_g[tau][3][j]);
  }
}

// Modified Gram-Schmidt carried out on coefficient vectors: v_j = sum_a
// Tm[j][a] basis_a, with <x, y> = x^T G y (G = Gram matrix of the basis).
// Same sequence of projections and the same eps as on the vectors
// (summary 3.3); exact in real arithmetic.
__device__ __forceinline__ void mgs_from_gram(const float (&G)[4][4], float eps, float (&Tm)[4][4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int b = 0; b < 4; ++b) Tm[j][b] = (j == b) ? 1.f : 0.f;
#pragma unroll
  for (int j = 1; j < 4; ++j) {
    float u[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) u[b] = (j == b) ? 1.f : 0.f;
#pragma unroll
    for (int i = 0; i < j; ++i) {
      float Gt[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        float s = 0.f;
#pragma unroll
        for (int y = 0; y < 4; ++y) s = fmaf(G[x][y], Tm[i][y], s);
        Gt[x] = s;
      }
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        num = fmaf(u[x], Gt[x], num);
        den = fmaf(Tm[i][x], Gt[x], den);
      }
      const float cf = num / (den + eps);
#pragma unroll
      for (int x = 0; x < 4; ++x) u[x] = fmaf(-cf, Tm[i][x], u[x]);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) Tm[j][b] = u[b];
  }
}

// Mix + gated write of the k active rows, in place.
template <class E, int K, int KR>
__global__ __launch_bounds__(256) void xhc_apply_kernel(XhcPostArgs a) {
  using T = typename E::T;
  using Qd = Quad<E>;
  const int tid = threadIdx.x;
  const int slice = blockIdx.y;
  const int c = slice * PSLICE + tid * PCH;
  const bool act = c < a.C;
  const int cc = act ? c : 0;
  const int t0 = blockIdx.x * PT;
  T* __restrict__ X = reinterpret_cast<T*>(a.X);
  const T* __restrict__ out = reinterpret_cast<const T*>(a.out);
  __shared__ float s_Q[PT][K][KR];
  __shared__ float s_H[PT][K][K];
  __shared__ int s_I[PT][K];

  for (int tau = tid; tau < PT; tau += 256) {
    const int t = t0 + tau;
    if (t >= a.T) break;
    float Tm[4][4];
    if (KR == 4 && a.use_mgs) {
      float pg[10];
#pragma unroll
      for (int j = 0; j < 10; ++j) pg[j] = 0.f;
      for (int sl = 0; sl < a.nslices; ++sl)
#pragma unroll
        for (int j = 0; j < 10; ++j) pg[j] += a.gram[((size_t)sl * a.T + t) * 10 + j];
      float G[4][4];
      int q = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = u; v < 4; ++v) { G[u][v] = pg[q]; G[v][u] = pg[q]; ++q; }
      mgs_from_gram(G, a.eps_mgs, Tm);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b) Tm[j][b] = (j == b) ? 1.f : 0.f;
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
      int ij = a.idx[(size_t)t * K + j];
      ij = ij < 0 ? 0 : (ij >= a.N ? a.N - 1 : ij);
      s_I[tau][j] = ij;
      const float pj = a.p[(size_t)t * K + j];
#pragma unroll
      for (int i = 0; i < K; ++i) s_H[tau][j][i] = a.h_res[((size_t)t * K + j) * K + i];
      float hpo[KR];
#pragma unroll
      for (int r = 0; r < KR; ++r) hpo[r] = a.h_post[((size_t)t * K + j) * KR + r];
#pragma unroll
      for (int b = 0; b < KR; ++b) {
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < KR; ++r) s = fmaf(hpo[r], Tm[r][b], s);
        s_Q[tau][j][b] = pj * s;
      }
    }
  }
  __syncthreads();

  float w1[4][4], w2[8][4], w3[12][4];
  if (KR == 4) load_conv_weights(a.conv_w, a.C, cc, act, w1, w2, w3);
  if (!act) return;
  for (int tau = 0; tau < PT; ++tau) {
    const int t = t0 + tau;
    if (t >= a.T) break;
    float b[4][4];
    if (KR == 4) {
      conv_basis<E>(out, t, t % a.S, a.C, c, w1, w2, w3, b);
    } else {
      Qd::unpack(*reinterpret_cast<const typename Qd::V*>(out + (size_t)t * a.C + c), b[0]);
    }
    float xa[K][4];
#pragma unroll
    for (int j = 0; j < K; ++j)
      Qd::unpack(*reinterpret_cast<const typename Qd::V*>(X + ((size_t)t * a.N + s_I[tau][j]) * a.C + c), xa[j]);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      float nv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < K; ++i) s = fmaf(s_H[tau][j][i], xa[i][e], s);
#pragma unroll
        for (int q = 0; q < KR; ++q) s = fmaf(s_Q[tau][j][q], b[q][e], s);
        nv[e] = s;
      }
      *reinterpret_cast<typename Qd::V*>(X + ((size_t)t * a.N + s_I[tau][j]) * a.C + c) = Qd::pack(nv);
    }
  }
}

// mHC post: X_i <- sum_j H_res[i][j] X_j + H_post[i] out for every stream.
template <class E, int N>
__global__ __launch_bounds__(256) void mhc_post_kernel(MhcPostArgs a) {
  using T = typename E::T;
  using Qd = Quad<E>;
  constexpr int PTM = 32;
  const int tid = threadIdx.x;
  const int slice = blockIdx.y;
  const int c = slice * PSLICE + tid * PCH;
  const bool act = c < a.C;
  const int t0 = blockIdx.x * PTM;
  T* __restrict__ X = reinterpret_cast<T*>(a.X);
  const T* __restrict__ out = reinterpret_cast<const T*>(a.out);
  __shared__ float s_H[PTM][N][N];
  __shared__ float s_P[PTM][N];
  for (int u = tid; u < PTM * N * N; u += 256) {
    const int tau = u / (N * N), rest = u % (N * N);
    const int t = t0 + tau;
    s_H[tau][rest / N][rest % N] = t < a.T ? a.h_res[(size_t)t * N * N + rest] : 0.f;
  }
  for (int u = tid; u < PTM * N; u += 256) {
    const int tau = u / N, i = u % N;
    const int t = t0 + tau;
    s_P[tau][i] = t < a.T ? a.h_post[(size_t)t * N + i] : 0.f;
  }
  __syncthreads();
  if (!act) return;
  for (int tau = 0; tau < PTM; ++tau) {
    const int t = t0 + tau;
    if (t >= a.T) break;
    float x[N][4], o[4];
#pragma unroll
    for (int j = 0; j < N; ++j)
      Qd::unpack(*reinterpret_cast<const typename Qd::V*>(X + ((size_t)t * N + j) * a.C + c), x[j]);
    Qd::unpack(*reinterpret_cast<const typename Qd::V*>(out + (size_t)t * a.C + c), o);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      float nv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < N; ++j) s = fmaf(s_H[tau][i][j], x[j][e], s);
        nv[e] = fmaf(s_P[tau][i], o[e], s);
      }
      *reinterpret_cast<typename Qd::V*>(X + ((size_t)t * N + i) * a.C + c) = Qd::pack(nv);
    }
  }
}

// ---------------------------------------------------------------------------
// launchers (host side)
// ---------------------------------------------------------------------------
template <class E>
static void launch_pack(const void* W, long nkb, int ncol, int NT, void* out, hipStream_t st) {
  const long n = nkb * NT * WAVE;
  if (n == 0) return;
  pack_b_kernel<E><<<(unsigned)((n + 255) / 256), 256, 0, st>>>(reinterpret_cast<const typename E::T*>(W), nkb,
                                                                ncol, NT, reinterpret_cast<uint4*>(out));
}

template <class E, int NT>
static void launch_gen(const void* X, int T, long K, const void* Wp, long nkb, int KS, float* part, float* stats,
                       hipStream_t st) {
  dim3 grid((T + 63) / 64, KS);
  proj_gen_kernel<E, NT><<<grid, 256, 0, st>>>(reinterpret_cast<const typename E::T*>(X), T, K,
                                               reinterpret_cast<const uint4*>(Wp), nkb, KS, part, stats);
}

template <class E>
static bool gen_dispatch(int NT, const void* X, int T, long K, const void* Wp, long nkb, int KS, float* part,
                         float* stats, hipStream_t st) {
  switch (NT) {
    case 1: launch_gen<E, 1>(X, T, K, Wp, nkb, KS, part, stats, st); return true;
    case 2: launch_gen<E, 2>(X, T, K, Wp, nkb, KS, part, stats, st); return true;
    case 5: launch_gen<E, 5>(X, T, K, Wp, nkb, KS, part, stats, st); return true;
    case 18: launch_gen<E, 18>(X, T, K, Wp, nkb, KS, part, stats, st); return true;
    default: return false;
  }
}

template <class E, int K, int KR>
static void launch_xhc_apply(const XhcPostArgs& a, hipStream_t st) {
  dim3 grid((a.T + PT - 1) / PT, a.nslices);
  xhc_apply_kernel<E, K, KR><<<grid, 256, 0, st>>>(a);
}

template <class E, int N>
static void launch_mhc_read(const MhcReadArgs& a, hipStream_t st) {
  mhc_read_kernel<E, N><<<(a.T + RT - 1) / RT, 256, 0, st>>>(a);
}

template <class E, int N>
static void launch_mhc_post(const MhcPostArgs& a, hipStream_t st) {
  dim3 grid((a.T + 31) / 32, a.nslices);
  mhc_post_kernel<E, N><<<grid, 256, 0, st>>>(a);
}

template <class E>
static bool xhc_post_launch(const Plan& P, void* X, const void* out, const xhc_weights* w, char* ws, hipStream_t st) {
  XhcPostArgs a;
  a.X = X; a.out = out; a.T = (int)P.T; a.S = P.S; a.C = P.C; a.N = P.N; a.nslices = P.nslices;
  a.idx = reinterpret_cast<const int*>(ws + P.o_idx);
  a.p = reinterpret_cast<const float*>(ws + P.o_p);
  a.h_res = reinterpret_cast<const float*>(ws + P.o_hres);
  a.h_post = reinterpret_cast<const float*>(ws + P.o_hpost);
  a.conv_w = w->conv_w; a.use_mgs = P.use_mgs; a.eps_mgs = P.eps_mgs;
  a.gram = reinterpret_cast<float*>(ws + P.o_gram);
  if (P.KR == 4 && P.use_mgs) {
    dim3 grid((a.T + PT - 1) / PT, a.nslices);
    xhc_gram_kernel<E><<<grid, 256, 0, st>>>(a);
  }
  switch (P.K * 10 + P.KR) {
    case 41: launch_xhc_apply<E, 4, 1>(a, st); return true;
    case 44: launch_xhc_apply<E, 4, 4>(a, st); return true;
    case 21: launch_xhc_apply<E, 2, 1>(a, st); return true;
    case 24: launch_xhc_apply<E, 2, 4>(a, st); return true;
    case 11: launch_xhc_apply<E, 1, 1>(a, st); return true;
    case 14: launch_xhc_apply<E, 1, 4>(a, st); return true;
    default: return false;
  }
}

template <class E>
static bool mhc_pre_launch(const Plan& P, const void* X, void* inp, const xhc_weights* w, char* ws, hipStream_t st) {
  launch_pack<E>(w->w_full, P.nkb_full, P.ncol_full, P.NTF, ws + P.o_wfull, st);
  if (!gen_dispatch<E>(P.NTF, X, (int)P.T, (long)P.N * P.C, ws + P.o_wfull, P.nkb_full, P.KS,
                       reinterpret_cast<float*>(ws + P.o_part), reinterpret_cast<float*>(ws + P.o_stats), st))
    return false;
  MhcReadArgs a;
  a.X = X; a.inp = inp; a.T = (int)P.T; a.C = P.C; a.KS = P.KS;
  a.part = reinterpret_cast<const float*>(ws + P.o_part);
  a.stats = reinterpret_cast<const float*>(ws + P.o_stats);
  a.b_pre = w->b_pre; a.b_res = w->b_res; a.b_post = w->b_post;
  a.a_pre = w->alpha_pre; a.a_res = w->alpha_res; a.a_post = w->alpha_post;
  a.iters = P.iters; a.eps = P.eps_norm;
  a.h_pre = reinterpret_cast<float*>(ws + P.o_hpre);
  a.h_res = reinterpret_cast<float*>(ws + P.o_hres);
  a.h_post = reinterpret_cast<float*>(ws + P.o_hpost);
  switch (P.N) {
    case 1: launch_mhc_read<E, 1>(a, st); return true;
    case 2: launch_mhc_read<E, 2>(a, st); return true;
    case 4: launch_mhc_read<E, 4>(a, st); return true;
    case 8: launch_mhc_read<E, 8>(a, st); return true;
    case 16: launch_mhc_read<E, 16>(a, st); return true;
    default: return false;
  }
}

template <class E>
static bool mhc_post_launch(const Plan& P, void* X, const void* out, char* ws, hipStream_t st) {
  MhcPostArgs a;
  a.X = X; a.out = out; a.T = (int)P.T; a.C = P.C; a.nslices = P.nslices;
  a.h_res = reinterpret_cast<const float*>(ws + P.o_hres);
  a.h_post = reinterpret_cast<const float*>(ws + P.o_hpost);
  switch (P.N) {
    case 1: launch_mhc_post<E, 1>(a, st); return true;
    case 2: launch_mhc_post<E, 2>(a, st); return true;
    case 4: launch_mhc_post<E, 4>(a, st); return true;
    case 8: launch_mhc_post<E, 8>(a, st); return true;
    case 16: launch_mhc_post<E, 16>(a, st); return true;
    default: return false;
  }
}

bool launch_xhc_post(const Plan& P, void* X, const void* out, const xhc_weights* w, char* ws, hipStream_t st) {
  return P.dtype == XHC_BF16 ? xhc_post_launch<Bf16>(P, X, out, w, ws, st) : xhc_post_launch<F32>(P, X, out, w, ws, st);
}
bool launch_mhc_pre(const Plan& P, const void* X, void* inp, const xhc_weights* w, char* ws, hipStream_t st) {
  return P.dtype == XHC_BF16 ? mhc_pre_launch<Bf16>(P, X, inp, w, ws, st) : mhc_pre_launch<F32>(P, X, inp, w, ws, st);
}
bool launch_mhc_post(const Plan& P, void* X, const void* out, char* ws, hipStream_t st) {
  return P.dtype == XHC_BF16 ? mhc_post_launch<Bf16>(P, X, out, ws, st) : mhc_post_launch<F32>(P, X, out, ws, st);
}

}  // namespace xhc
