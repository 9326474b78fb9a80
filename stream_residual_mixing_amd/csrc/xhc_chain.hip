// xHC sublayers in a chain, with each layer's routing prepared ahead (gfx950).
//
// A sublayer's mapping generation contracts the whole flattened state of a
// token (xHC paper "xHC: Expanded Hyper-Connections", paragraph "Mapping
// generation"), and the dense read of that same state needs its result
// (paragraph "Mapping application").  Done inside one sublayer, that costs
// either a second read of the state or a wait across workgroups while the
// state is held on chip.  In a chain of sublayers the contraction can be done
// earlier and exactly, because it is linear in the state and the state only
// changes in the k rows a sublayer writes (explainer "xHC: sixteen residual
// streams, four written at a time", section "What xHC changes"):
//
//   vec X_{l+1} . W = sum over the rows i not in I_l of x_i . W_i
//                   + sum over the rows i in I_l of x'_i . W_i,
//
// and likewise the sums of x and x^2 behind LayerNorm and RMSNorm.  So
//
//   xhc_pre_chained (layer l)  reads X_l once: dense read with the routing
//       already in the workspace, gather + partial active projection of
//       layer l, and the partial routing projection of layer l+1 over the
//       rows that layer l leaves untouched (its own rows masked to zero);
//   act_fin                    sums the active partials: Sinkhorn + row clamp
//       and H_post of layer l;
//   (the sublayer F, then the usual post kernels of layer l)
//   corr                       reads the k rewritten rows and adds their
//       routing projection for layer l+1;
//   route_fin                  sums both partials: router logits, H_pre, the
//       active list and router weights of layer l+1.
//
// The first layer of a chain gets its routing from one projection pass over
// its state (xhc_route).  No workgroup ever waits for another: partial
// results cross launch boundaries only, and every sum runs in a fixed order.
#include <type_traits>

#include "xhc_internal.hpp"
#include "xhc_tile.hpp"

namespace xhc {

namespace {

constexpr int NTHR = TNTHR;
#ifndef XHC_PRE_WD
#define XHC_PRE_WD 2
#endif
constexpr int WDP = XHC_PRE_WD;   // weight items in flight ahead of the MFMAs (last-sublayer pre kernel)
#ifndef XHC_CORR_WD
#define XHC_CORR_WD 4
#endif
constexpr int WDC = XHC_CORR_WD;  // and for the correction kernel (measured best of 2, 4, 8, 16)
#ifndef XHC_STATE_AUX
#define XHC_STATE_AUX 0
#endif
constexpr int STATE_AUX = XHC_STATE_AUX;   // cache policy of the persistent kernels' state loads (streaming: ~20% slower)
#ifndef XHC_PRE_ONE_PHASE
#define XHC_PRE_ONE_PHASE 1
#endif
#ifndef XHC_ROW_ST_AUX
#define XHC_ROW_ST_AUX 0
#endif
#ifndef XHC_INP_ST_AUX
#define XHC_INP_ST_AUX 2
#endif
constexpr int ROW_ST_AUX = XHC_ROW_ST_AUX;   // cache policy of the rewritten rows' stores (default: measured ~4% faster per post call than streaming, and the next pre pass reads them)
constexpr int INP_ST_AUX = XHC_INP_ST_AUX;   // and of the sublayer input's (streaming: measured ~1% faster)

template <int N>
struct RouteDims {
  static constexpr int NTF = (2 * N + 15) / 16;  // 16-column MFMA tiles of [W_r | W_pre]
  static constexpr int NPF = NTF * 16;
  static constexpr int NSUM = TM * NPF + 2 * TM;  // projection + (sum x, sum x^2) per token
  static constexpr int P1 = NSUM + 16;            // + column sums of W_r
  static constexpr int FT = (P1 / 2 + WAVE - 1) / WAVE * WAVE;   // routing finalize: a pair of entries per thread
};

template <int K, int KR>
struct ActDims {
  static constexpr int NA = K * K + K * KR;
  static constexpr int NTA = (NA + 15) / 16;
  static constexpr int NPA = NTA * 16;
  static constexpr int P2 = TM * NPA + TM;  // projection + sum of squares per token
  static constexpr int FT = (P2 / 2 + WAVE - 1) / WAVE * WAVE;   // active finalize: a pair of entries per thread
};

// Running sum of x and of x^2 over one fragment, in float.  (The packed bf16
// dot product would do this in half the instructions, but in back-to-back
// accumulation chains like these it returned wrong sums on gfx950, so it is
// not used.)
template <class E>
__device__ __forceinline__ void add_stats(const u32x4_t& v, float& s1, float& s2) {
  float f[E::VEC];
  E::unpack(v, f);
#pragma unroll
  for (int e = 0; e < E::VEC; ++e) {
    s1 += f[e];
    s2 = fmaf(f[e], f[e], s2);
  }
}

// Per-token sums on the matrix cores.  With the A fragment of a 16-token
// block in the same registers as a B operand, the MFMA computes A A^T, whose
// diagonal holds each token's sum of squares over the block's contraction
// range; with an all-ones B it computes every token's plain sum in each
// column.  Lane (16 g + r) holds rows 4 g .. 4 g + 3 of the result, column r.
template <class E>
__device__ __forceinline__ void mma_sums(const u32x4_t& a, const u32x4_t& ones, f32x4_t& S1, f32x4_t& S2) {
  S1 = E::mma(S1, a, ones);
  S2 = E::mma(S2, a, a);
}
// Token r's entry of the diagonal (held by the lanes with r / 4 == g).
__device__ __forceinline__ float diag_of(const f32x4_t& S, int r) {
  const int i = r & 3;
  return i == 0 ? S[0] : i == 1 ? S[1] : i == 2 ? S[2] : S[3];
}
// Write (sum x, sum x^2) of the block's 16 tokens to dst[2 tau], dst[2 tau + 1].
__device__ __forceinline__ void sums_to_lds(float* dst, int g, int r, const f32x4_t& S1, const f32x4_t& S2) {
  if (r == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[2 * (4 * g + i)] = S1[i];
  }
  if ((r >> 2) == g) dst[2 * r + 1] = diag_of(S2, r);
}

// Column-0..15 accumulators of one wave to LDS rows of a partial: element
// (token 4 g + i, column n 16 + r) of the MFMA result.
template <int NT, int NP, int PM>
__device__ __forceinline__ void acc_to_lds(float (&dst)[TWV][PM], int wave, int g, int r, const f32x4_t (&acc)[NT]) {
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[wave][(4 * g + i) * NP + n * 16 + r] = acc[n][i];
}

}  // namespace

// ---------------------------------------------------------------------------
// Routing of a tile from the summed partials: the G routing partials of the
// state (or of its untouched rows), plus, when given, the G partials of the
// rewritten rows; router logits, H_pre, active list and router weights.
// ---------------------------------------------------------------------------
struct RouteFinArgs {
  int T, C, m, G, Gc;   // slices of part and of corr
  const float* part;
  const float* corr;   // may be null
  const float* b_pre;
  float a_pre, eps;
  int* idx;
  float *p, *h_pre, *z;
  float* gstat;   // per token: the raw pre-map logits [N], then sum x, sum x^2 (for a backward)
};

template <int N, int K>
__global__ __launch_bounds__(RouteDims<N>::FT) void xhc_route_fin_kernel(RouteFinArgs a) {
  using D = RouteDims<N>;
  constexpr int NPF = D::NPF, NSUM = D::NSUM, P1 = D::P1, FT = D::FT;
  __shared__ float s_sum[P1];
  __shared__ float s_z[TM][N];
  __shared__ float s_hpre[TM][N];
  const int tid = threadIdx.x, G = a.G, Gc = a.Gc;
  const int tile = blockIdx.x, t0 = tile * TM;

  // entries u, u + 1 of the tile's partial: the G routing slices, then the
  // Gc correction slices (projection and sums only), added in that order.
  // With up to 32 of each, all loads go out at once.
  const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.part + (size_t)tile * G * P1, (uint32_t)((size_t)G * P1 * 4));
  const __amdgpu_buffer_rsrc_t rc =
      make_rsrc(a.corr ? a.corr + (size_t)tile * Gc * P1 : a.part, a.corr ? (uint32_t)((size_t)Gc * P1 * 4) : 0u);
  {
    const int u = 2 * tid;
    const uint32_t off = u < P1 ? (uint32_t)(u * 4) : OUT_OF_RANGE;
    const uint32_t offc = u < NSUM ? (uint32_t)(u * 4) : OUT_OF_RANGE;
    float v[2] = {0.f, 0.f};
    if (G <= 32 && Gc <= 32) {
      uint64_t x[32], y[32];
#pragma unroll
      for (int q = 0; q < 32; ++q) x[q] = ld_b64<XHC_FIN_AUX>(rp, off + (uint32_t)(q * P1 * 4));
#pragma unroll
      for (int q = 0; q < 32; ++q) y[q] = ld_b64<XHC_FIN_AUX>(rc, offc + (uint32_t)(q * P1 * 4));
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        v[0] += __uint_as_float((uint32_t)x[q]);
        v[1] += __uint_as_float((uint32_t)(x[q] >> 32));
      }
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        v[0] += __uint_as_float((uint32_t)y[q]);
        v[1] += __uint_as_float((uint32_t)(y[q] >> 32));
      }
    } else {
      add_slices2<32>(rp, G, P1, off, v);
      add_slices2<32>(rc, Gc, P1, offc, v);
    }
    if (u < P1) {
      s_sum[u] = v[0];
      s_sum[u + 1] = v[1];
    }
  }
  __syncthreads();
  const float n_el = (float)N * (float)a.C;
  for (int u = tid; u < TM * N; u += FT) {
    const int tau = u / N, i = u % N;
    route_logits(s_sum[tau * NPF + i], s_sum[tau * NPF + N + i], s_sum[TM * NPF + 2 * tau],
                 s_sum[TM * NPF + 2 * tau + 1], s_sum[NSUM + i], n_el, a.eps, a.a_pre, a.b_pre[i], t0 + tau < a.T,
                 &s_z[tau][i], &s_hpre[tau][i]);
  }
  __syncthreads();
  for (int u = tid; u < TM * N; u += FT) {
    const int tau = u / N, i = u % N, t = t0 + tau;
    if (t < a.T) {
      a.z[(size_t)t * N + i] = s_z[tau][i];
      a.h_pre[(size_t)t * N + i] = s_hpre[tau][i];
      float* gs = a.gstat + (size_t)t * (N + 2);
      gs[i] = s_sum[tau * NPF + N + i];
      if (i == 0) {
        gs[N] = s_sum[TM * NPF + 2 * tau];
        gs[N + 1] = s_sum[TM * NPF + 2 * tau + 1];
      }
    }
  }
  if (tid < TM && t0 + tid < a.T) {
    const int t = t0 + tid;
    float zt[N];
#pragma unroll
    for (int i = 0; i < N; ++i) zt[i] = s_z[tid][i];
    int sel[K];
    route_select<N, K>(zt, a.m, sel);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      a.idx[(size_t)t * K + j] = sel[j];
      a.p[(size_t)t * K + j] = j < a.m ? 1.f : sigmoidf_(zt[sel[j]]);
    }
  }
}

// ---------------------------------------------------------------------------
// Pre-application of a layer whose routing is in the workspace: dense read,
// gather + partial active projection, and (LOOK) the next layer's partial
// routing projection over the rows this layer does not write.
// ---------------------------------------------------------------------------
struct PreChainArgs {
  const void* X;
  void* inp;
  int T, C, G, m, ntiles;
  const uint4* wact;   // this layer's packed [W_res | W_post]
  const uint4* wnext;  // next layer's packed [W_r | W_pre] (LOOK)
  const int* idx;
  const float* h_pre;
  float* part2;        // active partials [ntiles][G][P2]
  float* look;         // next layer's routing partials [ntiles][G][P1] (LOOK)
};

// RB row blocks of 16 tokens per workgroup share every weight fragment
// fetched.  RB = 2 halves the weight traffic, but the workgroup then holds
// 128 VGPRs of state per lane and runs one per CU; measured no faster than
// RB = 1, which is the default.  Partials are written per 16-token tile.
template <class E, int N, int K, int KR, bool LOOK, int RB>
__global__ __launch_bounds__(NTHR, RB == 1 ? 4 : 2) void xhc_pre_chained_kernel(PreChainArgs a) {
  using T = typename E::T;
  using D = RouteDims<N>;
  using A = ActDims<K, KR>;
  constexpr int NTF = D::NTF, NPF = D::NPF, P1 = D::P1;
  constexpr int NTA = A::NTA, NPA = A::NPA, P2 = A::P2;
  constexpr int KB = E::KB, VEC = E::VEC;
  constexpr int TT = TM * RB;   // tokens per workgroup
  // Weight items in order of use: N streams of the next layer's routing
  // weights (LOOK), then the K positions of this layer's active weights.
  constexpr int NL = LOOK ? N : 0;
  constexpr int NI = NL + K;
  constexpr int NTR = NTF > NTA ? NTF : NTA;
  __shared__ float s_red2[TWV][P2];
  __shared__ float s_red1[LOOK ? TWV : 1][LOOK ? P1 : 2];
  __shared__ float s_hpre[TT][N];
  __shared__ int s_idx[TT][K];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r = lane & 15;
  const int C = a.C, G = a.G, nkbC = C / KB;
  const int tile = blockIdx.x / G, slice = blockIdx.x % G;
  const int t0 = tile * TT;
  const int rows = a.T - t0 < TT ? a.T - t0 : TT;
  const int kb0 = slice * TWV + wave;
  const bool kvalid = kb0 < nkbC;

  // routing of the tokens (written by an earlier launch)
  for (int u = tid; u < TT * N; u += NTHR) {
    const int tau = u / N;
    s_hpre[tau][u % N] = tau < rows ? a.h_pre[(size_t)t0 * N + u] : 0.f;
  }
  for (int u = tid; u < TT * K; u += NTHR) {
    const int tau = u / K, j = u % K;
    const int v = tau < rows ? a.idx[(size_t)t0 * K + u] : j;
    s_idx[tau][j] = v < 0 ? 0 : (v >= N ? N - 1 : v);
  }

  const __amdgpu_buffer_rsrc_t rwf =
      make_rsrc(LOOK ? (const void*)a.wnext : (const void*)a.wact, LOOK ? (uint32_t)((size_t)N * nkbC * NTF * WAVE * 16) : 0u);
  const uint32_t vwf = kvalid ? (uint32_t)(((size_t)kb0 * NTF * WAVE + lane) * 16) : OUT_OF_RANGE;
  const uint32_t wf_stream = (uint32_t)nkbC * NTF * WAVE * 16;
  const __amdgpu_buffer_rsrc_t rwa = make_rsrc(a.wact, (uint32_t)((size_t)K * nkbC * NTA * WAVE * 16));
  const uint32_t vwa = kvalid ? (uint32_t)(((size_t)kb0 * NTA * WAVE + lane) * 16) : OUT_OF_RANGE;
  const uint32_t wa_pos = (uint32_t)nkbC * NTA * WAVE * 16;
  u32x4_t wb[WDP][NTR];
  auto fetch = [&](int q) {
    if (q < NL) {
#pragma unroll
      for (int n = 0; n < NTF; ++n) wb[q % WDP][n] = ld_b128(rwf, vwf + n * WAVE * 16, q * wf_stream);
    } else {
#pragma unroll
      for (int n = 0; n < NTA; ++n) wb[q % WDP][n] = ld_b128(rwa, vwa + n * WAVE * 16, (q - NL) * wa_pos);
    }
  };
#pragma unroll
  for (int q = 0; q < WDP && q < NI; ++q) fetch(q);
  __builtin_amdgcn_sched_barrier(0);

  const __amdgpu_buffer_rsrc_t rx =
      make_rsrc(reinterpret_cast<const T*>(a.X) + (size_t)t0 * N * C, (uint32_t)((size_t)rows * N * C * sizeof(T)));
  u32x4_t xd[RB][N];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const uint32_t vx =
        kvalid ? (uint32_t)(((size_t)(TM * b + r) * N * C + (size_t)kb0 * KB + VEC * g) * sizeof(T)) : OUT_OF_RANGE;
#pragma unroll
    for (int i = 0; i < N; ++i) xd[b][i] = ld_b128(rx, vx, (uint32_t)(i * C * (int)sizeof(T)));
  }
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  int I[RB][K];
  uint32_t amask[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    amask[b] = 0;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      I[b][j] = s_idx[TM * b + r][j];
      amask[b] |= 1u << I[b][j];
    }
  }

  // dense read over all N streams -> sublayer input
  if (kvalid) {
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      float o[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[e] = 0.f;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const float hpi = s_hpre[TM * b + r][i];
        float f[VEC];
        E::unpack(xd[b][i], f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = fmaf(hpi, f[e], o[e]);
      }
      if (TM * b + r < rows)
        st16_nt(reinterpret_cast<T*>(a.inp) + (size_t)(t0 + TM * b + r) * C + kb0 * KB + VEC * g, E::packv(o));
    }
  }

  const u32x4_t zero = u32x4_t{0u, 0u, 0u, 0u};
  const u32x4_t ones = ones_frag<E>();
  f32x4_t acc[LOOK ? RB : 1][NTF];
  f32x4_t S1[LOOK ? RB : 1], S2[LOOK ? RB : 1];
  f32x4_t acs = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (LOOK) {
    // next layer's routing projection over the rows this layer leaves as they are
#pragma unroll
    for (int b = 0; b < RB; ++b) {
#pragma unroll
      for (int n = 0; n < NTF; ++n) acc[b][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      S1[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      S2[b] = S1[b];
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const u32x4_t v = ((amask[b] >> i) & 1u) ? zero : xd[b][i];
        mma_sums<E>(v, ones, S1[b], S2[b]);
#pragma unroll
        for (int n = 0; n < NTF; ++n) acc[b][n] = E::mma(acc[b][n], v, wb[i % WDP][n]);
      }
      acs = E::mma(acs, ones, wb[i % WDP][0]);
      if (i + WDP < NI) fetch(i + WDP);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (RB == 1) {   // to LDS now, so the accumulators are free for the gather
      acc_to_lds<NTF, NPF>(s_red1, wave, g, r, acc[0]);
      sums_to_lds(&s_red1[wave][TM * NPF], g, r, S1[0], S2[0]);
      if (g == 0) s_red1[wave][TM * NPF + 2 * TM + r] = acs[0];
    }
  }

  // gather of the k active rows, their sum of squares and active projection
  f32x4_t acc2[RB][NTA];
  f32x4_t SS[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
#pragma unroll
    for (int n = 0; n < NTA; ++n) acc2[b][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    SS[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int j = 0; j < K; ++j) {
    constexpr int Q0 = NL;
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      // position j < m holds stream j; a routed position holds one of m..N-1
      u32x4_t v = xd[b][j < N ? j : 0];
      if (j >= a.m) {
#pragma unroll
        for (int i = 0; i < N; ++i)
          if (i != j) v = (I[b][j] == i) ? xd[b][i] : v;
      }
      SS[b] = E::mma(SS[b], v, v);
#pragma unroll
      for (int n = 0; n < NTA; ++n) acc2[b][n] = E::mma(acc2[b][n], v, wb[(Q0 + j) % WDP][n]);
    }
    if (Q0 + j + WDP < NI) fetch(Q0 + j + WDP);
    __builtin_amdgcn_sched_barrier(0);
  }

  // partials of each 16-token row block, summed over the waves in a fixed order
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int tile16 = (t0 / TM) + b;
    if (b > 0) __syncthreads();   // the previous block's sums have been read
    acc_to_lds<NTA, NPA>(s_red2, wave, g, r, acc2[b]);
    if ((r >> 2) == g) s_red2[wave][TM * NPA + r] = diag_of(SS[b], r);
    if constexpr (LOOK && RB > 1) {
      acc_to_lds<NTF, NPF>(s_red1, wave, g, r, acc[b]);
      sums_to_lds(&s_red1[wave][TM * NPF], g, r, S1[b], S2[b]);
      if (g == 0) s_red1[wave][TM * NPF + 2 * TM + r] = acs[0];
    }
    __syncthreads();
    if (tile16 < a.ntiles) {
      float* d2 = a.part2 + ((size_t)tile16 * G + slice) * P2;
      for (int u = tid; u < P2; u += NTHR) d2[u] = sum_waves(s_red2, u);
      if constexpr (LOOK) {
        float* d1 = a.look + ((size_t)tile16 * G + slice) * P1;
        for (int u = tid; u < P1; u += NTHR) d1[u] = sum_waves(s_red1, u);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Active maps of a tile from the summed active partials: RMSNorm of the
// gathered rows, k x k Sinkhorn + row clamp, and H_post.  One wave per tile.
// ---------------------------------------------------------------------------
struct ActFinArgs {
  int T, C, G, ntiles;
  const float* part2;
  const float *b_res, *b_post;
  float a_res, a_post, eps;
  int iters;
  float *h_res, *h_post;
};

template <int K, int KR>
__global__ __launch_bounds__((ActDims<K, KR>::FT)) void xhc_act_fin_kernel(ActFinArgs a) {
  using A = ActDims<K, KR>;
  constexpr int NPA = A::NPA, P2 = A::P2;
  __shared__ float s_sum[P2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int tile = blockIdx.x;
  const int G = a.G, t0 = tile * TM;
  // entries u, u + 1 summed over the G slices in order, all loads at once
  {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.part2 + (size_t)tile * G * P2, (uint32_t)((size_t)G * P2 * 4));
    const int u = 2 * tid;
    float v[2] = {0.f, 0.f};
    add_slices2<32>(rs, G, P2, u < P2 ? (uint32_t)(u * 4) : OUT_OF_RANGE, v);
    if (u < P2) {
      s_sum[u] = v[0];
      s_sum[u + 1] = v[1];
    }
  }
  __syncthreads();
  if (tid >= WAVE) return;   // one wave finishes the tile
  const float* sm = &s_sum[0];
  constexpr int TPP = WAVE / K;
  constexpr int PASSES = (TM + TPP - 1) / TPP;
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    const int tau = pass * TPP + lane / K;
    const int row = lane % K;
    const int t = t0 + tau;
    const bool valid = tau < TM && t < a.T;
    const int tq = tau < TM ? tau : 0;
    const float rr = 1.f / sqrtf(sm[TM * NPA + tq] / ((float)K * (float)a.C) + a.eps);
    float L[K];
#pragma unroll
    for (int b = 0; b < K; ++b) {
      const int col = row * K + b;
      L[b] = fmaf(a.a_res * sm[tq * NPA + col], rr, a.b_res[col]);
    }
    sinkhorn_rows<K>(L, a.iters);
    float rs = 0.f;
#pragma unroll
    for (int b = 0; b < K; ++b) rs += L[b];
    const float d = fmaxf(rs, 1.f);
#pragma unroll
    for (int b = 0; b < K; ++b) L[b] = L[b] / d;
    if (valid) {
#pragma unroll
      for (int b = 0; b < K; ++b) a.h_res[((size_t)t * K + row) * K + b] = L[b];
#pragma unroll
      for (int q = 0; q < KR; ++q) {
        const int col = K * K + row * KR + q;
        a.h_post[((size_t)t * K + row) * KR + q] =
            2.f * sigmoidf_(fmaf(a.a_post * sm[tq * NPA + col], rr, a.b_post[row * KR + q]));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The rewritten rows' share of the next layer's routing: per RB x 16 tokens
// and channel slice, sum over the k active rows i of x'_i . W_i (the next
// layer's [W_r | W_pre] rows of stream i), sum x' and sum x'^2.  Rows are
// read with the active list of the layer that wrote them; each stream's MFMA
// takes, per token, the active row that sits in that stream (or zero).
// ---------------------------------------------------------------------------
struct CorrArgs {
  const void* X;
  int T, C, G, ntiles, m;
  const int* idx;
  const uint4* wnext;
  float* corr;   // [ntiles][G][P1] (the first NSUM entries of each)
};

// MS: the number of fixed streams when known at compile time (-1: a.m at run time).
template <class E, int N, int K, int RB, int MS>
__global__ __launch_bounds__(NTHR, 2) void xhc_corr_kernel(CorrArgs a) {
  using T = typename E::T;
  using D = RouteDims<N>;
  constexpr int NTF = D::NTF, NPF = D::NPF, NSUM = D::NSUM, P1 = D::P1;
  constexpr int KB = E::KB, VEC = E::VEC;
  constexpr int TB = TM * RB;   // tokens per block
  __shared__ int s_idx[TB][K];
  __shared__ float s_red[TWV][NSUM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r = lane & 15;
  const int C = a.C, G = a.G, nkbC = C / KB;
  const int blk = blockIdx.x / G, slice = blockIdx.x % G;
  const int t0 = blk * TB;
  const int rows = a.T - t0 < TB ? a.T - t0 : TB;
  const int kb0 = slice * TWV + wave;
  const bool kvalid = kb0 < nkbC;

  for (int u = tid; u < TB * K; u += NTHR) {
    const int tau = u / K, j = u % K;
    const int v = tau < rows ? a.idx[(size_t)t0 * K + u] : j;
    s_idx[tau][j] = v < 0 ? 0 : (v >= N ? N - 1 : v);
  }

  const __amdgpu_buffer_rsrc_t rwf = make_rsrc(a.wnext, (uint32_t)((size_t)N * nkbC * NTF * WAVE * 16));
  const uint32_t vwf = kvalid ? (uint32_t)(((size_t)kb0 * NTF * WAVE + lane) * 16) : OUT_OF_RANGE;
  const uint32_t wf_stream = (uint32_t)nkbC * NTF * WAVE * 16;
  u32x4_t wb[WDC][NTF];
#pragma unroll
  for (int d = 0; d < WDC && d < N; ++d)
#pragma unroll
    for (int n = 0; n < NTF; ++n) wb[d][n] = ld_b128(rwf, vwf + n * WAVE * 16, d * wf_stream);
  __syncthreads();

  int I[RB][K];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int j = 0; j < K; ++j) I[b][j] = s_idx[TM * b + r][j];
  const __amdgpu_buffer_rsrc_t rx =
      make_rsrc(reinterpret_cast<const T*>(a.X) + (size_t)t0 * N * C, (uint32_t)((size_t)rows * N * C * sizeof(T)));
  const uint32_t vk = (uint32_t)(((size_t)kb0 * KB + VEC * g) * sizeof(T));
  u32x4_t xa[RB][K];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const uint32_t off = kvalid ? (uint32_t)(((size_t)(TM * b + r) * N + I[b][j]) * C * sizeof(T)) + vk : OUT_OF_RANGE;
      xa[b][j] = ld_b128(rx, off, 0);
    }
  __builtin_amdgcn_sched_barrier(0);

  float s1[RB], s2[RB];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    s1[b] = 0.f;
    s2[b] = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) add_stats<E>(xa[b][j], s1[b], s2[b]);
  }
  f32x4_t acc[RB][NTF];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int n = 0; n < NTF; ++n) acc[b][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const u32x4_t zero = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < N; ++i) {
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      // stream i holds the active position that chose it, if any: with m
      // known, stream i < m holds fixed position i and only routed positions
      // can hold a stream i >= m
      u32x4_t v = zero;
      if constexpr (MS >= 0) {
        if (i < MS) {
          v = xa[b][i < K ? i : 0];
        } else {
#pragma unroll
          for (int j = MS; j < K; ++j) v = (I[b][j] == i) ? xa[b][j] : v;
        }
      } else {
#pragma unroll
        for (int j = 0; j < K; ++j) v = (I[b][j] == i) ? xa[b][j] : v;
      }
#pragma unroll
      for (int n = 0; n < NTF; ++n) acc[b][n] = E::mma(acc[b][n], v, wb[i % WDC][n]);
    }
    if (i + WDC < N) {
#pragma unroll
      for (int n = 0; n < NTF; ++n) wb[i % WDC][n] = ld_b128(rwf, vwf + n * WAVE * 16, (i + WDC) * wf_stream);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    s1[b] += __shfl_xor(s1[b], 16, WAVE);
    s1[b] += __shfl_xor(s1[b], 32, WAVE);
    s2[b] += __shfl_xor(s2[b], 16, WAVE);
    s2[b] += __shfl_xor(s2[b], 32, WAVE);
  }
  const int tile0 = t0 / TM;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    if (b > 0) __syncthreads();   // the previous block's sums have been read
    acc_to_lds<NTF, NPF>(s_red, wave, g, r, acc[b]);
    if (g == 0) {
      s_red[wave][TM * NPF + 2 * r] = s1[b];
      s_red[wave][TM * NPF + 2 * r + 1] = s2[b];
    }
    __syncthreads();
    if (tile0 + b < a.ntiles) {
      float* dst = a.corr + ((size_t)(tile0 + b) * G + slice) * P1;
      for (int u = tid; u < NSUM; u += NTHR) dst[u] = sum_waves(s_red, u);
    }
  }
}

// ---------------------------------------------------------------------------
// Persistent form of the routing projection and of the chained pre pass.
//
// The routing weights [W_r | W_pre] of one channel slice are as large as the
// state a 16-token tile holds in that slice, and the kernels above read them
// from L2 again for every tile, behind the state loads in the same memory
// queue.  Here a workgroup owns one slice of PSB contraction blocks for the
// whole launch, keeps that slice's routing fragments in LDS (read from L2
// once per workgroup) and walks steps of PTL 16-token tiles, one wave per
// (tile of the step, block of the slice).  The state of the next step is
// loaded into a second register set while this step computes.  Partials keep
// the per-tile layout, over Gp = ceil(C / (PSB KB)) slices.
// ---------------------------------------------------------------------------
constexpr int PSB = 4;                    // contraction blocks per slice
constexpr int PTL = 2;                    // 16-token tiles per step
constexpr int PNTHR = PSB * PTL * WAVE;   // 512 threads, 8 waves
static_assert(PSB * PTL == TWV, "one wave per (tile, block)");

template <int N>
struct XTile {
  u32x4_t x[N];
};

// One wave's share of a step: token r of tile b of the step, VEC channels of
// block kb in every stream (lane_off covers b, r and kb, or is OUT_OF_RANGE
// for a block past C).  The buffer resource spans the step's valid rows only
// (rows, from step_rows), so rows past T read zeros without touching memory;
// it depends on the step alone, which keeps it in scalar registers.
template <class E, int N>
__device__ __forceinline__ void load_xtile(XTile<N>& xs, const typename E::T* X, int C, int step, int rows,
                                           uint32_t lane_off) {
  using TT = typename E::T;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(X + (size_t)(rows > 0 ? step : 0) * PTL * TM * N * C,
                                              (uint32_t)((size_t)rows * N * C * sizeof(TT)));
#pragma unroll
  for (int i = 0; i < N; ++i) xs.x[i] = ld_b128<STATE_AUX>(rx, lane_off, (uint32_t)(i * C * (int)sizeof(TT)));
}

// Valid rows of a step (full steps, then the ragged one, then none), written
// with compares and selects only so that it stays a scalar.
__device__ __forceinline__ int step_rows(int step, int full, int tail) {
  return step < full ? PTL * TM : (step == full ? tail : 0);
}

// The slice's packed routing fragments of streams FS .. N-1 -> LDS (zero for
// blocks past C).
template <int N, int NTF, int FS = 0>
__device__ __forceinline__ void load_wslice(u32x4_t (&s_w)[PSB][N - FS][NTF][WAVE], const uint4* wfull, int nkbC,
                                            int slice, int tid) {
  constexpr int NS = N - FS;
  constexpr int TOT = PSB * NS * NTF * WAVE;
  constexpr int IT = (TOT + PNTHR - 1) / PNTHR;
  u32x4_t v[IT];
#pragma unroll
  for (int k = 0; k < IT; ++k) {
    const int u = tid + k * PNTHR;
    const int l = u % WAVE, n = (u / WAVE) % NTF, i = FS + (u / (WAVE * NTF)) % NS, c = u / (WAVE * NTF * NS);
    const int kb = slice * PSB + c;
    v[k] = u32x4_t{0u, 0u, 0u, 0u};
    if (u < TOT && kb < nkbC)
      v[k] = ld16v(wfull + (((size_t)i * nkbC + kb) * NTF + n) * WAVE + l);
  }
#pragma unroll
  for (int k = 0; k < IT; ++k) {
    const int u = tid + k * PNTHR;
    if (u < TOT) (&s_w[0][0][0][0])[u] = v[k];
  }
}

// Column sums of the slice's W_r (every routing partial carries them), summed
// over the blocks in a fixed order.  Uses s_red as scratch; ends synchronized.
template <class E, int N, int NTF, int PM>
__device__ __forceinline__ void slice_colsums(const u32x4_t (&s_w)[PSB][N][NTF][WAVE], float (&s_red)[TWV][PM],
                                              float* s_acs, int tid, int wave, int lane) {
  if (wave < PSB) {
    const u32x4_t ones = ones_frag<E>();
    f32x4_t acs = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < N; ++i) acs = E::mma(acs, ones, s_w[wave][i][0][lane]);
    if (lane < 16) s_red[wave][lane] = acs[0];
  }
  __syncthreads();
  if (tid < 16) {
    float v = 0.f;
#pragma unroll
    for (int c = 0; c < PSB; ++c) v += s_red[c][tid];
    s_acs[tid] = v;
  }
  __syncthreads();
}

// The same column sums from the packed weights in global memory (for a
// kernel that keeps only some streams' fragments in LDS): the same
// fragments in the same order, so the same bits.
template <class E, int N, int NTF, int PM>
__device__ __forceinline__ void slice_colsums_g(const uint4* wfull, int nkbC, int slice, float (&s_red)[TWV][PM],
                                                float* s_acs, int tid, int wave, int lane) {
  if (wave < PSB) {
    const int kb = slice * PSB + wave;
    const u32x4_t ones = ones_frag<E>();
    u32x4_t f[N];
#pragma unroll
    for (int i = 0; i < N; ++i)
      f[i] = kb < nkbC ? ld16v(wfull + (((size_t)i * nkbC + kb) * NTF) * WAVE + lane) : u32x4_t{0u, 0u, 0u, 0u};
    f32x4_t acs = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < N; ++i) acs = E::mma(acs, ones, f[i]);
    if (lane < 16) s_red[wave][lane] = acs[0];
  }
  __syncthreads();
  if (tid < 16) {
    float v = 0.f;
#pragma unroll
    for (int c = 0; c < PSB; ++c) v += s_red[c][tid];
    s_acs[tid] = v;
  }
  __syncthreads();
}

// Next-layer routing projection of one tile (rows in amask masked to zero),
// with the sums of x and x^2, B operands from LDS.  The N x NTF weight
// fragments are read ROUTE_BD - 1 MFMAs ahead of their use (a ring of
// ROUTE_BD registers), each step pinned by a scheduling barrier: left to
// itself the compiler reads each fragment right before its MFMA and waits
// for the LDS every time.  The first S0 streams are known to be masked
// (the fixed streams of the active list) and are skipped.
#ifndef XHC_ROUTE_BD
#define XHC_ROUTE_BD 3
#endif
template <class E, int N, int NTF, int S0 = 0, int BD = XHC_ROUTE_BD, int NWS = N>
__device__ __forceinline__ void route_mma(const XTile<N>& xs, const u32x4_t (&w)[NWS][NTF][WAVE], int lane,
                                          uint32_t amask, f32x4_t (&acc)[NTF], f32x4_t& S1, f32x4_t& S2) {
  static_assert(S0 >= N - NWS, "w holds the fragments of streams N - NWS .. N - 1");
  constexpr int WOFS = N - NWS;   // stream i's fragments sit at w[i - WOFS]
  const u32x4_t zero = u32x4_t{0u, 0u, 0u, 0u};
  const u32x4_t ones = ones_frag<E>();
  constexpr int TOT = N * NTF, Q0 = S0 * NTF;
#pragma unroll
  for (int n = 0; n < NTF; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  S1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
  S2 = S1;
  u32x4_t b[BD];
#pragma unroll
  for (int q = Q0; q < Q0 + BD - 1 && q < TOT; ++q) b[q % BD] = w[q / NTF - WOFS][q % NTF][lane];
#pragma unroll
  for (int i = S0; i < N; ++i) {
    const u32x4_t v = ((amask >> i) & 1u) ? zero : xs.x[i];
    mma_sums<E>(v, ones, S1, S2);
#pragma unroll
    for (int n = 0; n < NTF; ++n) {
      const int q = i * NTF + n;
      if (q + BD - 1 < TOT) b[(q + BD - 1) % BD] = w[(q + BD - 1) / NTF - WOFS][(q + BD - 1) % NTF][lane];
      acc[n] = E::mma(acc[n], v, b[q % BD]);
      if constexpr (BD > 1) __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Routing partials of the step's PTL tiles from the per-wave blocks in s_red
// (written before a barrier): per tile the sum over its PSB blocks in order,
// plus the slice's column sums, stored per (tile, slice).
template <int N, int PM>
__device__ __forceinline__ void route_partials_store(const float (&s_red)[TWV][PM], const float* s_acs, float* dst,
                                                     int G, int slice, int step, int ntiles, int tid) {
  using D = RouteDims<N>;
  constexpr int NSUM = D::NSUM, P1 = D::P1;
  // stores through a resource over the partials: entries past the step or
  // past the last tile go out of its range (no store under a branch)
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(dst, (uint32_t)((size_t)ntiles * G * P1 * 4));
  constexpr int IT = (PTL * P1 + PNTHR - 1) / PNTHR;
#pragma unroll
  for (int k = 0; k < IT; ++k) {
    const int u0 = tid + k * PNTHR;
    const bool in = u0 < PTL * P1;
    const int u = in ? u0 : 0;
    const int bb = u / P1, v = u % P1;
    const int tile = PTL * step + bb;
    float x = 0.f;
#pragma unroll
    for (int c = 0; c < PSB; ++c) x += s_red[bb * PSB + c][v < NSUM ? v : 0];
    if (v >= NSUM) x = s_acs[v - NSUM >= 0 ? v - NSUM : 0];
    st_b32(x, rd, in && tile < ntiles ? (uint32_t)((((size_t)tile * G + slice) * P1 + v) * 4) : OUT_OF_RANGE);
  }
}

// The same with the waves' blocks written to s_red first, between barriers.
template <int N, int PM>
__device__ __forceinline__ void route_partials(float (&s_red)[TWV][PM], const float* s_acs, const f32x4_t (&acc)[RouteDims<N>::NTF],
                                               const f32x4_t& S1, const f32x4_t& S2, float* dst, int G, int slice,
                                               int step, int ntiles, int tid, int wave, int g, int r) {
  using D = RouteDims<N>;
  constexpr int NTF = D::NTF, NPF = D::NPF;
  acc_to_lds<NTF, NPF>(s_red, wave, g, r, acc);
  sums_to_lds(&s_red[wave][TM * NPF], g, r, S1, S2);
  __syncthreads();
  route_partials_store<N>(s_red, s_acs, dst, G, slice, step, ntiles, tid);
  __syncthreads();
}

struct ProjPArgs {
  const void* X;
  int T, C, G, ntiles;
  const uint4* wfull;
  float* part;
};

// Routing projection of a whole state (first layer of a chain).
template <class E, int N>
__global__ __launch_bounds__(PNTHR, 1) void xhc_proj_p_kernel(ProjPArgs a) {
  using T = typename E::T;
  using D = RouteDims<N>;
  constexpr int NTF = D::NTF, NSUM = D::NSUM;
  constexpr int KB = E::KB, VEC = E::VEC;
  __shared__ u32x4_t s_w[PSB][N][NTF][WAVE];
  __shared__ float s_red[TWV][NSUM];
  __shared__ float s_acs[16];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform, so tile resources stay scalar
  const int b = wave / PSB, cb = wave % PSB;
  const int C = a.C, G = a.G, nkbC = C / KB;
  const int slice = blockIdx.x % G, team = blockIdx.x / G, nteams = gridDim.x / G;
  const int nsteps = (a.ntiles + PTL - 1) / PTL;
  const int kb0 = slice * PSB + cb;
  const uint32_t lane_off =
      kb0 < nkbC ? (uint32_t)(((size_t)(TM * b + r) * N * C + (size_t)kb0 * KB + VEC * g) * sizeof(T)) : OUT_OF_RANGE;
  const T* X = reinterpret_cast<const T*>(a.X);
  const int full = a.T / (PTL * TM), tail = a.T % (PTL * TM);

  XTile<N> xa, xb;
  int p = team;
  load_xtile<E, N>(xa, X, C, p, step_rows(p, full, tail), lane_off);
  load_wslice<N, NTF>(s_w, a.wfull, nkbC, slice, tid);
  __syncthreads();
  slice_colsums<E, N, NTF>(s_w, s_red, s_acs, tid, wave, lane);

  f32x4_t acc[NTF], S1, S2;
  while (p < nsteps) {
    // the next step's loads are always issued (past the end they read
    // nothing), so the waits of this step never cover them
    const int p1 = p + nteams;
    load_xtile<E, N>(xb, X, C, p1, step_rows(p1, full, tail), lane_off);
    __builtin_amdgcn_sched_barrier(0);
    route_mma<E, N, NTF>(xa, s_w[cb], lane, 0u, acc, S1, S2);
    route_partials<N>(s_red, s_acs, acc, S1, S2, a.part, G, slice, p, a.ntiles, tid, wave, g, r);
    if (p1 >= nsteps) break;
    const int p2 = p1 + nteams;
    load_xtile<E, N>(xa, X, C, p2, step_rows(p2, full, tail), lane_off);
    __builtin_amdgcn_sched_barrier(0);
    route_mma<E, N, NTF>(xb, s_w[cb], lane, 0u, acc, S1, S2);
    route_partials<N>(s_red, s_acs, acc, S1, S2, a.part, G, slice, p1, a.ntiles, tid, wave, g, r);
    p = p2;
  }
}

// ---------------------------------------------------------------------------
// xHC-Flash routing projection, persistent (N = 16): the packed full-state
// weights have three 16-column tiles per block (router, attention pre-map,
// MLP pre-map).  The first two stay in LDS for the launch as in
// xhc_proj_p_kernel; the third, for the wave's own block, stays in registers.
// Partials per (16-token tile, slice): 48 projection columns, sum x and
// sum x^2 per token, then the slice's router column sums.
// ---------------------------------------------------------------------------
struct FlashDims16 {
  static constexpr int NTF = 3;
  static constexpr int NPF = 48;
  static constexpr int NSUM = TM * NPF + 2 * TM;
  static constexpr int P1 = NSUM + 16;
};

template <class E>
__global__ __launch_bounds__(PNTHR, 1) void xhcf_proj_p_kernel(ProjPArgs a) {
  using T = typename E::T;
  constexpr int N = 16, NTL = 2, NT3 = 3;
  constexpr int NPF = FlashDims16::NPF, NSUM = FlashDims16::NSUM, P1 = FlashDims16::P1;
  constexpr int KB = E::KB, VEC = E::VEC;
  __shared__ u32x4_t s_w[PSB][N][NTL][WAVE];
  __shared__ float s_red[TWV][NSUM];
  __shared__ float s_acs[16];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = wave / PSB, cb = wave % PSB;
  const int C = a.C, G = a.G, nkbC = C / KB;
  const int slice = blockIdx.x % G, team = blockIdx.x / G, nteams = gridDim.x / G;
  const int nsteps = (a.ntiles + PTL - 1) / PTL;
  const int kb0 = slice * PSB + cb;
  const uint32_t lane_off =
      kb0 < nkbC ? (uint32_t)(((size_t)(TM * b + r) * N * C + (size_t)kb0 * KB + VEC * g) * sizeof(T)) : OUT_OF_RANGE;
  const T* X = reinterpret_cast<const T*>(a.X);
  const int full = a.T / (PTL * TM), tail = a.T % (PTL * TM);

  XTile<N> xa, xb;
  int p = team;
  load_xtile<E, N>(xa, X, C, p, step_rows(p, full, tail), lane_off);
  // tiles 0 and 1 of the slice's blocks -> LDS; tile 2 of this wave's block -> registers
  {
    constexpr int TOT = PSB * N * NTL * WAVE;
    constexpr int IT = (TOT + PNTHR - 1) / PNTHR;
    u32x4_t v[IT];
#pragma unroll
    for (int q = 0; q < IT; ++q) {
      const int u = tid + q * PNTHR;
      const int l = u % WAVE, n = (u / WAVE) % NTL, i = (u / (WAVE * NTL)) % N, c = u / (WAVE * NTL * N);
      const int kb = slice * PSB + c;
      v[q] = u32x4_t{0u, 0u, 0u, 0u};
      if (u < TOT && kb < nkbC) v[q] = ld16v(a.wfull + (((size_t)i * nkbC + kb) * NT3 + n) * WAVE + l);
    }
#pragma unroll
    for (int q = 0; q < IT; ++q) {
      const int u = tid + q * PNTHR;
      if (u < TOT) (&s_w[0][0][0][0])[u] = v[q];
    }
  }
  u32x4_t wm[N];
#pragma unroll
  for (int i = 0; i < N; ++i)
    wm[i] = kb0 < nkbC ? ld16v(a.wfull + (((size_t)i * nkbC + kb0) * NT3 + 2) * WAVE + lane) : u32x4_t{0u, 0u, 0u, 0u};
  __syncthreads();
  slice_colsums<E, N, NTL>(s_w, s_red, s_acs, tid, wave, lane);

  auto step_partials = [&](const XTile<N>& xs, int step) {
    f32x4_t acc[NTL], acc3 = f32x4_t{0.f, 0.f, 0.f, 0.f}, S1, S2;
    route_mma<E, N, NTL>(xs, s_w[cb], lane, 0u, acc, S1, S2);
#pragma unroll
    for (int i = 0; i < N; ++i) acc3 = E::mma(acc3, xs.x[i], wm[i]);
    const f32x4_t all[NT3] = {acc[0], acc[1], acc3};
    acc_to_lds<NT3, NPF>(s_red, wave, g, r, all);
    sums_to_lds(&s_red[wave][TM * NPF], g, r, S1, S2);
    __syncthreads();
    constexpr int IT = (PTL * P1 + PNTHR - 1) / PNTHR;
#pragma unroll
    for (int q = 0; q < IT; ++q) {
      const int u = tid + q * PNTHR;
      if (u < PTL * P1) {
        const int bb = u / P1, v = u % P1;
        const int tile = PTL * step + bb;
        float x;
        if (v < NSUM) {
          x = 0.f;
#pragma unroll
          for (int c = 0; c < PSB; ++c) x += s_red[bb * PSB + c][v];
        } else {
          x = s_acs[v - NSUM];
        }
        if (tile < a.ntiles) a.part[((size_t)tile * G + slice) * P1 + v] = x;
      }
    }
    __syncthreads();
  };

  while (p < nsteps) {
    const int p1 = p + nteams;
    load_xtile<E, N>(xb, X, C, p1, step_rows(p1, full, tail), lane_off);
    __builtin_amdgcn_sched_barrier(0);
    step_partials(xa, p);
    if (p1 >= nsteps) break;
    const int p2 = p1 + nteams;
    load_xtile<E, N>(xa, X, C, p2, step_rows(p2, full, tail), lane_off);
    __builtin_amdgcn_sched_barrier(0);
    step_partials(xb, p1);
    p = p2;
  }
}

// The xHC-Flash-4sub projection: router and four pre-maps per block.
struct Flash4Dims16 {
  static constexpr int NTF = 5;
  static constexpr int NPF = 80;
  static constexpr int NSUM = TM * NPF + 2 * TM;
  static constexpr int P1 = NSUM + 16;
};
static_assert(Flash4Dims16::P1 == (int)FLASH4_P1, "the workspace sizes the 4sub partials with FLASH4_P1");

struct FlashRouteFinArgs {
  int T, C, m, G;
  const float* part;
  const float *b_pa, *b_pm;
  float a_pa, a_pm, eps;
  int* idx;
  float *p, *h_pa, *h_pm, *z;
};

// Routing of a tile from the summed persistent partials (N = 16): router
// logits, both pre-maps, the active list and router weights.
template <int K>
__global__ __launch_bounds__(256) void xhcf_route_fin_kernel(FlashRouteFinArgs a) {
  constexpr int N = 16, NPF = FlashDims16::NPF, NSUM = FlashDims16::NSUM, P1 = FlashDims16::P1;
  __shared__ float s_sum[P1];
  __shared__ float s_z[TM][N];
  const int tid = threadIdx.x, G = a.G;
  const int tile = blockIdx.x, t0 = tile * TM;
  sum_slices<256, XHC_FIN_AUX>(a.part + (size_t)tile * G * P1, G, P1, P1, s_sum, tid);
  __syncthreads();
  const float n_el = (float)N * (float)a.C;
  for (int u = tid; u < TM * N; u += 256) {
    const int tau = u / N, i = u % N, t = t0 + tau;
    const bool valid = t < a.T;
    float z, hpa, hpm, zz;
    const float q1 = s_sum[TM * NPF + 2 * tau], q2 = s_sum[TM * NPF + 2 * tau + 1], cs = s_sum[NSUM + i];
    route_logits(s_sum[tau * NPF + i], s_sum[tau * NPF + N + i], q1, q2, cs, n_el, a.eps, a.a_pa, a.b_pa[i], valid,
                 &z, &hpa);
    route_logits(s_sum[tau * NPF + i], s_sum[tau * NPF + 2 * N + i], q1, q2, cs, n_el, a.eps, a.a_pm, a.b_pm[i],
                 valid, &zz, &hpm);
    s_z[tau][i] = z;
    if (valid) {
      a.z[(size_t)t * N + i] = z;
      a.h_pa[(size_t)t * N + i] = hpa;
      a.h_pm[(size_t)t * N + i] = hpm;
    }
  }
  __syncthreads();
  if (tid < TM && t0 + tid < a.T) {
    const int t = t0 + tid;
    float zt[N];
#pragma unroll
    for (int i = 0; i < N; ++i) zt[i] = s_z[tid][i];
    int sel[K];
    route_select<N, K>(zt, a.m, sel);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      a.idx[(size_t)t * K + j] = sel[j];
      a.p[(size_t)t * K + j] = j < a.m ? 1.f : sigmoidf_(zt[sel[j]]);
    }
  }
}

// Routing of a tile from the summed persistent partials of the xHC-Flash-4sub
// projection (N = 16): router logits, the four pre-maps, the active list and
// router weights (per token the arithmetic of the split-K path's routing
// kernel, from partials summed over the slices in order).
struct Flash4RouteFinArgs {
  int T, C, m, G;
  const float* part;
  float eps;
  Flash4Route o;
};
template <int K>
__global__ __launch_bounds__(256) void xhcf4_route_fin_kernel(Flash4RouteFinArgs a) {
  constexpr int N = 16, NPF = Flash4Dims16::NPF, NSUM = Flash4Dims16::NSUM, P1 = Flash4Dims16::P1;
  __shared__ float s_sum[P1];
  __shared__ float s_z[TM][N];
  const int tid = threadIdx.x, G = a.G;
  const int tile = blockIdx.x, t0 = tile * TM;
  sum_slices<256, XHC_FIN_AUX>(a.part + (size_t)tile * G * P1, G, P1, P1, s_sum, tid);
  __syncthreads();
  const float n_el = (float)N * (float)a.C;
  for (int u = tid; u < TM * N; u += 256) {
    const int tau = u / N, i = u % N, t = t0 + tau;
    const bool valid = t < a.T;
    const float q1 = s_sum[TM * NPF + 2 * tau], q2 = s_sum[TM * NPF + 2 * tau + 1], cs = s_sum[NSUM + i];
    float z = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float hp, zz;
      route_logits(s_sum[tau * NPF + i], s_sum[tau * NPF + (1 + q) * N + i], q1, q2, cs, n_el, a.eps, a.o.a_pre[q],
                   a.o.b_pre[q][i], valid, &zz, &hp);
      if (q == 0) z = zz;
      if (valid) a.o.h_pre[q][(size_t)t * N + i] = hp;
    }
    s_z[tau][i] = z;
    if (valid) a.o.z[(size_t)t * N + i] = z;
  }
  __syncthreads();
  if (tid < TM && t0 + tid < a.T) {
    const int t = t0 + tid;
    float zt[N];
#pragma unroll
    for (int i = 0; i < N; ++i) zt[i] = s_z[tid][i];
    int sel[K];
    route_select<N, K>(zt, a.m, sel);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      a.o.idx[(size_t)t * K + j] = sel[j];
      a.o.p[(size_t)t * K + j] = j < a.m ? 1.f : sigmoidf_(zt[sel[j]]);
    }
  }
}

// Chained pre pass of a layer that has a next layer (dense read, gather +
// active partials of this layer, masked routing partials of the next one).
// The routing of the next step (h_pre rows, then active lists) is loaded by
// the first RQ threads along with the state and moved to LDS after compute.
// MS: the number of fixed streams when known at compile time (-1: a.m at run
// time); fixed position j then reads stream j directly, a routed one selects
// among streams MS .. N-1 only, and the fixed streams (always in the active
// list) drop out of the next layer's routing partials without any MFMA.
template <class E, int N, int K, int KR, int MS>
__global__ __launch_bounds__(PNTHR, 1) void xhc_pre_chained_p_kernel(PreChainArgs a) {
  using T = typename E::T;
  using D = RouteDims<N>;
  using A = ActDims<K, KR>;
  constexpr int NTF = D::NTF, NSUM = D::NSUM;
  constexpr int NTA = A::NTA, NPA = A::NPA, P2 = A::P2;
  constexpr int KB = E::KB, VEC = E::VEC;
  constexpr int PM = NSUM > P2 ? NSUM : P2;
  // routing rows of a step in 16-byte units: h_pre rows (whole waves WH)
  // then active lists (waves WI), each wave loading 64 units
  constexpr int HQ = PTL * TM * N / 4, IQ = PTL * TM * K / 4;
  constexpr int WH = (HQ + WAVE - 1) / WAVE, WI = (IQ + WAVE - 1) / WAVE;
  static_assert((PTL * TM * N) % 4 == 0 && (PTL * TM * K) % 4 == 0 && WH + WI <= TWV, "routing rows of a step");
  // With m known the fixed streams 0 .. MS-1 are always in the active list,
  // so the next layer's routing never reads their fragments: LDS keeps
  // streams FS .. N-1 only, and the room this frees holds the active
  // partials apart from the routing ones, so that both go through one
  // barrier phase per step instead of two.
  constexpr int FS = MS > 0 && MS < N ? MS : 0;
  constexpr bool ONE_PHASE =
      XHC_PRE_ONE_PHASE && FS > 0 && (size_t)PSB * (N - FS) * NTF * WAVE * 16 + (size_t)TWV * (PM + P2) * 4 + 16 * 4 +
                        (size_t)2 * (WH + WI) * WAVE * 16 <= 160 * 1024;
  __shared__ u32x4_t s_w[PSB][N - FS][NTF][WAVE];
  __shared__ float s_red[TWV][PM];
  __shared__ float s_red2[ONE_PHASE ? TWV : 1][ONE_PHASE ? P2 : 1];
  __shared__ float s_acs[16];
  __shared__ u32x4_t s_rh[2][WH * WAVE];
  __shared__ u32x4_t s_ri[2][WI * WAVE];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform, so tile resources stay scalar
  const int b = wave / PSB, cb = wave % PSB;
  const int C = a.C, G = a.G, nkbC = C / KB;
  const int slice = blockIdx.x % G, team = blockIdx.x / G, nteams = gridDim.x / G;
  const int nsteps = (a.ntiles + PTL - 1) / PTL;
  const int kb0 = slice * PSB + cb;
  const bool kvalid = kb0 < nkbC;
  const uint32_t lane_off =
      kvalid ? (uint32_t)(((size_t)(TM * b + r) * N * C + (size_t)kb0 * KB + VEC * g) * sizeof(T)) : OUT_OF_RANGE;
  const T* X = reinterpret_cast<const T*>(a.X);
  const __amdgpu_buffer_rsrc_t rp2 = make_rsrc(a.part2, (uint32_t)((size_t)a.ntiles * G * P2 * 4));
  const int full = a.T / (PTL * TM), tail = a.T % (PTL * TM);

  // The step's routing rows; which array a wave loads is wave-uniform, so no
  // lane waits for its data before the state prefetch is issued.  Units past
  // the valid rows read zeros.
  // every wave issues the load (a wave without a share reads an empty
  // range), so that no memory operation sits under a branch
  auto load_route = [&](int step) {
    const int valid = step_rows(step, full, tail);
    const int ts = valid > 0 ? PTL * TM * step : 0;
    const void* base = a.h_pre;
    uint32_t bytes = 0, unit = (uint32_t)((wave * WAVE + lane) * 16);
    if (wave < WH) {
      base = a.h_pre + (size_t)ts * N;
      bytes = (uint32_t)(valid * N * 4);
    } else if (wave < WH + WI) {
      base = a.idx + (size_t)ts * K;
      bytes = (uint32_t)(valid * K * 4);
      unit = (uint32_t)(((wave - WH) * WAVE + lane) * 16);
    }
    return ld_b128(make_rsrc(base, bytes), unit, 0);
  };
  auto store_route = [&](int buf, const u32x4_t& v) {
    if (wave < WH)
      s_rh[buf][wave * WAVE + lane] = v;
    else if (wave < WH + WI)
      s_ri[buf][(wave - WH) * WAVE + lane] = v;
  };

  // this layer's active weights of the wave's block, loaded once and held in
  // registers for the whole launch
  const __amdgpu_buffer_rsrc_t rwa = make_rsrc(a.wact, (uint32_t)((size_t)K * nkbC * NTA * WAVE * 16));
  const uint32_t vwa = kvalid ? (uint32_t)(((size_t)kb0 * NTA * WAVE + lane) * 16) : OUT_OF_RANGE;
  u32x4_t wa[K][NTA];
  auto load_wact = [&]() {
#pragma unroll
    for (int j = 0; j < K; ++j)
#pragma unroll
      for (int n = 0; n < NTA; ++n)
        wa[j][n] = ld_b128(rwa, vwa + n * WAVE * 16, (uint32_t)j * nkbC * NTA * WAVE * 16);
  };
  XTile<N> xa, xb;
  int p = team;
  load_wact();
  u32x4_t rt = load_route(p);
  load_xtile<E, N>(xa, X, C, p, step_rows(p, full, tail), lane_off);
  load_wslice<N, NTF, FS>(s_w, a.wnext, nkbC, slice, tid);
  store_route(0, rt);
  __syncthreads();
  if constexpr (FS > 0)
    slice_colsums_g<E, N, NTF>(a.wnext, nkbC, slice, s_red, s_acs, tid, wave, lane);
  else
    slice_colsums<E, N, NTF>(s_w, s_red, s_acs, tid, wave, lane);

  auto compute = [&](const XTile<N>& xs, int step, int buf, const u32x4_t& rnext) {
    const int tile = PTL * step + b;
    const int tok = TM * tile + r;
    const uint32_t* rh = reinterpret_cast<const uint32_t*>(&s_rh[buf][0]);
    const uint32_t* ri = reinterpret_cast<const uint32_t*>(&s_ri[buf][0]);
    int I[K];
    uint32_t amask = 0;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      int v = (int)ri[(b * TM + r) * K + j];
      v = v < 0 ? 0 : (v >= N ? N - 1 : v);
      I[j] = v;
      amask |= 1u << v;
    }
    // dense read over all N streams -> sublayer input
    {
      float o[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[e] = 0.f;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const float hpi = __uint_as_float(rh[(b * TM + r) * N + i]);
        float f[VEC];
        E::unpack(xs.x[i], f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = fmaf(hpi, f[e], o[e]);
      }
      // the step's rows of inp; a block past C or a token past T is out of range
      const int rows = kvalid ? step_rows(step, full, tail) : 0;
      const __amdgpu_buffer_rsrc_t ri = make_rsrc(reinterpret_cast<T*>(a.inp) + (size_t)(rows > 0 ? step : 0) * PTL * TM * C,
                                                  (uint32_t)((size_t)rows * C * sizeof(T)));
      st_b128<INP_ST_AUX>(E::packv_cvt(o), ri, (uint32_t)(((size_t)(TM * b + r) * C + kb0 * KB + VEC * g) * sizeof(T)));
      (void)tok;
      (void)tile;
    }
    // with m known at run time only, the longer-lived register would spill:
    // the next step's routing goes to LDS here (see below)
    if constexpr (MS < 0) store_route(buf ^ 1, rnext);
    // gather of the k active rows, their sum of squares and active projection
    f32x4_t acc2[NTA], SS = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < NTA; ++n) acc2[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < K; ++j) {
      // position j < m holds stream j; a routed position holds one of m..N-1
      u32x4_t v;
      if constexpr (MS >= 0) {
        if (j < MS) {
          v = xs.x[j];
        } else {
          v = xs.x[MS < N ? MS : 0];
#pragma unroll
          for (int i = MS + 1; i < N; ++i) v = (I[j] == i) ? xs.x[i] : v;
        }
      } else {
        v = xs.x[j < N ? j : 0];
        if (j >= a.m) {
#pragma unroll
          for (int i = 0; i < N; ++i)
            if (i != j) v = (I[j] == i) ? xs.x[i] : v;
        }
      }
      SS = E::mma(SS, v, v);
#pragma unroll
      for (int n = 0; n < NTA; ++n) acc2[n] = E::mma(acc2[n], v, wa[j][n]);
    }
    // next layer's routing over the rows this layer leaves as they are
    f32x4_t acc[NTF], S1, S2;
    route_mma<E, N, NTF, FS, XHC_ROUTE_BD, N - FS>(xs, s_w[cb], lane, amask, acc, S1, S2);
    // the active partials' per-wave blocks: in their own LDS rows (one
    // phase), or in s_red after the routing partials are done (two phases)
    auto act_to_lds = [&](auto& dst) __attribute__((always_inline)) {
      acc_to_lds<NTA, NPA>(dst, wave, g, r, acc2);
      if ((r >> 2) == g) dst[wave][TM * NPA + r] = diag_of(SS, r);
    };
    if constexpr (ONE_PHASE) {
      acc_to_lds<NTF, D::NPF>(s_red, wave, g, r, acc);
      sums_to_lds(&s_red[wave][TM * D::NPF], g, r, S1, S2);
      act_to_lds(s_red2);
      __syncthreads();
      route_partials_store<N>(s_red, s_acs, a.look, G, slice, step, a.ntiles, tid);
    } else {
      route_partials<N>(s_red, s_acs, acc, S1, S2, a.look, G, slice, step, a.ntiles, tid, wave, g, r);
      act_to_lds(s_red);
      __syncthreads();
    }
    const auto& sr2 = [&]() -> const auto& {
      if constexpr (ONE_PHASE) return s_red2; else return s_red;
    }();
    constexpr int IT = (PTL * P2 + PNTHR - 1) / PNTHR;
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int u0 = tid + k * PNTHR;
      const bool in = u0 < PTL * P2;
      const int u = in ? u0 : 0;
      const int bb = u / P2, v = u % P2;
      const int t16 = PTL * step + bb;
      float x = 0.f;
#pragma unroll
      for (int c = 0; c < PSB; ++c) x += sr2[bb * PSB + c][v];
      st_b32(x, rp2, in && t16 < a.ntiles ? (uint32_t)((((size_t)t16 * G + slice) * P2 + v) * 4) : OUT_OF_RANGE);
    }
    // the next step's routing to the other buffer, last: its load was issued
    // with the next step's state, so waiting for it here rather than early
    // in this step leaves the whole compute to cover its latency (every wave
    // has finished reading that buffer before the last barrier of the
    // previous step)
    if constexpr (MS >= 0) store_route(buf ^ 1, rnext);
    __syncthreads();
  };

  while (p < nsteps) {
    const int p1 = p + nteams;
    rt = load_route(p1);
    load_xtile<E, N>(xb, X, C, p1, step_rows(p1, full, tail), lane_off);
    __builtin_amdgcn_sched_barrier(0);
    compute(xa, p, 0, rt);
    if (p1 >= nsteps) break;
    const int p2 = p1 + nteams;
    rt = load_route(p2);
    load_xtile<E, N>(xa, X, C, p2, step_rows(p2, full, tail), lane_off);
    __builtin_amdgcn_sched_barrier(0);
    compute(xb, p1, 1, rt);
    p = p2;
  }
}

// ---------------------------------------------------------------------------
// Chained pre pass with the state staged through LDS (bf16, m known, C a
// multiple of the 128-channel slice).
//
// A workgroup of SSB = 4 waves owns one slice of 4 contraction blocks for the
// launch and walks 16-token tiles, one wave per block.  The tile's rows of
// the slice (16 tokens x N streams x 256 B) go from HBM straight into LDS by
// buffer-to-LDS loads, each covering 4 token rows x 256 B: a quarter of the
// address translations per byte of a load in the MFMA fragment layout
// (16 rows x 64 B), which is what holds the register-staged kernel back.
// Two tiles' loads are in flight while one computes: a step reads its tile
// from one slot of a two-tile ring into registers, and once every wave is
// past those reads the slot takes the loads of the tile two steps on, while
// the other slot's (issued a step earlier) complete.  The two slots are
// separate LDS arrays, so that the compiler tells a read of one from the
// loads into the other.  Lane l of a load takes 16-byte chunk
// (l mod 16) xor (token within the tile) of its row, and lands at slot l of
// the load's 1 KiB, so a fragment read (one chunk of 16 tokens) touches 16
// different bank groups.  The next layer's routing fragments of the wave's
// block and this layer's active weights stay in registers for the launch;
// the active rows are read from LDS at the token's own streams.
// ---------------------------------------------------------------------------
#ifndef XHC_PRE_STAGED
#define XHC_PRE_STAGED 1
#endif
#ifndef XHC_STAGE_AUX
#define XHC_STAGE_AUX 2   // streaming: whole 128-byte lines per load here (measured ~7% faster per pre call, 13% per routing call)
#endif
#ifndef XHC_STAGE_AHEAD
#define XHC_STAGE_AHEAD 2   // tiles whose loads are in flight while one computes (1 or 2)
#endif
constexpr int STAGE_AHEAD = XHC_STAGE_AHEAD;
static_assert(STAGE_AHEAD == 1 || STAGE_AHEAD == 2, "one or two tiles ahead");
constexpr int SSB = 4;                   // contraction blocks per slice, one wave each
constexpr int SNTHR = SSB * WAVE;        // 256 threads
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Valid tokens of 16-token tile `tile` (full tiles, the ragged one, then none).
__device__ __forceinline__ int tile_rows(int tile, int full, int tail) {
  return tile < full ? TM : (tile == full ? tail : 0);
}

// A tile's rows of the slice (bf16: 16 tokens x N streams x 256 B) from HBM
// into one ring slot, by the SSB waves of the workgroup: load u of a wave
// covers stream i, token quad b (4 rows x 256 B); lane l takes chunk
// (l mod 16) xor token of row (token 4 b + l / 16) and lands at slot l.
// Past the valid tokens the loads read zero.
template <int N>
__device__ __forceinline__ void stage_tile(u32x4_t (&sx)[N][TM / 4][WAVE], const uint16_t* X, int tile, int full,
                                           int tail, int C, int slice, int wave, int lane) {
  constexpr int NQ = TM / 4, LPW = N * NQ / SSB;
  static_assert((N * NQ) % SSB == 0, "the loads of a tile split evenly over the waves");
  const uint32_t rowstride = (uint32_t)((size_t)N * C * 2);
  const int rows = tile_rows(tile, full, tail);
  const __amdgpu_buffer_rsrc_t rx =
      make_rsrc(X + (size_t)(rows > 0 ? tile : 0) * TM * N * C, (uint32_t)((size_t)rows * rowstride));
  const int lrow = lane >> 4, lslot = lane & 15;
#pragma unroll
  for (int u = 0; u < LPW; ++u) {
    const int v = wave * LPW + u, i = v / NQ, bq = v % NQ;
    const int tok = 4 * bq + lrow;
    const uint32_t voff = (uint32_t)tok * rowstride + (uint32_t)(slice * 256 + ((lslot ^ tok) << 4));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)&sx[i][bq][0], 16, (int)voff, (int)((uint32_t)i * C * 2), 0,
                                             XHC_STAGE_AUX);
  }
}
// Byte offset, within a stream's rows of a ring slot, of lane (g, r)'s
// fragment of block `wave` of the slice (token r, chunk 4 wave + g).
__device__ __forceinline__ uint32_t staged_frag(int wave, int g, int r) {
  return (uint32_t)(((r >> 2) * WAVE + 16 * (r & 3) + ((4 * wave + g) ^ r)) * 16);
}

template <class E, int N, int K, int KR, int MS, bool LOOK = true>
__global__ __launch_bounds__(SNTHR, 1) void xhc_pre_chained_s_kernel(PreChainArgs a) {
  static_assert(std::is_same<E, Bf16>::value, "the staged pre pass is written for bf16 state");
  static_assert(MS > 0 && MS <= K && MS < N, "the fixed streams are known");
  using T = typename E::T;
  using D = RouteDims<N>;
  using A = ActDims<K, KR>;
  constexpr int NTF = D::NTF, NPF = D::NPF, NSUM = D::NSUM, P1 = D::P1;
  constexpr int NTA = A::NTA, NPA = A::NPA, P2 = A::P2;
  constexpr int KB = E::KB, VEC = E::VEC;
  constexpr int FS = MS;                       // streams whose routing fragments are read
  constexpr int NQ = TM / 4;                   // token quads per tile
  static_assert(SSB * KB * 2 == 256, "a load covers 4 rows x 256 B");
  static_assert(TM * N / 4 <= WAVE && TM * K / 4 <= WAVE, "a tile's routing rows fit one wave each");
  __shared__ u32x4_t s_x0[N][NQ][WAVE];        // ring of two tiles: [stream][token quad][16-byte slot]
  __shared__ u32x4_t s_x1[N][NQ][WAVE];
  __shared__ float s_red[SSB][NSUM];
  __shared__ float s_red2[SSB][P2];
  __shared__ float s_acs[16];
  __shared__ float s_rh[2][TM * N];
  __shared__ int s_ri[2][TM * K];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int C = a.C, G = a.G, nkbC = C / KB;
  const int slice = blockIdx.x % G, team = blockIdx.x / G, nteams = gridDim.x / G;
  const int ntiles = a.ntiles;
  const int kb0 = slice * SSB + wave;          // this wave's contraction block
  const int full = a.T / TM, tail = a.T % TM;

  auto dma = [&](int tile, auto qc) __attribute__((always_inline)) {
    if constexpr (decltype(qc)::value == 0)
      stage_tile<N>(s_x0, reinterpret_cast<const uint16_t*>(a.X), tile, full, tail, C, slice, wave, lane);
    else
      stage_tile<N>(s_x1, reinterpret_cast<const uint16_t*>(a.X), tile, full, tail, C, slice, wave, lane);
  };
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;
  // a tile's routing rows: wave 0 the h_pre rows, wave 1 the active lists
  // (units past the valid tokens read zero; other waves read nothing)
  auto load_route = [&](int tile) __attribute__((always_inline)) {
    const int rows = tile_rows(tile, full, tail);
    const size_t t0 = rows > 0 ? (size_t)TM * tile : 0;
    const bool wh = wave == 0;
    const void* base = wh ? (const void*)(a.h_pre + t0 * N) : (const void*)(a.idx + t0 * K);
    const uint32_t bytes = wh ? (uint32_t)(rows * N * 4) : (wave == 1 ? (uint32_t)(rows * K * 4) : 0u);
    return ld_b128(make_rsrc(base, bytes), (uint32_t)(lane * 16), 0);
  };
  auto store_route = [&](int q, const u32x4_t& v) __attribute__((always_inline)) {
    if (wave == 0) reinterpret_cast<u32x4_t*>(&s_rh[q][0])[lane] = v;
    else if (wave == 1 && lane < TM * K / 4) reinterpret_cast<u32x4_t*>(&s_ri[q][0])[lane] = v;
  };

  // ---- weights in registers -------------------------------------------------
  // (through resources, unconditionally: a block past C reads zeros)
  const bool kvalid = kb0 < nkbC;
  const __amdgpu_buffer_rsrc_t rwn = make_rsrc(LOOK ? a.wnext : a.wact, LOOK ? (uint32_t)((size_t)N * nkbC * NTF * WAVE * 16) : 0u);
  const __amdgpu_buffer_rsrc_t rwa = make_rsrc(a.wact, (uint32_t)((size_t)K * nkbC * NTA * WAVE * 16));
  const uint32_t lo = kvalid ? (uint32_t)lane * 16 : OUT_OF_RANGE;
  u32x4_t wn[LOOK ? N - FS : 1][NTF];   // next layer's routing fragments of this block, streams FS .. N-1
  if constexpr (LOOK) {
#pragma unroll
    for (int i = FS; i < N; ++i)
#pragma unroll
      for (int n = 0; n < NTF; ++n)
        wn[i - FS][n] = ld_b128(rwn, lo, (uint32_t)((((size_t)i * nkbC + kb0) * NTF + n) * WAVE * 16));
  }
  u32x4_t wa[K][NTA];
#pragma unroll
  for (int j = 0; j < K; ++j)
#pragma unroll
    for (int n = 0; n < NTA; ++n)
      wa[j][n] = ld_b128(rwa, lo, (uint32_t)((((size_t)j * nkbC + kb0) * NTA + n) * WAVE * 16));
  // column sums of the slice's W_r over all N streams (the same fragments in
  // the same order as the register-staged kernels)
  if constexpr (LOOK) {
    const u32x4_t ones = ones_frag<E>();
    u32x4_t f[N];
#pragma unroll
    for (int i = 0; i < N; ++i) f[i] = ld_b128(rwn, lo, (uint32_t)((((size_t)i * nkbC + kb0) * NTF) * WAVE * 16));
    f32x4_t acs = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < N; ++i) acs = E::mma(acs, ones, f[i]);
    if (lane < 16) s_red[wave][lane] = acs[0];
  }
  __syncthreads();
  if (tid < 16) {
    float v = 0.f;
#pragma unroll
    for (int c = 0; c < SSB; ++c) v += s_red[c][tid];
    s_acs[tid] = v;
  }

  int p = team;
  if (p >= ntiles) return;
  constexpr int LPW = N * NQ / SSB;   // buffer-to-LDS loads per wave and tile
  dma(p, Q0{});
  {
    const u32x4_t rt = load_route(p);
    if constexpr (STAGE_AHEAD == 2) dma(p + nteams, Q1{});
    wait_vmcnt<STAGE_AHEAD == 2 ? LPW : 0>();   // the first tile and its routing rows
    store_route(0, rt);
  }
  stage_barrier<STAGE_AHEAD == 2 ? LPW : 0>();

  const __amdgpu_buffer_rsrc_t rlook =
      make_rsrc(LOOK ? a.look : a.part2, LOOK ? (uint32_t)((size_t)ntiles * G * P1 * 4) : 0u);
  const __amdgpu_buffer_rsrc_t rp2 = make_rsrc(a.part2, (uint32_t)((size_t)ntiles * G * P2 * 4));
  // byte offset of this lane's fragment (token r, chunk 4 wave + g) within a
  // stream's [quad][slot] block of the ring
  const uint32_t fofs = staged_frag(wave, g, r);
  const u32x4_t zero = u32x4_t{0u, 0u, 0u, 0u};
  const u32x4_t ones = ones_frag<E>();

  // The partial sums of the previous tile (its waves' blocks in s_red and
  // s_red2), stored per (tile, slice); a tile past the last stores nothing.
  constexpr int IT1 = (P1 + SNTHR - 1) / SNTHR, IT2 = (P2 + SNTHR - 1) / SNTHR;
  auto store_partials = [&](int tile) __attribute__((always_inline)) {
    const bool tin = tile >= 0 && tile < ntiles;
    if constexpr (LOOK) {
#pragma unroll
      for (int it = 0; it < IT1; ++it) {
        const int u0 = tid + it * SNTHR;
        const bool in = u0 < P1;
        const int u = in ? u0 : 0;
        float x = 0.f;
#pragma unroll
        for (int c = 0; c < SSB; ++c) x += s_red[c][u < NSUM ? u : 0];
        if (u >= NSUM) x = s_acs[u - NSUM >= 0 ? u - NSUM : 0];
        st_b32(x, rlook, in && tin ? (uint32_t)((((size_t)tile * G + slice) * P1 + u) * 4) : OUT_OF_RANGE);
      }
    }
#pragma unroll
    for (int it = 0; it < IT2; ++it) {
      const int u0 = tid + it * SNTHR;
      const bool in = u0 < P2;
      const int u = in ? u0 : 0;
      float x = 0.f;
#pragma unroll
      for (int c = 0; c < SSB; ++c) x += s_red2[c][u];
      st_b32(x, rp2, in && tin ? (uint32_t)((((size_t)tile * G + slice) * P2 + u) * 4) : OUT_OF_RANGE);
    }
  };

  // One tile, in ring slot Q (a constant, so that the compiler can tell
  // accesses to the two slots apart).  Every LDS read of the step comes
  // before the next tile's loads into the other slot are issued: after a
  // buffer-to-LDS load the compiler makes any later LDS read it cannot
  // separate from that load's target wait for it.
  // vector memory operations of one step, every one issued unconditionally:
  // the partial stores, the routing rows, the tile loads, the store of inp
  constexpr int VM_STEP = (LOOK ? IT1 : 0) + IT2 + 1 + LPW + 1;
  int pprev = -1;
  auto tile_step = [&](auto qc) __attribute__((always_inline)) {
    constexpr int q = decltype(qc)::value;
    const int p1 = p + nteams;
    const char* xq = reinterpret_cast<const char*>(q == 0 ? &s_x0[0][0][0] : &s_x1[0][0][0]);
    constexpr uint32_t SBYTES = NQ * WAVE * 16;   // bytes of one stream's tile rows in the ring
    // ---- reads: routing rows, the tile's fragments, the active rows
    int I[K];
    uint32_t amask = 0;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      int v = s_ri[q][r * K + j];
      v = v < 0 ? 0 : (v >= N ? N - 1 : v);
      I[j] = v;
      amask |= 1u << v;
    }
    float hp[N];
#pragma unroll
    for (int i = 0; i < N; ++i) hp[i] = s_rh[q][r * N + i];
    u32x4_t x[N], gat[K];
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = *reinterpret_cast<const u32x4_t*>(xq + (uint32_t)i * SBYTES + fofs);
#pragma unroll
    for (int j = 0; j < K; ++j)
      gat[j] = j < MS ? x[j < MS ? j : 0] : *reinterpret_cast<const u32x4_t*>(xq + (uint32_t)I[j] * SBYTES + fofs);
    // ---- the previous tile's partial sums, then every wave is past its reads
    store_partials(pprev);
    stage_barrier<63>();
    // ---- the next tile's routing rows, then the loads of the tile two steps
    // on into this slot (or, one ahead, of the next into the other); past the
    // last tile they read nothing
    const u32x4_t rnext = load_route(p1);
    if constexpr (STAGE_AHEAD == 2) dma(p1 + nteams, qc);
    else dma(p1, std::integral_constant<int, q ^ 1>{});
    // ---- compute from registers
    float o[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[e] = 0.f;
    f32x4_t acc[NTF], S1 = f32x4_t{0.f, 0.f, 0.f, 0.f}, S2 = S1;
#pragma unroll
    for (int n = 0; n < NTF; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < N; ++i) {
      // the dense read, and the next layer's routing projection of the rows
      // this layer leaves as they are
      float f[VEC];
      E::unpack(x[i], f);
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[e] = fmaf(hp[i], f[e], o[e]);
      if (LOOK && i >= FS) {
        const u32x4_t v = ((amask >> i) & 1u) ? zero : x[i];
        mma_sums<E>(v, ones, S1, S2);
#pragma unroll
        for (int n = 0; n < NTF; ++n) acc[n] = E::mma(acc[n], v, wn[i - FS][n]);
      }
    }
    {
      const int rows = kvalid ? tile_rows(p, full, tail) : 0;
      const __amdgpu_buffer_rsrc_t ri =
          make_rsrc(reinterpret_cast<T*>(a.inp) + (size_t)(rows > 0 ? p : 0) * TM * C, (uint32_t)((size_t)rows * C * sizeof(T)));
      st_b128<INP_ST_AUX>(E::packv_cvt(o), ri, (uint32_t)(((size_t)r * C + kb0 * KB + VEC * g) * sizeof(T)));
    }
    // the k active rows: sum of squares and this layer's active projection
    f32x4_t acc2[NTA], SS = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < NTA; ++n) acc2[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < K; ++j) {
      SS = E::mma(SS, gat[j], gat[j]);
#pragma unroll
      for (int n = 0; n < NTA; ++n) acc2[n] = E::mma(acc2[n], gat[j], wa[j][n]);
    }
    // ---- this tile's per-wave partials and the next tile's routing rows to
    // LDS; then this wave's loads of the next tile are complete (two ahead:
    // all but this step's), and after the barrier every wave's are
    if constexpr (LOOK) {
#pragma unroll
      for (int n = 0; n < NTF; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_red[wave][(4 * g + i) * NPF + n * 16 + r] = acc[n][i];
      sums_to_lds(&s_red[wave][TM * NPF], g, r, S1, S2);
    }
#pragma unroll
    for (int n = 0; n < NTA; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_red2[wave][(4 * g + i) * NPA + n * 16 + r] = acc2[n][i];
    if ((r >> 2) == g) s_red2[wave][TM * NPA + r] = diag_of(SS, r);
    store_route(q ^ 1, rnext);
    stage_barrier<STAGE_AHEAD == 2 ? VM_STEP : 0>();
    pprev = p;
    p = p1;
  };
  // two tiles per trip and the only exit at its end (a tile past the last
  // loads and stores nothing)
  do {
    tile_step(Q0{});
    tile_step(Q1{});
  } while (p < ntiles);
  store_partials(pprev);
  wait_vmcnt<0>();   // no load into LDS outlives the workgroup
}

// xHC-Flash readouts staged through LDS (N = 16, bf16, C a multiple of 128):
// the NPRE weighted sums of a token's streams (the pages' readout equation
// of xHC-Flash) from one pass over the state, as flash_read_kernel computes
// them and in its order, with the rows loaded as in the staged pre pass (a
// persistent workgroup of 4 waves per 128-channel slice, 16-token tiles,
// two tiles in flight).  With MASK, readouts 1.. leave out the token's
// active streams (the non-active bases of xHC-Flash-4sub).
struct FlashReadSArgs {
  const void* X;
  void* out[4];
  const float* h_pre[4];
  const int* idx;   // MASK only
  int T, C, G, K, ntiles;
};
template <int NPRE, bool MASK>
__global__ __launch_bounds__(SNTHR, 1) void flash_read_s_kernel(FlashReadSArgs a) {
  using E = Bf16;
  using T = typename E::T;
  constexpr int N = 16, KB = E::KB, VEC = E::VEC, NQ = TM / 4;
  constexpr int KMAX = 4;
  static_assert(NPRE * TM * N / 4 <= SNTHR, "a tile's readout weights take one unit per thread");
  __shared__ u32x4_t s_x0[N][NQ][WAVE];
  __shared__ u32x4_t s_x1[N][NQ][WAVE];
  __shared__ float s_h[2][NPRE][TM * N];
  __shared__ int s_ri[2][TM * KMAX];
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int C = a.C, G = a.G, K = a.K;
  const int slice = blockIdx.x % G, team = blockIdx.x / G, nteams = gridDim.x / G;
  const int ntiles = a.ntiles;
  const int kb0 = slice * SSB + wave;
  const int full = a.T / TM, tail = a.T % TM;
  const uint16_t* X = reinterpret_cast<const uint16_t*>(a.X);

  auto dma = [&](int tile, auto qc) __attribute__((always_inline)) {
    if constexpr (decltype(qc)::value == 0) stage_tile<N>(s_x0, X, tile, full, tail, C, slice, wave, lane);
    else stage_tile<N>(s_x1, X, tile, full, tail, C, slice, wave, lane);
  };
  // a tile's readout weights: thread u loads 16 bytes of readout u / 64
  // (a 16 x 16 float block), and (MASK) the first 16 lanes of wave 0 the
  // active lists; units past the valid tokens read zero
  struct Rows { u32x4_t h, li; };
  auto load_rows = [&](int tile) __attribute__((always_inline)) {
    const int rows = tile_rows(tile, full, tail);
    const size_t t0 = rows > 0 ? (size_t)TM * tile : 0;
    const int q = wave < NPRE ? wave : 0;   // uniform over the wave
    Rows v;
    v.h = ld_b128(make_rsrc(a.h_pre[q] + t0 * N, wave < NPRE ? (uint32_t)(rows * N * 4) : 0u), (uint32_t)(lane * 16), 0);
    if constexpr (MASK)
      v.li = ld_b128(make_rsrc(a.idx + t0 * K, (uint32_t)(rows * K * 4)), (uint32_t)(tid * 16), 0);
    return v;
  };
  auto store_rows = [&](int q, const Rows& v) __attribute__((always_inline)) {
    if (wave < NPRE) reinterpret_cast<u32x4_t*>(&s_h[q][wave][0])[lane] = v.h;
    if constexpr (MASK)
      if (tid * 4 < TM * K) reinterpret_cast<u32x4_t*>(&s_ri[q][0])[tid] = v.li;
  };

  int p = team;
  if (p >= ntiles) return;
  constexpr int LPW = N * NQ / SSB;
  dma(p, Q0{});
  {
    const Rows v = load_rows(p);
    dma(p + nteams, Q1{});
    wait_vmcnt<LPW>();
    store_rows(0, v);
  }
  stage_barrier<LPW>();

  const uint32_t fofs = staged_frag(wave, g, r);
  constexpr uint32_t SBYTES = NQ * WAVE * 16;
  // vector memory operations of one step: the next tile's rows, the tile
  // loads, the readout stores
  constexpr int VM_STEP = 1 + (MASK ? 1 : 0) + LPW + NPRE;
  auto tile_step = [&](auto qc) __attribute__((always_inline)) {
    constexpr int q = decltype(qc)::value;
    const int p1 = p + nteams;
    const char* xq = reinterpret_cast<const char*>(q == 0 ? &s_x0[0][0][0] : &s_x1[0][0][0]);
    u32x4_t x[N];
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = *reinterpret_cast<const u32x4_t*>(xq + (uint32_t)i * SBYTES + fofs);
    float h[NPRE][N];
#pragma unroll
    for (int qq = 0; qq < NPRE; ++qq)
#pragma unroll
      for (int i = 0; i < N; ++i) h[qq][i] = s_h[q][qq][r * N + i];
    uint32_t mk = 0;
    if constexpr (MASK) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        const int v = j < K ? s_ri[q][r * K + j] : -1;
        if (v >= 0 && v < N) mk |= 1u << v;
      }
    }
    stage_barrier<63>();   // every wave is past its reads of this slot
    const Rows nx = load_rows(p1);
    dma(p1 + nteams, qc);
    float acc[NPRE][VEC];
#pragma unroll
    for (int qq = 0; qq < NPRE; ++qq)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[qq][e] = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      float f[VEC];
      E::unpack(x[i], f);
#pragma unroll
      for (int qq = 0; qq < NPRE; ++qq) {
        const float hv = (qq > 0 && ((mk >> i) & 1u)) ? 0.f : h[qq][i];
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[qq][e] = fmaf(hv, f[e], acc[qq][e]);
      }
    }
    {
      const int rows = kb0 < C / KB ? tile_rows(p, full, tail) : 0;
      const size_t t0 = rows > 0 ? (size_t)TM * p : 0;
      const uint32_t o = (uint32_t)(((size_t)r * C + (size_t)kb0 * KB + VEC * g) * sizeof(T));
#pragma unroll
      for (int qq = 0; qq < NPRE; ++qq)
        st_b128<CP_NT>(E::packv(acc[qq]),
                       make_rsrc(reinterpret_cast<T*>(a.out[qq]) + t0 * C, (uint32_t)((size_t)rows * C * sizeof(T))), o);
    }
    store_rows(q ^ 1, nx);
    stage_barrier<VM_STEP>();
    p = p1;
  };
  do {
    tile_step(Q0{});
    tile_step(Q1{});
  } while (p < ntiles);
  wait_vmcnt<0>();   // no load into LDS outlives the workgroup
}

bool flash_read_s_applies(const Plan& P) {
  return XHC_PRE_STAGED && P.N == 16 && P.dtype == XHC_BF16 && P.C % (SSB * Bf16::KB) == 0 && P.ntiles > 0 &&
         P.K <= 4;
}

// Routing projection of a whole state (first layer of a chain), with the
// state staged through LDS as in the pre pass above: every stream's rows,
// no masking, the routing partials alone.  D gives the column tiles and the
// partial layout: RouteDims<N> (W_r, W_pre) or, for xHC-Flash,
// FlashDims16 (router, attention and MLP pre-maps).
template <class E, int N, class D = RouteDims<N>>
__global__ __launch_bounds__(SNTHR, 1) void xhc_proj_s_kernel(ProjPArgs a) {
  static_assert(std::is_same<E, Bf16>::value, "the staged projection is written for bf16 state");
  constexpr int NTF = D::NTF, NPF = D::NPF, NSUM = D::NSUM, P1 = D::P1;
  constexpr int KB = E::KB;
  constexpr int NQ = TM / 4;
  static_assert(SSB * KB * 2 == 256, "a load covers 4 rows x 256 B");
  __shared__ u32x4_t s_x0[N][NQ][WAVE];
  __shared__ u32x4_t s_x1[N][NQ][WAVE];
  __shared__ float s_red[SSB][NSUM];
  __shared__ float s_acs[16];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int C = a.C, G = a.G, nkbC = C / KB;
  const int slice = blockIdx.x % G, team = blockIdx.x / G, nteams = gridDim.x / G;
  const int ntiles = a.ntiles;
  const int kb0 = slice * SSB + wave;
  const int full = a.T / TM, tail = a.T % TM;
  const uint16_t* X = reinterpret_cast<const uint16_t*>(a.X);

  // the routing fragments of this block, every stream, in registers; the
  // slice's column sums of W_r (the same fragments in the same order as the
  // register-staged kernels)
  const bool kvalid = kb0 < nkbC;
  const __amdgpu_buffer_rsrc_t rwn = make_rsrc(a.wfull, (uint32_t)((size_t)N * nkbC * NTF * WAVE * 16));
  const uint32_t lo = kvalid ? (uint32_t)lane * 16 : OUT_OF_RANGE;
  u32x4_t wn[N][NTF];
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int n = 0; n < NTF; ++n) wn[i][n] = ld_b128(rwn, lo, (uint32_t)((((size_t)i * nkbC + kb0) * NTF + n) * WAVE * 16));
  const u32x4_t ones = ones_frag<E>();
  {
    f32x4_t acs = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < N; ++i) acs = E::mma(acs, ones, wn[i][0]);
    if (lane < 16) s_red[wave][lane] = acs[0];
  }
  __syncthreads();
  if (tid < 16) {
    float v = 0.f;
#pragma unroll
    for (int c = 0; c < SSB; ++c) v += s_red[c][tid];
    s_acs[tid] = v;
  }
  int p = team;
  if (p >= ntiles) return;
  constexpr int LPW = N * NQ / SSB;
  stage_tile<N>(s_x0, X, p, full, tail, C, slice, wave, lane);
  if constexpr (STAGE_AHEAD == 2) stage_tile<N>(s_x1, X, p + nteams, full, tail, C, slice, wave, lane);
  stage_barrier<STAGE_AHEAD == 2 ? LPW : 0>();

  const __amdgpu_buffer_rsrc_t rpart = make_rsrc(a.part, (uint32_t)((size_t)ntiles * G * P1 * 4));
  const uint32_t fofs = staged_frag(wave, g, r);
  constexpr int IT1 = (P1 + SNTHR - 1) / SNTHR;
  auto store_partials = [&](int tile) __attribute__((always_inline)) {
    const bool tin = tile >= 0 && tile < ntiles;
#pragma unroll
    for (int it = 0; it < IT1; ++it) {
      const int u0 = tid + it * SNTHR;
      const bool in = u0 < P1;
      const int u = in ? u0 : 0;
      float x = 0.f;
#pragma unroll
      for (int c = 0; c < SSB; ++c) x += s_red[c][u < NSUM ? u : 0];
      if (u >= NSUM) x = s_acs[u - NSUM >= 0 ? u - NSUM : 0];
      st_b32(x, rpart, in && tin ? (uint32_t)((((size_t)tile * G + slice) * P1 + u) * 4) : OUT_OF_RANGE);
    }
  };
  constexpr int VM_STEP = IT1 + LPW;   // vector memory operations of one step
  int pprev = -1;
  auto tile_step = [&](auto qc) __attribute__((always_inline)) {
    constexpr int q = decltype(qc)::value;
    const int p1 = p + nteams;
    const char* xq = reinterpret_cast<const char*>(q == 0 ? &s_x0[0][0][0] : &s_x1[0][0][0]);
    constexpr uint32_t SBYTES = NQ * WAVE * 16;
    u32x4_t x[N];
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = *reinterpret_cast<const u32x4_t*>(xq + (uint32_t)i * SBYTES + fofs);
    store_partials(pprev);
    stage_barrier<63>();
    // two ahead: the tile two steps on into this slot; one ahead: the next
    // into the other
    if constexpr ((STAGE_AHEAD == 2) == (q == 0)) stage_tile<N>(s_x0, X, STAGE_AHEAD == 2 ? p1 + nteams : p1, full, tail, C, slice, wave, lane);
    else stage_tile<N>(s_x1, X, STAGE_AHEAD == 2 ? p1 + nteams : p1, full, tail, C, slice, wave, lane);
    f32x4_t acc[NTF], S1 = f32x4_t{0.f, 0.f, 0.f, 0.f}, S2 = S1;
#pragma unroll
    for (int n = 0; n < NTF; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < N; ++i) {
      mma_sums<E>(x[i], ones, S1, S2);
#pragma unroll
      for (int n = 0; n < NTF; ++n) acc[n] = E::mma(acc[n], x[i], wn[i][n]);
    }
#pragma unroll
    for (int n = 0; n < NTF; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_red[wave][(4 * g + i) * NPF + n * 16 + r] = acc[n][i];
    sums_to_lds(&s_red[wave][TM * NPF], g, r, S1, S2);
    stage_barrier<STAGE_AHEAD == 2 ? VM_STEP : 0>();
    pprev = p;
    p = p1;
  };
  do {
    tile_step(std::integral_constant<int, 0>{});
    tile_step(std::integral_constant<int, 1>{});
  } while (p < ntiles);
  store_partials(pprev);
  wait_vmcnt<0>();   // no load into LDS outlives the workgroup
}

// ---------------------------------------------------------------------------
// Persistent post pass of a layer with a next layer: the rewritten rows'
// share of the next layer's routing (the correction), and with it the
// layer's write (WR = 1 attention-type, 4 MLP-type), so the new rows are
// contracted from registers instead of being read back (WR = 0: the
// correction alone, of rows another kernel wrote).
//
// A workgroup owns one slice of PSB contraction blocks for the whole launch
// with the next layer's routing fragments of that slice in LDS, and walks
// steps of PTL 16-token tiles, one wave per (tile, block); lane (g, r) holds
// token r of its tile, VEC channels of its block.  Per step a lane loads the
// k active rows of its token and its row of out (MLP-type: also the row 16
// tokens earlier), forms the write basis (MLP-type: out and its three causal
// convolutions, the lags taken from neighbouring lanes by DPP row shifts,
// conv weights of the slice in LDS), and the new rows
// x'_j = sum_i H_res[j][i] x_{I_i} + sum_v Q[j][v] basis_v with the
// per-sublayer write's arithmetic in its order (Q = p_j H_post[j] for the
// attention type; diag(p) H_post Tm, Tm the Gram-Schmidt map, precomputed
// per token for the MLP type), and stores them in place; then per stream i
// of the next layer the MFMA takes, per token, the new row that sits in
// stream i (zero if none) against that stream's fragments, and the new
// rows' sums of x and x^2 go through the matrix cores as in the pre pass.
// The partials of the PSB waves of a tile are summed in LDS and written per
// (tile, slice) in the routing partials' layout.
//
// The state loads run PD steps ahead (PD + 1 register sets), as the rows of
// a step are few bytes per lane.  Their addresses need the active lists PD
// steps ahead, so the lists run one step further: loaded into LDS PD + 1
// steps ahead, a ring of PD + 2 slots.  The write coefficients of the next
// step are loaded during this one, double-buffered in LDS.
// ---------------------------------------------------------------------------
struct PostPArgs {
  void* X;
  const void* out;                      // a write: [T][C]
  const int* idx;                       // [T][K]
  const float *h_res, *p, *h_post;      // a write: [T][K][K]; attention-type: [T][K], [T][K]
  const float* wq;                      // MLP-type write: [T][K][4] coefficients diag(p) H_post Tm
  const float* conv_w;                  // MLP-type write: [24][C]
  int T, S, C, G, ntiles;
  const uint4* wnext;                   // next layer's packed [W_r | W_pre]
  float* corr;                          // [ntiles][G][P1] (the first NSUM entries of each)
};

#ifndef XHC_POST_PD
#define XHC_POST_PD 1
#endif
#ifndef XHC_POST_NS_SPLIT
#define XHC_POST_NS_SPLIT 1
#endif
constexpr int POST_PD = XHC_POST_PD;   // steps of state loads in flight ahead of the compute (1 measured best of 1, 2, 3)

// Calls f(std::integral_constant<int, Q>) for Q = 0 .. NQ - 1.
template <int NQ, int Q = 0, class F>
__device__ __forceinline__ void for_each_c(F&& f) {
  if constexpr (Q < NQ) {
    f(std::integral_constant<int, Q>{});
    for_each_c<NQ, Q + 1>(f);
  }
}

template <int K>
struct PStep {
  u32x4_t x[K];
  u32x4_t o;    // out (a write)
  u32x4_t op;   // out 16 tokens before (MLP-type write)
};

template <class E, int N, int K, int MS, int WR>
__global__ __launch_bounds__(PNTHR, 1) void xhc_post_p_kernel(PostPArgs a) {
  using T = typename E::T;
  using D = RouteDims<N>;
  constexpr int NTF = D::NTF, NPF = D::NPF, NSUM = D::NSUM, P1 = D::P1;
  constexpr int KB = E::KB, VEC = E::VEC;
  constexpr int PD = POST_PD, NR = PD + 1, NI = PD + 2;
  constexpr int STT = PTL * TM;                     // tokens per step
  constexpr int SLC = PSB * KB;                     // channels of a slice
  static_assert(WR == 0 || WR == 1 || WR == 4, "write kinds: none, attention-type, MLP-type");
  // per-step rows moved through LDS, in 16-byte units: the active lists,
  // then for a write H_res and (attention-type) p and H_post, or (MLP-type)
  // the write coefficients Q = diag(p) H_post (Gram-Schmidt map)
  constexpr int E2 = WR == 4 ? 4 * K : (WR == 1 ? K : 0), E3 = WR == 1 ? K : 0;
  constexpr int UI = STT * K / 4, UH = WR ? STT * K * K / 4 : 0, U2 = STT * E2 / 4, U3 = STT * E3 / 4;
  // each array is loaded by whole waves of its own, so that its buffer
  // resource stays uniform over a wave
  constexpr int WI = (UI + WAVE - 1) / WAVE, WH = (UH + WAVE - 1) / WAVE, W2 = (U2 + WAVE - 1) / WAVE,
                W3 = (U3 + WAVE - 1) / WAVE;
  static_assert((STT * K) % 4 == 0 && WI + WH + W2 + W3 <= TWV, "a step's rows fit one unit per thread");
  constexpr int CF = WR ? STT * (K * K + E2 + E3) : 1;
  // the per-tile partial sums: per wave, or (MLP-type, whose conv weights
  // take the room) per pair of block waves, added in two rounds
  constexpr int RW = WR == 4 ? PTL * 2 : TWV;
  __shared__ u32x4_t s_w[PSB][N][NTF][WAVE];
  __shared__ float s_red[RW][NSUM];
  __shared__ int s_idx[NI][STT * K];
  __shared__ float s_cf[2][CF];
  __shared__ float s_cw[WR == 4 ? 24 : 1][WR == 4 ? SLC : 1];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = wave / PSB, cb = wave % PSB;
  const int C = a.C, G = a.G, nkbC = C / KB;
  const int slice = blockIdx.x % G, team = blockIdx.x / G, nteams = gridDim.x / G;
  const int nsteps = (a.ntiles + PTL - 1) / PTL;
  const int kb0 = slice * PSB + cb;
  const bool kvalid = kb0 < nkbC;
  const int tau = TM * b + r;   // the lane's token within a step
  const int full = a.T / STT, tail = a.T % STT;
  // byte offset of the lane's fragment within its token's row of one stream
  const uint32_t cofs = (uint32_t)(((size_t)kb0 * KB + VEC * g) * sizeof(T));
  T* X = reinterpret_cast<T*>(a.X);
  const T* out = reinterpret_cast<const T*>(a.out);

  // one 16-byte unit of a step's rows; the resource spans the step's valid
  // tokens, so anything past them reads zero.  Every wave issues the load
  // (one without a share reads an empty range), so that no memory operation
  // sits under a branch.
  const float* arr2 = WR == 4 ? a.wq : a.p;
  auto load_unit = [&](int step, bool lists, bool coefs) __attribute__((always_inline)) {
    const int valid = step_rows(step, full, tail);
    const size_t ts = valid > 0 ? (size_t)STT * step : 0;
    const void* base = a.idx;
    uint32_t bytes = 0, first = 0;
    if (wave < WI) {
      base = a.idx + ts * K;
      bytes = lists ? (uint32_t)(valid * K * 4) : 0u;
    } else if (wave < WI + WH) {
      base = a.h_res + ts * K * K;
      bytes = coefs ? (uint32_t)(valid * K * K * 4) : 0u;
      first = WI;
    } else if (wave < WI + WH + W2) {
      base = arr2 + ts * E2;
      bytes = coefs ? (uint32_t)(valid * E2 * 4) : 0u;
      first = WI + WH;
    } else if (wave < WI + WH + W2 + W3) {
      base = a.h_post + ts * E3;
      bytes = coefs ? (uint32_t)(valid * E3 * 4) : 0u;
      first = WI + WH + W2;
    }
    return ld_b128(make_rsrc(base, bytes), (uint32_t)(16 * ((wave - (int)first) * WAVE + lane)), 0);
  };
  // s_cf: H_res [STT][K][K], then p [STT][K] or Q [STT][K][4], then H_post [STT][K]
  auto store_unit = [&](const u32x4_t& v, int islot, int cbuf, bool lists, bool coefs) __attribute__((always_inline)) {
    if (wave < WI) {
      const int u = wave * WAVE + lane;
      if (lists && u < UI) *reinterpret_cast<u32x4_t*>(&s_idx[islot][4 * u]) = v;
    } else if (wave < WI + WH + W2 + W3 && coefs) {
      // q: the unit within its array; base: the array's first unit in s_cf
      int q, n, base;
      if (wave < WI + WH) { q = (wave - WI) * WAVE + lane; n = UH; base = 0; }
      else if (wave < WI + WH + W2) { q = (wave - WI - WH) * WAVE + lane; n = U2; base = UH; }
      else { q = (wave - WI - WH - W2) * WAVE + lane; n = U3; base = UH + U2; }
      if (q < n) *reinterpret_cast<u32x4_t*>(&s_cf[cbuf][4 * (base + q)]) = v;
    }
  };
  // The step's rows of X (of out): a wave whose block lies past C gets an
  // empty range, so its loads read zeros and its stores are dropped.
  auto x_rsrc = [&](int step) __attribute__((always_inline)) {
    const int rows = kvalid ? step_rows(step, full, tail) : 0;
    return make_rsrc(X + (size_t)(rows > 0 ? step : 0) * STT * N * C, (uint32_t)((size_t)rows * N * C * sizeof(T)));
  };
  // the lane's state loads of a step: its k active rows; for a write its row
  // of out, and (MLP-type) the row 16 tokens before, whose tile supplies the
  // lags that reach back past this tile's first token
  auto issue = [&](PStep<K>& st, int step, int islot) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rx = x_rsrc(step);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      int ij = s_idx[islot][tau * K + j];
      ij = ij < 0 ? 0 : (ij >= N ? N - 1 : ij);
      st.x[j] = ld_b128<STATE_AUX>(rx, (uint32_t)(((size_t)tau * N + ij) * C * sizeof(T)) + cofs, 0);
    }
    if constexpr (WR != 0) {
      const int rows = kvalid ? step_rows(step, full, tail) : 0;
      const size_t t0 = rows > 0 ? (size_t)STT * step : 0;
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(out + t0 * C, (uint32_t)((size_t)rows * C * sizeof(T)));
      st.o = ld_b128(ro, (uint32_t)((size_t)tau * C * sizeof(T)) + cofs, 0);
      if constexpr (WR == 4) {
        // tokens t0 - 16 .. t0 + rows - 1 (from t0 on the first step)
        const bool back = t0 >= (size_t)TM;
        const __amdgpu_buffer_rsrc_t rp = make_rsrc(out + (back ? t0 - TM : 0) * C,
                                                    (uint32_t)((size_t)(rows > 0 ? rows + (back ? TM : 0) : 0) * C *
                                                               sizeof(T)));
        const uint32_t po = back ? (uint32_t)((size_t)tau * C * sizeof(T)) + cofs
                                 : (tau >= TM ? (uint32_t)((size_t)(tau - TM) * C * sizeof(T)) + cofs : OUT_OF_RANGE);
        st.op = ld_b128(rp, po, 0);
      }
    }
  };
  const __amdgpu_buffer_rsrc_t rcorr = make_rsrc(a.corr, (uint32_t)((size_t)a.ntiles * G * P1 * 4));

  // prologue: routing fragments and column sums of the slice, (MLP-type) its
  // conv weights, the lists of the first PD + 1 steps, the coefficients of
  // the first, then the state loads of the first PD steps
  load_wslice<N, NTF>(s_w, a.wnext, nkbC, slice, tid);
  if constexpr (WR == 4) {
    // all loads first, then the stores: one memory round trip
    static_assert((24 * SLC) % PNTHR == 0, "the conv weights of a slice split evenly over the threads");
    constexpr int NW = 24 * SLC / PNTHR;
    float cw[NW];
#pragma unroll
    for (int it = 0; it < NW; ++it) {
      const int u = tid + it * PNTHR, tap = u / SLC, c = slice * SLC + u % SLC;
      cw[it] = c < C ? a.conv_w[(size_t)tap * C + c] : 0.f;
    }
#pragma unroll
    for (int it = 0; it < NW; ++it) {
      const int u = tid + it * PNTHR;
      s_cw[u / SLC][u % SLC] = cw[it];
    }
  }
  {
    u32x4_t v[NI - 1];
#pragma unroll
    for (int d = 0; d < NI - 1; ++d) v[d] = load_unit(team + d * nteams, true, d == 0);
#pragma unroll
    for (int d = 0; d < NI - 1; ++d) store_unit(v[d], d, 0, true, d == 0);
  }
  __syncthreads();
  PStep<K> sr[NR];
#pragma unroll
  for (int d = 0; d < PD; ++d) issue(sr[d], team + d * nteams, d);
  // The first steps' loads complete here, once: otherwise the compiler's
  // waits at the loop head, which must also hold on entry (where these are
  // the latest loads), would drain the prefetch in every later trip.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

  const u32x4_t zero = u32x4_t{0u, 0u, 0u, 0u};
  const u32x4_t ones = ones_frag<E>();
  auto compute = [&](const PStep<K>& st, int step, int islot, int cbuf) __attribute__((always_inline)) {
    int I[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int v = s_idx[islot][tau * K + j];
      I[j] = v < 0 ? 0 : (v >= N ? N - 1 : v);
    }
    u32x4_t xn[K];
    if constexpr (WR != 0) {
      constexpr int NB = WR;   // write components
      float xa[K][VEC], bs[NB][VEC];
#pragma unroll
      for (int i = 0; i < K; ++i) E::unpack(st.x[i], xa[i]);
      E::unpack(st.o, bs[0]);
      if constexpr (WR == 4) {
        // the causal convolutions of out along the sequence (kernel sizes
        // 4, 8, 12; lag-i weights at conv_w row off_j + i), in the per-
        // sublayer write's order: lag 0 first, each branch accumulated from
        // zero.  Lag i of token r comes from lane r - i of this tile, or for
        // r < i from lane r + 16 - i of the 16 rows before; lags before the
        // token's sequence start are zero.
        const int spos = (STT * step + tau) % a.S;
        // whether any token of the wave's tile lies within 11 of its
        // sequence start (uniform over the wave; most tiles skip the masks)
        const bool near_start = __builtin_amdgcn_ballot_w64(spos < 11) != 0;
        const int cl = cb * KB + VEC * g;   // the lane's first channel within the slice
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          bs[1][e] = fmaf(s_cw[0][cl + e], bs[0][e], 0.f);
          bs[2][e] = fmaf(s_cw[4][cl + e], bs[0][e], 0.f);
          bs[3][e] = fmaf(s_cw[12][cl + e], bs[0][e], 0.f);
        }
        // lags 1 .. 11; with MASKED, those reaching before the token's
        // sequence start read zero
        auto lags = [&](auto masked) __attribute__((always_inline)) {
          for_each_c<11>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value + 1;   // lag
            u32x4_t lg;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              // row_shl (16 - i): lane r < i takes lane r + 16 - i of the rows
              // before; row_shr i: lane r >= i takes lane r - i of this tile
              const int pv = __builtin_amdgcn_update_dpp(0, (int)st.op[d], 0x100 + (16 - i), 0xf, 0xf, false);
              lg[d] = (uint32_t)__builtin_amdgcn_update_dpp(pv, (int)st.o[d], 0x110 + i, 0xf, 0xf, false);
            }
            if constexpr (decltype(masked)::value) lg = i <= spos ? lg : zero;
            float h[VEC];
            E::unpack(lg, h);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
              if constexpr (i < 4) bs[1][e] = fmaf(s_cw[i][cl + e], h[e], bs[1][e]);
              if constexpr (i < 8) bs[2][e] = fmaf(s_cw[4 + i][cl + e], h[e], bs[2][e]);
              bs[3][e] = fmaf(s_cw[12 + i][cl + e], h[e], bs[3][e]);
            }
          });
        };
        // Two copies under a branch that is uniform over the wave: left to
        // itself the compiler turns the mask into selects on every lag of
        // every tile (~55 vector instructions per step) though most tiles
        // lie clear of a sequence start.
        if constexpr (XHC_POST_NS_SPLIT) {
          if (near_start) lags(std::true_type{});
          else lags(std::false_type{});
        } else {
          lags(std::true_type{});
        }
      }
      const __amdgpu_buffer_rsrc_t rx = x_rsrc(step);
#pragma unroll
      for (int j = 0; j < K; ++j) {
        float q[NB];
        if constexpr (WR == 1) {
          q[0] = s_cf[cbuf][STT * K * K + tau * K + j] * s_cf[cbuf][STT * K * K + STT * K + tau * K + j];
        } else {
#pragma unroll
          for (int v = 0; v < NB; ++v) q[v] = s_cf[cbuf][STT * K * K + (tau * K + j) * NB + v];
        }
        float nv[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          float sum = 0.f;
#pragma unroll
          for (int i = 0; i < K; ++i) sum = fmaf(s_cf[cbuf][(tau * K + j) * K + i], xa[i][e], sum);
#pragma unroll
          for (int v = 0; v < NB; ++v) sum = fmaf(q[v], bs[v][e], sum);
          nv[e] = sum;
        }
        xn[j] = E::packv_cvt(nv);
        st_b128<ROW_ST_AUX>(xn[j], rx, (uint32_t)(((size_t)tau * N + I[j]) * C * sizeof(T)) + cofs);
      }
    } else {
#pragma unroll
      for (int j = 0; j < K; ++j) xn[j] = st.x[j];
    }
    // sums of x and x^2 over the new rows, and the next layer's projection
    f32x4_t S1 = f32x4_t{0.f, 0.f, 0.f, 0.f}, S2 = S1, acc[NTF];
#pragma unroll
    for (int n = 0; n < NTF; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < K; ++j) mma_sums<E>(xn[j], ones, S1, S2);
    // every stream of the next layer: the fixed ones hold rewritten rows too
    u32x4_t bw[2][NTF];
#pragma unroll
    for (int n = 0; n < NTF; ++n) bw[0][n] = s_w[cb][0][n][lane];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (i + 1 < N) {
#pragma unroll
        for (int n = 0; n < NTF; ++n) bw[(i + 1) & 1][n] = s_w[cb][i + 1][n][lane];
      }
      // the new row that sits in stream i, if any: with m known, stream
      // i < m holds fixed position i and only routed positions can hold a
      // stream i >= m
      u32x4_t v = zero;
      if constexpr (MS >= 0) {
        if (i < MS) {
          v = xn[i < K ? i : 0];
        } else {
#pragma unroll
          for (int j = MS; j < K; ++j) v = (I[j] == i) ? xn[j] : v;
        }
      } else {
#pragma unroll
        for (int j = 0; j < K; ++j) v = (I[j] == i) ? xn[j] : v;
      }
#pragma unroll
      for (int n = 0; n < NTF; ++n) acc[n] = E::mma(acc[n], v, bw[i & 1][n]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (WR == 4) {
      // two rounds: blocks 2 and 3 of each tile store, blocks 0 and 1 add
      if (cb >= 2) {
        const int w2 = b * 2 + cb - 2;
#pragma unroll
        for (int n = 0; n < NTF; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) s_red[w2][(4 * g + i) * NPF + n * 16 + r] = acc[n][i];
        sums_to_lds(&s_red[w2][TM * NPF], g, r, S1, S2);
      }
      __syncthreads();
      if (cb < 2) {
        const int w2 = b * 2 + cb;
#pragma unroll
        for (int n = 0; n < NTF; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) s_red[w2][(4 * g + i) * NPF + n * 16 + r] += acc[n][i];
        if (r == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) s_red[w2][TM * NPF + 2 * (4 * g + i)] += S1[i];
        }
        if ((r >> 2) == g) s_red[w2][TM * NPF + 2 * r + 1] += diag_of(S2, r);
      }
    } else {
      acc_to_lds<NTF, NPF>(s_red, wave, g, r, acc);
      sums_to_lds(&s_red[wave][TM * NPF], g, r, S1, S2);
    }
    __syncthreads();
    // partial sums of the step's tiles; entries past the step or past the
    // last tile go out of the store's range
    constexpr int IT = (PTL * NSUM + PNTHR - 1) / PNTHR;
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int u0 = tid + k * PNTHR;
      const bool in = u0 < PTL * NSUM;
      const int u = in ? u0 : 0;
      const int bb = u / NSUM, v = u % NSUM;
      const int tile = PTL * step + bb;
      float x;
      if constexpr (WR == 4) {
        x = s_red[bb * 2][v] + s_red[bb * 2 + 1][v];
      } else {
        x = 0.f;
#pragma unroll
        for (int c = 0; c < PSB; ++c) x += s_red[bb * PSB + c][v];
      }
      st_b32(x, rcorr, in && tile < a.ntiles ? (uint32_t)((((size_t)tile * G + slice) * P1 + v) * 4) : OUT_OF_RANGE);
    }
  };

  // steps team + k nteams; ring slots by k.  NR steps per trip and the only
  // exit at its end (a step past the last one loads and stores nothing): an
  // exit between steps would be merged by the compiler into a path back to
  // the loop head, whose memory-counter waits would then drain the loads
  // issued PD steps ahead.
  if (team >= nsteps) return;
  for (int k0 = 0; team + k0 * nteams < nsteps; k0 += NR) {
    for_each_c<NR>([&](auto qc) __attribute__((always_inline)) {
      constexpr int q = decltype(qc)::value;
      const int k = k0 + q;
      const int step = team + k * nteams;
      // rows of later steps: the list PD + 1 steps ahead, the coefficients
      // of the next step
      const u32x4_t nv = load_unit(step + (PD + 1) * nteams, true, false);
      const u32x4_t nc = WR ? load_unit(step + nteams, false, true) : zero;
      issue(sr[(q + PD) % NR], step + PD * nteams, (k + PD) % NI);
      __builtin_amdgcn_sched_barrier(0);
      compute(sr[q], step, k % NI, k & 1);
      store_unit(nv, (k + PD + 1) % NI, 0, true, false);
      if constexpr (WR != 0) store_unit(nc, 0, (k + 1) & 1, false, true);
      __syncthreads();
    });
  }
}

// ---------------------------------------------------------------------------
// Persistent post pass with the rows staged through LDS (bf16, m known, C a
// multiple of the 128-channel slice): the write (WR = 1 attention-type, 4
// MLP-type) and its share of the next layer's routing, with the arithmetic
// of the register-staged pass above, in its order.
//
// A workgroup of SSB = 4 waves owns one slice and walks steps of two 16-token
// tiles; wave w takes contraction block w of both tiles.  A step's k active
// rows and its rows of out (MLP-type: also the 16 rows of out before the
// step, whose last ones the first tile's lags reach) come from HBM by
// buffer-to-LDS loads of 4 token rows x 256 B into one slot of a two-step
// ring; as in the staged pre pass a step reads its slot into registers
// first, and the slot then takes the loads of the step two on (whose
// addresses need that step's active lists: the lists are in LDS three steps
// ahead).  The new rows go to LDS in the fragment layout, and the next step
// reads them back row by row and stores them, 4 rows x 256 B per store.  The
// next layer's routing fragments of the wave's block (every stream) stay in
// registers, one wave per SIMD.
// ---------------------------------------------------------------------------
#ifndef XHC_POST_STAGED
#define XHC_POST_STAGED 1
#endif
#ifndef XHC_POST_STAGED_M
#define XHC_POST_STAGED_M 0   // MLP-type too (correct, but 492 -> 576 us per call: its convolutions at one wave per
                              // SIMD are slower than the register-staged pass at two)
#endif
#ifndef XHC_POST_STAGE_AUX
#define XHC_POST_STAGE_AUX 2   // streaming loads (measured: 318 -> 314 us per attention-type call)
#endif
#ifndef XHC_POST_ROW_ST_AUX
#define XHC_POST_ROW_ST_AUX 2  // streaming row stores: whole lines here; with the default policy the dirty lines
                               // are written back during the next pre pass (measured: that pass 488 -> 478 us)
#endif
template <class E, int N, int K, int MS, int WR>
__global__ __launch_bounds__(SNTHR, 1) void xhc_post_s_kernel(PostPArgs a) {
  static_assert(std::is_same<E, Bf16>::value, "the staged post pass is written for bf16 state");
  static_assert(MS > 0 && MS <= K && MS < N, "the fixed streams are known");
  static_assert(WR == 1 || WR == 4, "write kinds: attention-type, MLP-type");
  using T = typename E::T;
  using D = RouteDims<N>;
  constexpr int NTF = D::NTF, NPF = D::NPF, NSUM = D::NSUM, P1 = D::P1;
  constexpr int KB = E::KB, VEC = E::VEC;
  constexpr int STT = 2 * TM;                   // tokens per step
  constexpr int SQ = STT / 4;                   // token quads per step
  constexpr int NKD = K + 1;                    // ring kinds: the k active positions, then out
  constexpr int NBQ = WR == 4 ? TM / 4 : 0;     // quads of the 16 rows of out before the step
  constexpr int NDMA = NKD * SQ + NBQ;
  static_assert(NDMA % SSB == 0 && (K * SQ) % SSB == 0, "a step's loads and stores split evenly over the waves");
  constexpr int LPW = NDMA / SSB;               // buffer-to-LDS loads per wave and step
  constexpr int NST = K * SQ / SSB;             // row stores per wave and step
  constexpr int SLC = SSB * KB;                 // channels of a slice
  // per-step coefficients: H_res [STT][K][K], then p [STT][K] and H_post
  // [STT][K] (attention-type) or Q = diag(p) H_post Tm [STT][K][4] (MLP-type)
  constexpr int E2 = WR == 4 ? 4 * K : K, E3 = WR == 4 ? 0 : K;
  constexpr int CF = STT * (K * K + E2 + E3);
  constexpr int NCL = WR == 4 ? 2 : 3;          // coefficient loads per thread
  constexpr int NL = 4;                         // ring of active lists
  static_assert(STT * K * K / 4 <= SNTHR && STT * E2 / 4 <= SNTHR, "a step's coefficient arrays take one unit per thread");
  static_assert(SSB * KB * 2 == 256, "a load covers 4 rows x 256 B");
  __shared__ u32x4_t s_y0[NKD][SQ][WAVE];       // ring of two steps: [kind][token quad][16-byte slot]
  __shared__ u32x4_t s_y1[NKD][SQ][WAVE];
  __shared__ u32x4_t s_b0[WR == 4 ? NBQ : 1][WAVE];   // MLP-type: the 16 rows of out before the step
  __shared__ u32x4_t s_b1[WR == 4 ? NBQ : 1][WAVE];
  __shared__ u32x4_t s_n[K][SQ][WAVE];          // the step's new rows, in the ring's layout
  __shared__ float s_red[SSB][2][NSUM];
  __shared__ int s_idx[NL][STT * K];
  __shared__ float s_cf[2][CF];
  __shared__ float s_cw[WR == 4 ? 24 : 1][WR == 4 ? SLC : 1];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int C = a.C, G = a.G, nkbC = C / KB;
  const int slice = blockIdx.x % G, team = blockIdx.x / G, nteams = gridDim.x / G;
  const int nsteps = (a.ntiles + 1) / 2;
  const int kb0 = slice * SSB + wave;
  const int full = a.T / STT, tail = a.T % STT;
  const uint32_t rowstride = (uint32_t)((size_t)N * C * sizeof(T));
  const uint32_t orow = (uint32_t)((size_t)C * sizeof(T));
  T* X = reinterpret_cast<T*>(a.X);
  const T* out = reinterpret_cast<const T*>(a.out);
  auto srows = [&](int step) { return step < full ? STT : (step == full ? tail : 0); };
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;

  int p = team;
  if (p >= nsteps) return;

  // ---- next layer's routing fragments of this block, every stream; the
  // slice's conv weights (MLP-type)
  const __amdgpu_buffer_rsrc_t rwn = make_rsrc(a.wnext, (uint32_t)((size_t)N * nkbC * NTF * WAVE * 16));
  u32x4_t wn[N][NTF];
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int n = 0; n < NTF; ++n)
      wn[i][n] = ld_b128(rwn, (uint32_t)lane * 16, (uint32_t)((((size_t)i * nkbC + kb0) * NTF + n) * WAVE * 16));
  if constexpr (WR == 4) {
    // all loads first, then the stores: one memory round trip
    static_assert((24 * SLC) % SNTHR == 0, "the conv weights of a slice split evenly over the threads");
    constexpr int NW = 24 * SLC / SNTHR;
    float cw[NW];
#pragma unroll
    for (int it = 0; it < NW; ++it) {
      const int u = tid + it * SNTHR, tap = u / SLC, c = slice * SLC + u % SLC;
      cw[it] = a.conv_w[(size_t)tap * C + c];
    }
#pragma unroll
    for (int it = 0; it < NW; ++it) {
      const int u = tid + it * SNTHR;
      s_cw[u / SLC][u % SLC] = cw[it];
    }
  }

  // ---- a step's lists and coefficients, one 16-byte unit per thread (units
  // past the array or the step's valid tokens read zero)
  const float* arr2 = WR == 4 ? a.wq : a.p;
  auto load_lists = [&](int step) __attribute__((always_inline)) {
    const int rows = srows(step);
    const size_t t0 = rows > 0 ? (size_t)STT * step : 0;
    return ld_b128(make_rsrc(a.idx + t0 * K, (uint32_t)(rows * K * 4)), (uint32_t)tid * 16, 0);
  };
  struct Coefs { u32x4_t h, c2, c3; };
  auto load_coefs = [&](int step) __attribute__((always_inline)) {
    const int rows = srows(step);
    const size_t t0 = rows > 0 ? (size_t)STT * step : 0;
    Coefs c;
    c.h = ld_b128(make_rsrc(a.h_res + t0 * K * K, (uint32_t)(rows * K * K * 4)), (uint32_t)tid * 16, 0);
    c.c2 = ld_b128(make_rsrc(arr2 + t0 * E2, (uint32_t)(rows * E2 * 4)), (uint32_t)tid * 16, 0);
    if constexpr (E3 > 0) c.c3 = ld_b128(make_rsrc(a.h_post + t0 * E3, (uint32_t)(rows * E3 * 4)), (uint32_t)tid * 16, 0);
    return c;
  };
  auto store_lists = [&](int slot, const u32x4_t& v) __attribute__((always_inline)) {
    if (tid < STT * K / 4) reinterpret_cast<u32x4_t*>(&s_idx[slot][0])[tid] = v;
  };
  auto store_coefs = [&](int buf, const Coefs& c) __attribute__((always_inline)) {
    if (tid < STT * K * K / 4) reinterpret_cast<u32x4_t*>(&s_cf[buf][0])[tid] = c.h;
    if (tid < STT * E2 / 4) reinterpret_cast<u32x4_t*>(&s_cf[buf][STT * K * K])[tid] = c.c2;
    if constexpr (E3 > 0)
      if (tid < STT * E3 / 4) reinterpret_cast<u32x4_t*>(&s_cf[buf][STT * K * K + STT * E2])[tid] = c.c3;
  };

  // ---- a step's rows into a ring slot.  Load v of the step: kinds 0..K-1
  // the active positions, K out (quads 0..SQ-1 each), then (MLP-type) the
  // NBQ quads of the rows before; lane l takes row (token 4 quad + l / 16),
  // chunk (l mod 16) xor (token mod 16).  A position's stream comes from the
  // step's list in LDS, read before the loads go out.
  const int lrow = lane >> 4, lslot = lane & 15;
  auto dma_streams = [&](int lslotidx, int (&ist)[LPW]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int v = wave * LPW + u;
      const int j = v / SQ, tok = 4 * (v % SQ) + lrow;
      const int iv = s_idx[lslotidx][tok * K + (j < K ? j : 0)];
      ist[u] = iv < 0 ? 0 : (iv >= N ? N - 1 : iv);
    }
  };
  auto dma = [&](int step, auto qc, const int (&ist)[LPW]) __attribute__((always_inline)) {
    const int rows = srows(step);
    const size_t t0 = rows > 0 ? (size_t)STT * step : 0;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X + t0 * N * C, (uint32_t)((size_t)rows * rowstride));
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(out + t0 * C, (uint32_t)((size_t)rows * orow));
    const bool back = rows > 0 && t0 >= (size_t)TM;
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(out + (back ? t0 - TM : 0) * C, back ? (uint32_t)(TM * orow) : 0u);
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
      const int v = wave * LPW + u;            // uniform over the wave
      const bool isx = v < K * SQ, isb = v >= NKD * SQ;
      const int j = isb ? K : v / SQ, bq = isb ? v - NKD * SQ : v % SQ;
      const int tok = 4 * bq + lrow;
      const uint32_t off = (uint32_t)tok * (isx ? rowstride : orow) + (isx ? (uint32_t)ist[u] * orow : 0u) +
                           (uint32_t)(slice * 256 + ((lslot ^ (tok & 15)) << 4));
      u32x4_t* dst;
      if constexpr (decltype(qc)::value == 0) dst = isb ? &s_b0[bq][0] : &s_y0[j][bq][0];
      else dst = isb ? &s_b1[bq][0] : &s_y1[j][bq][0];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isx ? rx : (isb ? rb : ro), (lds_ptr_t)dst, 16, (int)off, 0, 0,
                                               XHC_POST_STAGE_AUX);
    }
  };

  // ---- prologue: the first three steps' lists, the first step's
  // coefficients, then the rows of the first two steps
  {
    const u32x4_t l0 = load_lists(p), l1 = load_lists(p + nteams), l2 = load_lists(p + 2 * nteams);
    const Coefs c0 = load_coefs(p);
    wait_vmcnt<0>();
    store_lists(0, l0);
    store_lists(1, l1);
    store_lists(2, l2);
    store_coefs(0, c0);
  }
  __syncthreads();
  {
    int ist[LPW];
    dma_streams(0, ist);
    dma(p, Q0{}, ist);
    dma_streams(1, ist);
    dma(p + nteams, Q1{}, ist);
  }
  stage_barrier<LPW>();

  const __amdgpu_buffer_rsrc_t rcorr = make_rsrc(a.corr, (uint32_t)((size_t)a.ntiles * G * P1 * 4));
  const uint32_t fofs0 = staged_frag(wave, g, r);   // tile 0's fragment within a kind; tile 1 is 4 quads on
  constexpr uint32_t KBYTES = SQ * WAVE * 16;       // bytes of one kind of a step
  constexpr uint32_t TBYTES = 4 * WAVE * 16;        // bytes of one tile of a kind
  const u32x4_t zero = u32x4_t{0u, 0u, 0u, 0u};
  const u32x4_t ones = ones_frag<E>();
  const int cl = wave * KB + VEC * g;               // the lane's first channel within the slice
  constexpr int IT = (2 * NSUM + SNTHR - 1) / SNTHR;
  // vector memory operations of one step, every one issued unconditionally:
  // row stores, partial stores, the lists, the coefficients, the tile loads
  constexpr int VM_STEP = NST + IT + 1 + NCL + LPW;

  // the new rows of step `st` (in s_n) to their rows of X, and its partials
  auto store_step = [&](int st, int lslotidx) __attribute__((always_inline)) {
    u32x4_t stv[NST];
    int sti[NST];
#pragma unroll
    for (int u = 0; u < NST; ++u) {
      const int v = wave * NST + u, j = v / SQ, bq = v % SQ;
      stv[u] = s_n[j][bq][lane];
      const int iv = s_idx[lslotidx][(4 * bq + lrow) * K + j];
      sti[u] = iv < 0 ? 0 : (iv >= N ? N - 1 : iv);
    }
    float xs[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int u0 = tid + it * SNTHR;
      const int u = u0 < 2 * NSUM ? u0 : 0;
      const int bb = u / NSUM, vv = u % NSUM;
      float x = 0.f;
#pragma unroll
      for (int c = 0; c < SSB; ++c) x += s_red[c][bb][vv];
      xs[it] = x;
    }
    const int rows = st >= 0 ? srows(st) : 0;
    const size_t t0 = rows > 0 ? (size_t)STT * st : 0;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X + t0 * N * C, (uint32_t)((size_t)rows * rowstride));
#pragma unroll
    for (int u = 0; u < NST; ++u) {
      const int v = wave * NST + u, bq = v % SQ;
      const int tok = 4 * bq + lrow;
      st_b128<XHC_POST_ROW_ST_AUX>(stv[u], rx, (uint32_t)tok * rowstride + (uint32_t)sti[u] * orow +
                                                   (uint32_t)(slice * 256 + ((lslot ^ (tok & 15)) << 4)));
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int u0 = tid + it * SNTHR;
      const bool in = u0 < 2 * NSUM;
      const int u = in ? u0 : 0;
      const int bb = u / NSUM, vv = u % NSUM;
      const int tile = 2 * st + bb;
      st_b32(xs[it], rcorr, in && st >= 0 && tile < a.ntiles ? (uint32_t)((((size_t)tile * G + slice) * P1 + vv) * 4)
                                                            : OUT_OF_RANGE);
    }
  };

  int pprev = -1, k = 0;
  auto step_fn = [&](auto qc) __attribute__((always_inline)) {
    constexpr int q = decltype(qc)::value;
    const int p1 = p + nteams, p2 = p1 + nteams, p3 = p2 + nteams;
    const int lcur = k & 3, lnx2 = (k + 2) & 3, lprev = (k + 3) & 3;
    const char* yq = reinterpret_cast<const char*>(q == 0 ? &s_y0[0][0][0] : &s_y1[0][0][0]);
    // ---- reads: this step's lists and fragments; the active streams of the
    // step two on
    int I[2][K];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const int v = s_idx[lcur][(TM * tt + r) * K + j];
        I[tt][j] = v < 0 ? 0 : (v >= N ? N - 1 : v);
      }
    u32x4_t x[2][K], o[2], ob = zero;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint32_t f = fofs0 + (uint32_t)tt * TBYTES;
#pragma unroll
      for (int j = 0; j < K; ++j) x[tt][j] = *reinterpret_cast<const u32x4_t*>(yq + (uint32_t)j * KBYTES + f);
      o[tt] = *reinterpret_cast<const u32x4_t*>(yq + (uint32_t)K * KBYTES + f);
    }
    if constexpr (WR == 4)
      ob = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(q == 0 ? &s_b0[0][0] : &s_b1[0][0]) + fofs0);
    int ist[LPW];
    dma_streams(lnx2, ist);
    // ---- the previous step's rows and partials; then every wave is past
    // its reads of this slot
    store_step(pprev, lprev);
    stage_barrier<63>();
    // ---- lists three steps on, coefficients of the next step, then the
    // rows of the step two on into this slot (past the last step they read
    // nothing)
    const u32x4_t lnx = load_lists(p3);
    const Coefs cnx = load_coefs(p1);
    // (kept ahead of the tile loads, so that waiting for them does not wait
    // for the tile loads too)
    __builtin_amdgcn_sched_barrier(0);
    dma(p2, qc, ist);
    // ---- per tile: the write, its rows to LDS, the correction and its
    // partials to LDS
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tau = TM * tt + r;
      constexpr int NB = WR;   // write components
      float xa[K][VEC], bs[NB][VEC];
#pragma unroll
      for (int i = 0; i < K; ++i) E::unpack(x[tt][i], xa[i]);
      E::unpack(o[tt], bs[0]);
      if constexpr (WR == 4) {
        // the causal convolutions of out along the sequence (kernel sizes
        // 4, 8, 12; lag-i weights at conv_w row off_j + i) in the
        // per-sublayer write's order: lag i of token r from lane r - i of
        // this tile, or for r < i from lane r + 16 - i of the 16 rows before
        // (tile 0: the rows before the step; tile 1: tile 0); lags before
        // the token's sequence start are zero
        const u32x4_t opv = tt == 0 ? ob : o[0];
        const int spos = (STT * p + tau) % a.S;
        const bool near_start = __builtin_amdgcn_ballot_w64(spos < 11) != 0;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          bs[1][e] = fmaf(s_cw[0][cl + e], bs[0][e], 0.f);
          bs[2][e] = fmaf(s_cw[4][cl + e], bs[0][e], 0.f);
          bs[3][e] = fmaf(s_cw[12][cl + e], bs[0][e], 0.f);
        }
        for_each_c<11>([&](auto ic) __attribute__((always_inline)) {
          constexpr int i = decltype(ic)::value + 1;   // lag
          u32x4_t lg;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const int pv = __builtin_amdgcn_update_dpp(0, (int)opv[d], 0x100 + (16 - i), 0xf, 0xf, false);
            lg[d] = (uint32_t)__builtin_amdgcn_update_dpp(pv, (int)o[tt][d], 0x110 + i, 0xf, 0xf, false);
          }
          if (near_start) lg = i <= spos ? lg : zero;
          float h[VEC];
          E::unpack(lg, h);
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            if constexpr (i < 4) bs[1][e] = fmaf(s_cw[i][cl + e], h[e], bs[1][e]);
            if constexpr (i < 8) bs[2][e] = fmaf(s_cw[4 + i][cl + e], h[e], bs[2][e]);
            bs[3][e] = fmaf(s_cw[12 + i][cl + e], h[e], bs[3][e]);
          }
        });
      }
      u32x4_t xn[K];
#pragma unroll
      for (int j = 0; j < K; ++j) {
        float cq[NB];
        if constexpr (WR == 1) {
          cq[0] = s_cf[q][STT * K * K + tau * K + j] * s_cf[q][STT * K * K + STT * K + tau * K + j];
        } else {
#pragma unroll
          for (int v = 0; v < NB; ++v) cq[v] = s_cf[q][STT * K * K + (tau * K + j) * NB + v];
        }
        float hr[K];
#pragma unroll
        for (int i = 0; i < K; ++i) hr[i] = s_cf[q][(tau * K + j) * K + i];
        float nv[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          float sum = 0.f;
#pragma unroll
          for (int i = 0; i < K; ++i) sum = fmaf(hr[i], xa[i][e], sum);
#pragma unroll
          for (int v = 0; v < NB; ++v) sum = fmaf(cq[v], bs[v][e], sum);
          nv[e] = sum;
        }
        xn[j] = E::packv_cvt(nv);
        *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(&s_n[0][0][0]) + (uint32_t)j * KBYTES + fofs0 +
                                    (uint32_t)tt * TBYTES) = xn[j];
      }
      // sums of x and x^2 over the new rows, and the next layer's
      // projection: per stream, the new row that sits in it (zero if none)
      f32x4_t acc[NTF], S1 = f32x4_t{0.f, 0.f, 0.f, 0.f}, S2 = S1;
#pragma unroll
      for (int n = 0; n < NTF; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < K; ++j) mma_sums<E>(xn[j], ones, S1, S2);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        u32x4_t v = zero;
        if (i < MS) {
          v = xn[i < K ? i : 0];
        } else {
#pragma unroll
          for (int j = MS; j < K; ++j) v = (I[tt][j] == i) ? xn[j] : v;
        }
#pragma unroll
        for (int n = 0; n < NTF; ++n) acc[n] = E::mma(acc[n], v, wn[i][n]);
      }
#pragma unroll
      for (int n = 0; n < NTF; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_red[wave][tt][(4 * g + i) * NPF + n * 16 + r] = acc[n][i];
      sums_to_lds(&s_red[wave][tt][TM * NPF], g, r, S1, S2);
      // the second tile reads its weights and coefficients from LDS again
      // rather than keeping the first tile's in registers
      asm volatile("" ::: "memory");
    }
    // ---- the lists and coefficients to LDS; then this wave's loads of the
    // next step are complete (all but this step's operations), and after the
    // barrier every wave's are
    store_lists(lprev, lnx);
    store_coefs(q ^ 1, cnx);
    stage_barrier<VM_STEP>();
    pprev = p;
    p = p1;
    ++k;
  };
  // two steps per trip and the only exit at its end (a step past the last
  // loads and stores nothing)
  do {
    step_fn(Q0{});
    step_fn(Q1{});
  } while (p < nsteps);
  store_step(pprev, (k + 3) & 3);
  wait_vmcnt<0>();   // no load into LDS outlives the workgroup
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

#ifndef XHC_PRE_RB
#define XHC_PRE_RB 1
#endif
constexpr int PRE_RB = XHC_PRE_RB;   // 16-token row blocks per chained pre workgroup
#ifndef XHC_CORR_RB
#define XHC_CORR_RB 2
#endif
constexpr int CORR_RB = XHC_CORR_RB;   // 16-token row blocks per correction workgroup (best of 1, 2, 4)

// Workgroups of a persistent launch: one per compute unit (their LDS allows
// no more), Gp slices per team, no more teams than steps.
// The same for the staged pre pass: one 16-token tile per step.
int persist_grid_s(const Plan& P) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
  long teams = v / P.Gp;
  if (teams < 1) teams = 1;
  if (teams > P.ntiles) teams = P.ntiles;
  if (teams < 1) teams = 1;
  return (int)(teams * P.Gp);
}

int persist_grid(const Plan& P) {
  static int ncu[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (ncu[dev] <= 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    ncu[dev] = v;
  }
  const long nsteps = (P.ntiles + PTL - 1) / PTL;
  long teams = ncu[dev] / P.Gp;
  if (teams < 1) teams = 1;
  if (teams > nsteps) teams = nsteps;
  if (teams < 1) teams = 1;
  return (int)(teams * P.Gp);
}

template <class E, int N, int K, int KR>
void pre_chained_launch(const Plan& P, const xhc_weights* w, const Plan* Pn, const void* X, void* inp, char* ws,
                        char* wsn, hipStream_t st) {
  PreChainArgs a;
  a.X = X; a.inp = inp; a.T = (int)P.T; a.C = P.C; a.G = P.G; a.m = P.m; a.ntiles = (int)P.ntiles;
  a.wact = reinterpret_cast<const uint4*>(ws + P.o_wact);
  a.wnext = Pn ? reinterpret_cast<const uint4*>(wsn + Pn->o_wfull) : nullptr;
  a.idx = reinterpret_cast<const int*>(ws + P.o_idx);
  a.h_pre = reinterpret_cast<const float*>(ws + P.o_hpre);
  a.part2 = reinterpret_cast<float*>(ws + P.o_part2);
  a.look = Pn ? reinterpret_cast<float*>(wsn + Pn->o_part) : nullptr;
  constexpr int RB = PRE_RB;
  int Gpart;   // slices of the active partials
  if (Pn) {
    // persistent: routing weights of the next layer resident in LDS
    a.G = P.Gp;
    Gpart = P.Gp;
    if constexpr (XHC_PRE_STAGED && std::is_same<E, Bf16>::value && N == 16 && K > 2) {
      if (P.m == 2 && P.C % (SSB * Bf16::KB) == 0) {
        xhc_pre_chained_s_kernel<E, N, K, KR, 2><<<(unsigned)persist_grid_s(P), SNTHR, 0, st>>>(a);
        goto fin;
      }
    }
    if (P.m == 2 && K > 2)
      xhc_pre_chained_p_kernel<E, N, K, KR, 2><<<(unsigned)persist_grid(P), PNTHR, 0, st>>>(a);
    else
      xhc_pre_chained_p_kernel<E, N, K, KR, -1><<<(unsigned)persist_grid(P), PNTHR, 0, st>>>(a);
  } else {
    if constexpr (XHC_PRE_STAGED && std::is_same<E, Bf16>::value && N == 16 && K > 2) {
      if (P.m == 2 && P.C % (SSB * Bf16::KB) == 0) {
        // the last sublayer of a chain: the same staged pass without the
        // next layer's routing
        a.G = P.Gp;
        Gpart = P.Gp;
        xhc_pre_chained_s_kernel<E, N, K, KR, 2, false><<<(unsigned)persist_grid_s(P), SNTHR, 0, st>>>(a);
        goto fin;
      }
    }
    Gpart = P.G;
    const unsigned grid = (unsigned)(((P.T + TM * RB - 1) / (TM * RB)) * P.G);
    xhc_pre_chained_kernel<E, N, K, KR, false, RB><<<grid, NTHR, 0, st>>>(a);
  }

fin:
  ActFinArgs f;
  f.T = (int)P.T; f.C = P.C; f.G = Gpart; f.ntiles = (int)P.ntiles;
  f.part2 = a.part2;
  f.b_res = w->b_res; f.b_post = w->b_post;
  f.a_res = w->alpha_res; f.a_post = w->alpha_post; f.eps = P.eps_norm; f.iters = P.iters;
  f.h_res = reinterpret_cast<float*>(ws + P.o_hres);
  f.h_post = reinterpret_cast<float*>(ws + P.o_hpost);
  xhc_act_fin_kernel<K, KR><<<(unsigned)P.ntiles, ActDims<K, KR>::FT, 0, st>>>(f);
}

template <int N, int K>
void route_fin_launch(const Plan& P, const xhc_weights* w, char* ws, bool with_corr, int Gc, hipStream_t st) {
  RouteFinArgs f;
  // routing partials come from the persistent kernels, corrections (Gc
  // slices) from the correction kernel or the persistent post pass
  f.T = (int)P.T; f.C = P.C; f.m = P.m; f.G = P.Gp; f.Gc = Gc;
  f.part = reinterpret_cast<const float*>(ws + P.o_part);
  f.corr = with_corr ? reinterpret_cast<const float*>(ws + P.o_corr) : nullptr;
  f.b_pre = w->b_pre; f.a_pre = w->alpha_pre; f.eps = P.eps_norm;
  f.idx = reinterpret_cast<int*>(ws + P.o_idx);
  f.p = reinterpret_cast<float*>(ws + P.o_p);
  f.h_pre = reinterpret_cast<float*>(ws + P.o_hpre);
  f.z = reinterpret_cast<float*>(ws + P.o_z);
  f.gstat = reinterpret_cast<float*>(ws + P.o_gstat);
  xhc_route_fin_kernel<N, K><<<(unsigned)P.ntiles, RouteDims<N>::FT, 0, st>>>(f);
}

template <class E, int N, int K>
void route_launch(const Plan& P, const xhc_weights* w, const void* X, char* ws, hipStream_t st) {
  ProjPArgs a;
  a.X = X; a.T = (int)P.T; a.C = P.C; a.G = P.Gp; a.ntiles = (int)P.ntiles;
  a.wfull = reinterpret_cast<const uint4*>(ws + P.o_wfull);
  a.part = reinterpret_cast<float*>(ws + P.o_part);
  if constexpr (XHC_PRE_STAGED && std::is_same<E, Bf16>::value && N == 16) {
    if (P.C % (SSB * Bf16::KB) == 0) {
      xhc_proj_s_kernel<E, N><<<(unsigned)persist_grid_s(P), SNTHR, 0, st>>>(a);
      route_fin_launch<N, K>(P, w, ws, false, 0, st);
      return;
    }
  }
  xhc_proj_p_kernel<E, N><<<(unsigned)persist_grid(P), PNTHR, 0, st>>>(a);
  route_fin_launch<N, K>(P, w, ws, false, 0, st);
}

#ifndef XHC_POST_FUSE
#define XHC_POST_FUSE 1
#endif
#ifndef XHC_CORR_P
#define XHC_CORR_P 1
#endif

// The rewritten rows' share of the next layer's routing, then that layer's
// routing.  fuse: the write of this layer is done here too (for the MLP
// type after the Gram pass and the per-token write coefficients).
template <class E, int N, int K>
void tail_launch(const Plan& P, const Plan& Pn, const xhc_weights* w, const xhc_weights* wn, void* X,
                 const void* out, char* ws, char* wsn, bool fuse, hipStream_t st) {
  if (fuse || XHC_CORR_P) {
    PostPArgs a;
    a.X = X; a.out = out; a.T = (int)P.T; a.S = P.S; a.C = P.C; a.G = P.Gp; a.ntiles = (int)P.ntiles;
    a.idx = reinterpret_cast<const int*>(ws + P.o_idx);
    a.h_res = reinterpret_cast<const float*>(ws + P.o_hres);
    a.p = reinterpret_cast<const float*>(ws + P.o_p);
    a.h_post = reinterpret_cast<const float*>(ws + P.o_hpost);
    a.wq = reinterpret_cast<const float*>(ws + P.o_wcoef);
    a.conv_w = w ? w->conv_w : nullptr;
    a.wnext = reinterpret_cast<const uint4*>(wsn + Pn.o_wfull);
    a.corr = reinterpret_cast<float*>(wsn + Pn.o_corr);
    const unsigned grid = (unsigned)persist_grid(P);
    const bool m2 = P.m == 2 && K > 2;
    if (fuse && P.KR == 4) {
      launch_xhc_wcoef(P, out, w, ws, st);
      if constexpr (XHC_POST_STAGED_M && std::is_same<E, Bf16>::value && N == 16 && K > 2) {
        if (m2 && P.C % (SSB * Bf16::KB) == 0) {
          xhc_post_s_kernel<E, N, K, 2, 4><<<(unsigned)persist_grid_s(P), SNTHR, 0, st>>>(a);
          route_fin_launch<N, K>(Pn, wn, wsn, true, P.Gp, st);
          return;
        }
      }
      if (m2) xhc_post_p_kernel<E, N, K, 2, 4><<<grid, PNTHR, 0, st>>>(a);
      else xhc_post_p_kernel<E, N, K, -1, 4><<<grid, PNTHR, 0, st>>>(a);
    } else if (fuse) {
      if constexpr (XHC_POST_STAGED && std::is_same<E, Bf16>::value && N == 16 && K > 2) {
        if (m2 && P.C % (SSB * Bf16::KB) == 0) {
          xhc_post_s_kernel<E, N, K, 2, 1><<<(unsigned)persist_grid_s(P), SNTHR, 0, st>>>(a);
          route_fin_launch<N, K>(Pn, wn, wsn, true, P.Gp, st);
          return;
        }
      }
      if (m2) xhc_post_p_kernel<E, N, K, 2, 1><<<grid, PNTHR, 0, st>>>(a);
      else xhc_post_p_kernel<E, N, K, -1, 1><<<grid, PNTHR, 0, st>>>(a);
    } else {
      if (m2) xhc_post_p_kernel<E, N, K, 2, 0><<<grid, PNTHR, 0, st>>>(a);
      else xhc_post_p_kernel<E, N, K, -1, 0><<<grid, PNTHR, 0, st>>>(a);
    }
    route_fin_launch<N, K>(Pn, wn, wsn, true, P.Gp, st);
    return;
  }
  CorrArgs a;
  a.X = X; a.T = (int)P.T; a.C = P.C; a.G = P.G; a.ntiles = (int)P.ntiles; a.m = P.m;
  a.idx = reinterpret_cast<const int*>(ws + P.o_idx);
  a.wnext = reinterpret_cast<const uint4*>(wsn + Pn.o_wfull);
  a.corr = reinterpret_cast<float*>(wsn + Pn.o_corr);
  const long nblk = (P.T + TM * CORR_RB - 1) / (TM * CORR_RB);
  if (P.m == 2 && K >= 2)
    xhc_corr_kernel<E, N, K, CORR_RB, 2><<<(unsigned)(nblk * P.G), NTHR, 0, st>>>(a);
  else
    xhc_corr_kernel<E, N, K, CORR_RB, -1><<<(unsigned)(nblk * P.G), NTHR, 0, st>>>(a);
  route_fin_launch<N, K>(Pn, wn, wsn, true, P.G, st);
}

// Dispatch over the built (N, K) shapes; KR only matters for the active maps.
template <class F>
bool dispatch_shape(int N, int K, F&& f) {
  const int key = N * 100 + K;
  switch (key) {
    case 1604: f(std::integral_constant<int, 16>{}, std::integral_constant<int, 4>{}); return true;
    case 1602: f(std::integral_constant<int, 16>{}, std::integral_constant<int, 2>{}); return true;
    case 804: f(std::integral_constant<int, 8>{}, std::integral_constant<int, 4>{}); return true;
    case 404: f(std::integral_constant<int, 4>{}, std::integral_constant<int, 4>{}); return true;
    case 101: f(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{}); return true;
    default: return false;
  }
}

template <class E>
bool route_dispatch(const Plan& P, const xhc_weights* w, const void* X, char* ws, hipStream_t st) {
  return dispatch_shape(P.N, P.K, [&](auto n, auto k) { route_launch<E, decltype(n)::value, decltype(k)::value>(P, w, X, ws, st); });
}

template <class E>
bool pre_chained_dispatch(const Plan& P, const xhc_weights* w, const Plan* Pn, const void* X, void* inp, char* ws,
                          char* wsn, hipStream_t st) {
  return dispatch_shape(P.N, P.K, [&](auto n, auto k) {
    constexpr int NN = decltype(n)::value, KK = decltype(k)::value;
    if (P.KR == 4)
      pre_chained_launch<E, NN, KK, 4>(P, w, Pn, X, inp, ws, wsn, st);
    else
      pre_chained_launch<E, NN, KK, 1>(P, w, Pn, X, inp, ws, wsn, st);
  });
}

template <class E>
bool tail_dispatch(const Plan& P, const Plan& Pn, const xhc_weights* w, const xhc_weights* wn, void* X,
                   const void* out, char* ws, char* wsn, bool fuse, hipStream_t st) {
  return dispatch_shape(P.N, P.K, [&](auto n, auto k) {
    tail_launch<E, decltype(n)::value, decltype(k)::value>(P, Pn, w, wn, X, out, ws, wsn, fuse, st);
  });
}

}  // namespace

bool launch_xhc_route(const Plan& P, const void* X, const xhc_weights* w, char* ws, hipStream_t st) {
  if (!launch_pack(&P, w, ws, nullptr, nullptr, nullptr, &P, ws, st)) return false;
  return P.dtype == XHC_BF16 ? route_dispatch<Bf16>(P, w, X, ws, st) : route_dispatch<F32>(P, w, X, ws, st);
}

bool launch_xhc_pre_chained(const Plan& P, const xhc_weights* w, const Plan* Pn, const xhc_weights* wn,
                            const void* X, void* inp, char* ws, char* wsn, hipStream_t st) {
  if (!launch_pack(Pn, wn, wsn, &P, w, ws, &P, ws, st)) return false;
  return P.dtype == XHC_BF16 ? pre_chained_dispatch<Bf16>(P, w, Pn, X, inp, ws, wsn, st)
                             : pre_chained_dispatch<F32>(P, w, Pn, X, inp, ws, wsn, st);
}

// xHC-Flash readouts at N = 16 from the staged pass: NPRE outputs (4 with
// the active streams left out of readouts 1.., else 2).
bool launch_flash_read_s(const Plan& P, const void* X, void* const* out, const float* const* h_pre, const int* idx,
                         int npre, hipStream_t st) {
  if (!flash_read_s_applies(P) || (npre != 2 && npre != 4)) return false;
  FlashReadSArgs a;
  a.X = X; a.idx = idx; a.T = (int)P.T; a.C = P.C; a.G = P.Gp; a.K = P.K; a.ntiles = (int)P.ntiles;
  for (int q = 0; q < 4; ++q) {
    a.out[q] = q < npre ? out[q] : nullptr;
    a.h_pre[q] = q < npre ? h_pre[q] : nullptr;
  }
  if (npre == 2) flash_read_s_kernel<2, false><<<(unsigned)persist_grid_s(P), SNTHR, 0, st>>>(a);
  else flash_read_s_kernel<4, true><<<(unsigned)persist_grid_s(P), SNTHR, 0, st>>>(a);
  return true;
}

bool flash4_route_p_applies(const Plan& P) {
  return XHC_PRE_STAGED && P.N == 16 && P.K == 4 && P.dtype == XHC_BF16 && P.C % (SSB * Bf16::KB) == 0 &&
         P.ntiles > 0;
}

// xHC-Flash-4sub routing at N = 16: the staged persistent projection (packed
// weights of five tiles at wp, partials at part, Gp slices), then the routing
// of every tile.
bool launch_flash4_route_p(const Plan& P, const void* X, const void* wp, float* part, const Flash4Route& o,
                           hipStream_t st) {
  if (!flash4_route_p_applies(P)) return false;
  ProjPArgs a;
  a.X = X; a.T = (int)P.T; a.C = P.C; a.G = P.Gp; a.ntiles = (int)P.ntiles;
  a.wfull = reinterpret_cast<const uint4*>(wp);
  a.part = part;
  xhc_proj_s_kernel<Bf16, 16, Flash4Dims16><<<(unsigned)persist_grid_s(P), SNTHR, 0, st>>>(a);
  Flash4RouteFinArgs f;
  f.T = (int)P.T; f.C = P.C; f.m = P.m; f.G = P.Gp; f.part = part; f.eps = P.eps_norm; f.o = o;
  xhcf4_route_fin_kernel<4><<<(unsigned)P.ntiles, 256, 0, st>>>(f);
  return true;
}

// xHC-Flash routing at N = 16: the persistent projection (packed weights of
// three tiles at wp, partials at part, Gp slices) and the routing of every tile.
bool launch_flash_route_p(const Plan& P, const void* X, const void* wp, float* part, const xhcf_weights* w, int* idx,
                          float* p, float* h_pa, float* h_pm, float* z, hipStream_t st) {
  if (P.N != 16 || P.ntiles == 0) return false;
  ProjPArgs a;
  a.X = X; a.T = (int)P.T; a.C = P.C; a.G = P.Gp; a.ntiles = (int)P.ntiles;
  a.wfull = reinterpret_cast<const uint4*>(wp);
  a.part = part;
  if (P.dtype == XHC_BF16) {
    if (XHC_PRE_STAGED && P.C % (SSB * Bf16::KB) == 0)
      xhc_proj_s_kernel<Bf16, 16, FlashDims16><<<(unsigned)persist_grid_s(P), SNTHR, 0, st>>>(a);
    else
      xhcf_proj_p_kernel<Bf16><<<(unsigned)persist_grid(P), PNTHR, 0, st>>>(a);
  } else {
    xhcf_proj_p_kernel<F32><<<(unsigned)persist_grid(P), PNTHR, 0, st>>>(a);
  }
  FlashRouteFinArgs f;
  f.T = (int)P.T; f.C = P.C; f.m = P.m; f.G = P.Gp; f.part = part;
  f.b_pa = w->b_pre_attn; f.b_pm = w->b_pre_mlp; f.a_pa = w->alpha_pre_attn; f.a_pm = w->alpha_pre_mlp;
  f.eps = P.eps_norm;
  f.idx = idx; f.p = p; f.h_pa = h_pa; f.h_pm = h_pm; f.z = z;
  switch (P.K) {
    case 4: xhcf_route_fin_kernel<4><<<(unsigned)P.ntiles, 256, 0, st>>>(f); return true;
    default: return false;
  }
}

bool chain_post_fused(const Plan& P) { return XHC_POST_FUSE && !P.mhc && !P.flash && (P.KR == 1 || P.KR == 4); }

bool launch_xhc_chain_tail(const Plan& P, const Plan& Pn, const xhc_weights* w, const xhc_weights* wn, void* X,
                           const void* out, char* ws, char* wsn, bool fuse, hipStream_t st) {
  if (fuse && !chain_post_fused(P)) return false;
  return P.dtype == XHC_BF16 ? tail_dispatch<Bf16>(P, Pn, w, wn, X, out, ws, wsn, fuse, st)
                             : tail_dispatch<F32>(P, Pn, w, wn, X, out, ws, wsn, fuse, st);
}

// Active maps from active-projection partials laid out [ntiles][G][P2] of
// ActDims<K, KR> (used by the xHC-Flash MLP side).
bool launch_act_fin(const Plan& P, int G, const float* part2, const float* b_res, const float* b_post, float a_res,
                    float a_post, float* h_res, float* h_post, hipStream_t st) {
  ActFinArgs f;
  f.T = (int)P.T; f.C = P.C; f.G = G; f.ntiles = (int)P.ntiles;
  f.part2 = part2;
  f.b_res = b_res; f.b_post = b_post;
  f.a_res = a_res; f.a_post = a_post; f.eps = P.eps_norm; f.iters = P.iters;
  f.h_res = h_res; f.h_post = h_post;
  const unsigned grid = (unsigned)P.ntiles;
  switch (P.K * 10 + P.KR) {
    case 44: xhc_act_fin_kernel<4, 4><<<grid, ActDims<4, 4>::FT, 0, st>>>(f); return true;
    case 41: xhc_act_fin_kernel<4, 1><<<grid, ActDims<4, 1>::FT, 0, st>>>(f); return true;
    case 14: xhc_act_fin_kernel<1, 4><<<grid, ActDims<1, 4>::FT, 0, st>>>(f); return true;
    case 11: xhc_act_fin_kernel<1, 1><<<grid, ActDims<1, 1>::FT, 0, st>>>(f); return true;
    default: return false;
  }
}

}  // namespace xhc
