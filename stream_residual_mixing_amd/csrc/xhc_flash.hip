// xHC-Flash block (gfx950): one routing decision and two pre-maps shared by
// an attention + MLP pair of sublayers (xHC paper "xHC: Expanded
// Hyper-Connections", section "xHC-Flash", Eqs. 17-19, and paragraph
// "xHC-Flash kernel fusion").
//
//   xhcf_pre   pack    the three weight matrices into MFMA B fragments
//              colsum  column sums of the router weights (LayerNorm correction)
//              proj    one split-K projection pass over X: [W_r | W_pre^A |
//                      W_pre^M] and the sums of x and x^2 per token
//              route   router logits, both pre-maps, top-k, router weights
//              read    one pass over X: the two readouts (Eq. 17)
//              proj_a  the k block-entry active rows against W_post^A
//              fin_a   H_post^A
//   xhcf_mid   the attention write of Eq. 18 fused with the Eq. 19 correction
//              of the MLP input (the apply kernel of xhc_post.hip), then the
//              rewritten active rows against [W_res | W_post^M] and the
//              active-map finalize shared with the chained xHC calls
//   xhcf_post  full xHC's MLP write (xhc_post.hip)
//
// Every partial sum is written per split and summed in split order, so
// results do not depend on scheduling; nothing waits across workgroups.
#include "xhc_device.hpp"
#include "xhc_internal.hpp"
#include "xhc_tile.hpp"

namespace xhc {

namespace {

// cs[i] = sum over the rows of W (nrows x ncol, row-major) of W[row][i], for
// the router columns i < N, in two fixed-order stages: CSB workgroups each
// sum a contiguous range of rows (a thread reads a row's N router weights at
// a time) into part[b][i]; then one workgroup adds the CSB partials in order.
constexpr int CSB = 256;
template <class E, int N>
__global__ __launch_bounds__(256) void flash_colsum_kernel(const typename E::T* __restrict__ W, long nrows, int ncol,
                                                           float* __restrict__ part) {
  __shared__ float s[256][N];
  const int b = blockIdx.x, tid = threadIdx.x;
  const long lo = (long)b * nrows / CSB, hi = (long)(b + 1) * nrows / CSB;
  float acc[N];
#pragma unroll
  for (int i = 0; i < N; ++i) acc[i] = 0.f;
  for (long r = lo + tid; r < hi; r += 256) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if constexpr (sizeof(typename E::T) == 2) acc[i] += bf16_lo((uint32_t)W[r * ncol + i]);
      else acc[i] += W[r * ncol + i];
    }
  }
#pragma unroll
  for (int i = 0; i < N; ++i) s[tid][i] = acc[i];
  __syncthreads();
#pragma unroll
  for (int o = 128; o >= 1; o >>= 1) {
    if (tid < o) {
#pragma unroll
      for (int i = 0; i < N; ++i) s[tid][i] += s[tid + o][i];
    }
    __syncthreads();
  }
  if (tid < N) part[(size_t)b * N + tid] = s[0][tid];
}

template <int N>
__global__ __launch_bounds__(64) void flash_colsum_fin_kernel(const float* __restrict__ part, float* __restrict__ cs) {
  const int i = threadIdx.x;
  if (i >= N) return;
  float v = 0.f;
  for (int b = 0; b < CSB; ++b) v += part[(size_t)b * N + i];
  cs[i] = v;
}

struct FlashRouteArgs {
  int T, m, KS, NP;     // NP: columns per token of the projection partials
  long n_el;
  const float* part;    // [KS][T][NP]: router | pre-map 0 | pre-map 1 | ...
  const float* stats;   // [KS][T][2]: sum x, sum x^2
  const float* cs;      // [N]
  const float* b_pre[4];
  float a_pre[4], eps;
  int* idx;
  float *p, *z;
  float* h_pre[4];      // [T][N] per pre-map
};

// One token per thread: LayerNorm-corrected router logits, the NPRE
// RMS-scaled pre-maps, fixed-m + routed top-(k-m) and the router weights.
template <int N, int K, int NPRE>
__global__ __launch_bounds__(256) void flash_route_kernel(FlashRouteArgs a) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= a.T) return;
  constexpr int NC = (1 + NPRE) * N;
  float raw[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) raw[c] = 0.f;
  float q1 = 0.f, q2 = 0.f;
  for (int ks = 0; ks < a.KS; ++ks) {
    const float* pp = a.part + ((size_t)ks * a.T + t) * a.NP;
#pragma unroll
    for (int c = 0; c < NC; ++c) raw[c] += pp[c];
    q1 += a.stats[((size_t)ks * a.T + t) * 2];
    q2 += a.stats[((size_t)ks * a.T + t) * 2 + 1];
  }
  const float n_el = (float)a.n_el;
  float z[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
#pragma unroll
    for (int q = 0; q < NPRE; ++q) {
      float hp, zz;
      route_logits(raw[i], raw[(1 + q) * N + i], q1, q2, a.cs[i], n_el, a.eps, a.a_pre[q], a.b_pre[q][i], true, &zz,
                   &hp);
      if (q == 0) z[i] = zz;
      a.h_pre[q][(size_t)t * N + i] = hp;
    }
    a.z[(size_t)t * N + i] = z[i];
  }
  int sel[K];
  route_select<N, K>(z, a.m, sel);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    a.idx[(size_t)t * K + j] = sel[j];
    a.p[(size_t)t * K + j] = j < a.m ? 1.f : sigmoidf_(z[sel[j]]);
  }
}

struct FlashReadArgs {
  const void* X;
  void* out[4];
  int T, C, K;
  const float* h_pre[4];
  const int* idx;   // MASK only
};

// The NPRE readouts from one pass over X (Eq. 17).  A workgroup is one
// 16-token tile times a slice of 8 contraction blocks; each wave loads its
// block of all N streams at once (lane (g, r): token r, VEC channels) and
// forms every weighted sum.  With MASK, readouts 1.. leave out the token's
// active streams (the non-active bases of xHC-Flash-4sub).
template <class E, int N, int NPRE, bool MASK>
__global__ __launch_bounds__(512) void flash_read_kernel(FlashReadArgs a) {
  using T = typename E::T;
  constexpr int VEC = E::VEC, KB = E::KB;
  __shared__ float s_h[NPRE][TM][N];
  __shared__ uint32_t s_mask[TM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r = lane & 15;
  const int C = a.C, nkbC = C / KB;
  const int G = (nkbC + TWV - 1) / TWV;
  const int tile = blockIdx.x / G, slice = blockIdx.x % G;
  const int t0 = tile * TM;
  for (int u = tid; u < TM * N; u += TNTHR) {
    const int tau = u / N, t = t0 + tau;
#pragma unroll
    for (int q = 0; q < NPRE; ++q) s_h[q][tau][u % N] = t < a.T ? a.h_pre[q][(size_t)t0 * N + u] : 0.f;
  }
  if (MASK && tid < TM) {
    uint32_t mk = 0;
    if (t0 + tid < a.T)
      for (int j = 0; j < a.K; ++j) {
        const int v = a.idx[(size_t)(t0 + tid) * a.K + j];
        if (v >= 0 && v < N) mk |= 1u << v;
      }
    s_mask[tid] = mk;
  }
  const int kb = slice * TWV + wave;
  const int t = t0 + r;
  const bool valid = kb < nkbC && t < a.T;
  u32x4_t v[N];
  const T* xt = reinterpret_cast<const T*>(a.X) + (size_t)(valid ? t : 0) * N * C + (size_t)(valid ? kb : 0) * KB +
                VEC * g;
  if (valid) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = ld16v(xt + (size_t)i * C);
  }
  __syncthreads();
  if (!valid) return;
  const uint32_t mk = MASK ? s_mask[r] : 0u;
  float acc[NPRE][VEC];
#pragma unroll
  for (int q = 0; q < NPRE; ++q)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[q][e] = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float f[VEC];
    E::unpack(v[i], f);
#pragma unroll
    for (int q = 0; q < NPRE; ++q) {
      const float h = (q > 0 && ((mk >> i) & 1u)) ? 0.f : s_h[q][r][i];
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[q][e] = fmaf(h, f[e], acc[q][e]);
    }
  }
  const size_t o = (size_t)t * C + (size_t)kb * KB + VEC * g;
#pragma unroll
  for (int q = 0; q < NPRE; ++q) st16_nt(reinterpret_cast<T*>(a.out[q]) + o, E::packv(acc[q]));
}

struct ActProjArgs {
  const void* X;
  int T, C, N, G, ntiles;
  const int* idx;
  const uint4* wp;   // packed [k*C][NT*16] B fragments
  float* part;       // [ntiles][G][P]: token-major projection, then the sums of squares
};

// The k active rows of each token (in the order of the active list) against
// a packed [k*C] x [NT*16] weight, split over G ranges of the k*C
// contraction.  One wave per 16-token tile; lane (g, r) streams token r's
// active rows.  Writes per (tile, split) the projection and sum x^2 per token.
template <class E, int NT, int K>
__global__ __launch_bounds__(256) void flash_act_proj_kernel(ActProjArgs a) {
  using T = typename E::T;
  constexpr int VEC = E::VEC, KB = E::KB, NP = NT * 16, P = TM * NP + TM;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, r = lane & 15;
  const int tile = blockIdx.x * 4 + wave;
  if (tile >= a.ntiles) return;   // whole waves only; no barrier below
  const int split = blockIdx.y;
  const int C = a.C, nkbC = C / KB;
  const long nkb = (long)K * nkbC;
  const long kb0 = (long)split * nkb / a.G, kb1 = (long)(split + 1) * nkb / a.G;
  const int tok = tile * TM + r;
  const bool valid = tok < a.T;
  f32x4_t acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float s2 = 0.f;
  const uint4* wp = a.wp + lane;
  const u32x4_t zero = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const long jb0 = (long)j * nkbC, jb1 = jb0 + nkbC;
    const long lo = kb0 > jb0 ? kb0 : jb0, hi = kb1 < jb1 ? kb1 : jb1;
    if (lo >= hi) continue;
    int row = valid ? a.idx[(size_t)tok * K + j] : 0;
    row = row < 0 ? 0 : (row >= a.N ? a.N - 1 : row);
    const T* xr = reinterpret_cast<const T*>(a.X) + ((size_t)(valid ? tok : 0) * a.N + row) * C + VEC * g;
    auto step = [&](const u32x4_t& v, long kb) {
      float f[VEC];
      E::unpack(v, f);
#pragma unroll
      for (int e = 0; e < VEC; ++e) s2 = fmaf(f[e], f[e], s2);
#pragma unroll
      for (int n = 0; n < NT; ++n)
        acc[n] = E::mma(acc[n], v, __builtin_bit_cast(u32x4_t, wp[(kb * NT + n) * WAVE]));
    };
    constexpr int U = 4;
    long kb = lo;
    for (; kb + U <= hi; kb += U) {
      u32x4_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = valid ? ld16v(xr + (kb + u - jb0) * KB) : zero;
#pragma unroll
      for (int u = 0; u < U; ++u) step(v[u], kb + u);
    }
    for (; kb < hi; ++kb) step(valid ? ld16v(xr + (kb - jb0) * KB) : zero, kb);
  }
  s2 += __shfl_xor(s2, 16, WAVE);
  s2 += __shfl_xor(s2, 32, WAVE);
  float* dst = a.part + ((size_t)tile * a.G + split) * P;
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(4 * g + i) * NP + n * 16 + r] = acc[n][i];
  if (g == 0) dst[TM * NP + r] = s2;
}

struct AttnFinArgs {
  int T, C, G;
  const float* part;   // [ntiles][G][TM * NT * 16 + TM]
  const float* b_po;
  float a_po, eps;
  float* h_post;       // [T][K][KR]
};

// H_post = 2 sigmoid(alpha RMSNorm(vec X_act) W_post + b) of an unmixed
// sublayer (entry (j, r) at column j KR + r), one token per thread.
template <int K, int KR, int NT>
__global__ __launch_bounds__(256) void flash_post_fin_kernel(AttnFinArgs a) {
  constexpr int NP = NT * 16, P = TM * NP + TM;
  static_assert(K * KR <= NP, "post-map columns");
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= a.T) return;
  const int tile = t / TM, tau = t % TM;
  float raw[K * KR], s2 = 0.f;
#pragma unroll
  for (int j = 0; j < K * KR; ++j) raw[j] = 0.f;
  for (int s = 0; s < a.G; ++s) {
    const float* pp = a.part + ((size_t)tile * a.G + s) * P;
#pragma unroll
    for (int j = 0; j < K * KR; ++j) raw[j] += pp[tau * NP + j];
    s2 += pp[TM * NP + tau];
  }
  const float rr = 1.f / sqrtf(s2 / ((float)K * (float)a.C) + a.eps);
#pragma unroll
  for (int j = 0; j < K * KR; ++j)
    a.h_post[(size_t)t * K * KR + j] = 2.f * sigmoidf_(fmaf(a.a_po * raw[j], rr, a.b_po[j]));
}

struct ActInArgs {
  const void* X;
  void* inp;
  const void* base;    // [T][C]: this sublayer's non-active base
  int T, C, N, G, ntiles;
  const int* idx;
  const float* h_pre;  // [T][N]: this sublayer's pre-map
  const uint4* wp;     // packed [k*C][NT*16] B fragments of its active-map weights
  float* part;         // [ntiles][G][TM * NT * 16 + TM]
};

// Input and active-map projection of an xHC-Flash-4sub sublayer from one read
// of the k active rows: inp = base + sum_j H_pre[I_j] x_j (the active-state
// form of the input), and the rows against the packed weights, with their
// sum of squares.  One wave per 16-token tile, G splits of the channels; the
// k rows of a channel block are loaded together.
template <class E, int NT, int K>
__global__ __launch_bounds__(256) void flash_act_input_kernel(ActInArgs a) {
  using T = typename E::T;
  constexpr int VEC = E::VEC, KB = E::KB, NP = NT * 16, P = TM * NP + TM;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, r = lane & 15;
  const int tile = blockIdx.x * 4 + wave;
  if (tile >= a.ntiles) return;   // whole waves only; no barrier below
  const int split = blockIdx.y;
  const int C = a.C, nkbC = C / KB;
  const int kc0 = (int)((long)split * nkbC / a.G), kc1 = (int)((long)(split + 1) * nkbC / a.G);
  const int tok = tile * TM + r;
  const bool valid = tok < a.T;
  const int tk = valid ? tok : 0;
  int row[K];
  float hI[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    int v = valid ? a.idx[(size_t)tok * K + j] : 0;
    v = v < 0 ? 0 : (v >= a.N ? a.N - 1 : v);
    row[j] = v;
    hI[j] = valid ? a.h_pre[(size_t)tok * a.N + v] : 0.f;
  }
  const T* X = reinterpret_cast<const T*>(a.X);
  const T* base = reinterpret_cast<const T*>(a.base) + (size_t)tk * C + VEC * g;
  T* inp = reinterpret_cast<T*>(a.inp) + (size_t)tk * C + VEC * g;
  f32x4_t acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float s2 = 0.f;
  const uint4* wp = a.wp + lane;
  const u32x4_t zero = u32x4_t{0u, 0u, 0u, 0u};
  for (int kbc = kc0; kbc < kc1; ++kbc) {
    const int c = kbc * KB;
    u32x4_t xa[K];
#pragma unroll
    for (int j = 0; j < K; ++j) xa[j] = valid ? ld16v(X + ((size_t)tk * a.N + row[j]) * C + c + VEC * g) : zero;
    const u32x4_t bv = valid ? ld16v(base + c) : zero;
    float o[VEC];
    E::unpack(bv, o);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      float f[VEC];
      E::unpack(xa[j], f);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        o[e] = fmaf(hI[j], f[e], o[e]);
        s2 = fmaf(f[e], f[e], s2);
      }
#pragma unroll
      for (int n = 0; n < NT; ++n)
        acc[n] = E::mma(acc[n], xa[j], __builtin_bit_cast(u32x4_t, wp[(((size_t)j * nkbC + kbc) * NT + n) * WAVE]));
    }
    if (valid) st16_nt(inp + c, E::packv(o));
  }
  s2 += __shfl_xor(s2, 16, WAVE);
  s2 += __shfl_xor(s2, 32, WAVE);
  float* dst = a.part + ((size_t)tile * a.G + split) * P;
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(4 * g + i) * NP + n * 16 + r] = acc[n][i];
  if (g == 0) dst[TM * NP + r] = s2;
}

template <class E, int NT, int K>
void act_proj_launch(const Plan& P, const void* X, const char* ws, const uint4* wp, float* part, hipStream_t st) {
  ActProjArgs a;
  a.X = X; a.T = (int)P.T; a.C = P.C; a.N = P.N; a.G = P.G2; a.ntiles = (int)P.ntiles;
  a.idx = reinterpret_cast<const int*>(ws + P.o_idx);
  a.wp = wp;
  a.part = part;
  dim3 grid((unsigned)((P.ntiles + 3) / 4), (unsigned)P.G2);
  flash_act_proj_kernel<E, NT, K><<<grid, 256, 0, st>>>(a);
}

template <class E, int N, int K>
bool flash_pre_launch(const Plan& P, const xhcf_weights* w, const void* X, void* inp_a, void* inp_m, char* ws,
                      hipStream_t st) {
  using TT = typename E::T;
  launch_pack_b(P.dtype, w->w_full, P.nkb_full, P.ncol_full, P.NTF, ws + P.o_wfull, st);
  launch_pack_b(P.dtype, w->w_post_attn, P.nkb_act, P.K, 1, ws + P.o_wact_a, st);
  launch_pack_b(P.dtype, w->w_act_mlp, P.nkb_act, P.ncol_act, P.NTA, ws + P.o_wact, st);
  float* cs = reinterpret_cast<float*>(ws + P.o_colsum);
  float* part = reinterpret_cast<float*>(ws + P.o_part);
  float* stats = reinterpret_cast<float*>(ws + P.o_stats);
  FlashRouteArgs r{};
  r.idx = reinterpret_cast<int*>(ws + P.o_idx);
  r.p = reinterpret_cast<float*>(ws + P.o_p);
  r.h_pre[0] = reinterpret_cast<float*>(ws + P.o_hpre);
  r.h_pre[1] = reinterpret_cast<float*>(ws + P.o_hpre_m);
  r.z = reinterpret_cast<float*>(ws + P.o_z);
  if (N == 16 && K == 4) {
    // persistent projection with the slice's weights on chip
    if (!launch_flash_route_p(P, X, ws + P.o_wfull, part, w, r.idx, r.p, r.h_pre[0], r.h_pre[1], r.z, st))
      return false;
  } else {
  flash_colsum_kernel<E, N><<<CSB, 256, 0, st>>>(reinterpret_cast<const TT*>(w->w_full), (long)N * P.C, P.ncol_full,
                                                 cs + N);
  flash_colsum_fin_kernel<N><<<1, 64, 0, st>>>(cs + N, cs);
  if (!launch_projection(P.dtype, P.NTF, X, (int)P.T, (long)N * P.C, ws + P.o_wfull, P.nkb_full, P.KS, part, stats,
                         st))
    return false;

  r.T = (int)P.T; r.m = P.m; r.KS = P.KS; r.NP = P.NTF * 16; r.n_el = (long)N * P.C;
  r.part = part; r.stats = stats; r.cs = cs;
  r.b_pre[0] = w->b_pre_attn; r.b_pre[1] = w->b_pre_mlp;
  r.a_pre[0] = w->alpha_pre_attn; r.a_pre[1] = w->alpha_pre_mlp; r.eps = P.eps_norm;
  flash_route_kernel<N, K, 2><<<(unsigned)((P.T + 255) / 256), 256, 0, st>>>(r);
  }

  FlashReadArgs d{};
  d.X = X; d.out[0] = inp_a; d.out[1] = inp_m; d.T = (int)P.T; d.C = P.C; d.K = P.K;
  d.h_pre[0] = r.h_pre[0]; d.h_pre[1] = r.h_pre[1];
  const int nkbC = P.C / E::KB;
  if (flash_read_s_applies(P)) {
    if (!launch_flash_read_s(P, X, d.out, d.h_pre, nullptr, 2, st)) return false;
  } else {
    flash_read_kernel<E, N, 2, false><<<(unsigned)(P.ntiles * ((nkbC + TWV - 1) / TWV)), TNTHR, 0, st>>>(d);
  }

  float* part2 = reinterpret_cast<float*>(ws + P.o_part2);
  act_proj_launch<E, 1, K>(P, X, ws, reinterpret_cast<const uint4*>(ws + P.o_wact_a), part2, st);
  AttnFinArgs f;
  f.T = (int)P.T; f.C = P.C; f.G = P.G2; f.part = part2;
  f.b_po = w->b_post_attn; f.a_po = w->alpha_post_attn; f.eps = P.eps_norm;
  f.h_post = reinterpret_cast<float*>(ws + P.o_hpost_a);
  flash_post_fin_kernel<K, 1, 1><<<(unsigned)((P.T + 255) / 256), 256, 0, st>>>(f);
  return true;
}

template <class E, int K, int KR>
bool flash_mid_launch(const Plan& P, const xhcf_weights* w, void* X, const void* out_a, void* inp_m, char* ws,
                      hipStream_t st) {
  if (!launch_flash_attn_write(P, X, out_a, inp_m, ws, st)) return false;
  constexpr int NTA = (K * K + K * KR + 15) / 16;
  float* part2 = reinterpret_cast<float*>(ws + P.o_part2);
  act_proj_launch<E, NTA, K>(P, X, ws, reinterpret_cast<const uint4*>(ws + P.o_wact), part2, st);
  return launch_act_fin(P, P.G2, part2, w->b_res, w->b_post_mlp, w->alpha_res, w->alpha_post_mlp,
                        reinterpret_cast<float*>(ws + P.o_hres), reinterpret_cast<float*>(ws + P.o_hpost), st);
}

template <class E>
bool flash_pre_dispatch(const Plan& P, const xhcf_weights* w, const void* X, void* inp_a, void* inp_m, char* ws,
                        hipStream_t st) {
  switch (P.N * 10 + P.K) {
    case 164: return flash_pre_launch<E, 16, 4>(P, w, X, inp_a, inp_m, ws, st);
    case 84: return flash_pre_launch<E, 8, 4>(P, w, X, inp_a, inp_m, ws, st);
    case 44: return flash_pre_launch<E, 4, 4>(P, w, X, inp_a, inp_m, ws, st);
    case 11: return flash_pre_launch<E, 1, 1>(P, w, X, inp_a, inp_m, ws, st);
    default: return false;
  }
}

template <class E>
bool flash_mid_dispatch(const Plan& P, const xhcf_weights* w, void* X, const void* out_a, void* inp_m, char* ws,
                        hipStream_t st) {
  switch (P.K * 10 + P.KR) {
    case 44: return flash_mid_launch<E, 4, 4>(P, w, X, out_a, inp_m, ws, st);
    case 41: return flash_mid_launch<E, 4, 1>(P, w, X, out_a, inp_m, ws, st);
    case 14: return flash_mid_launch<E, 1, 4>(P, w, X, out_a, inp_m, ws, st);
    case 11: return flash_mid_launch<E, 1, 1>(P, w, X, out_a, inp_m, ws, st);
    default: return false;
  }
}

// ---------------------------------------------------------------------------
// xHC-Flash-4sub: one routing and four pre-maps for two blocks.
// ---------------------------------------------------------------------------
template <class E, int N, int K>
bool flash4_pre_launch(const Plan& P, const xhcf4_weights* w, const void* X, void* inp, void* bases, char* ws,
                       hipStream_t st) {
  using TT = typename E::T;
  const int KRm = P.KR;
  launch_pack_b(P.dtype, w->w_full, P.nkb_full, P.ncol_full, P.NTF, ws + P.o_wfull, st);
  const int ncq[3] = {P.K, P.K * KRm, P.K};
  for (int q = 0; q < 3; ++q)
    launch_pack_b(P.dtype, w->w_post[q], P.nkb_act, ncq[q], (ncq[q] + 15) / 16, ws + P.o_wq[q], st);
  launch_pack_b(P.dtype, w->w_act_last, P.nkb_act, P.ncol_act, P.NTA, ws + P.o_wact, st);
  float* part = reinterpret_cast<float*>(ws + P.o_part);
  FlashRouteArgs r{};
  for (int q = 0; q < 4; ++q) {
    r.b_pre[q] = w->b_pre[q];
    r.a_pre[q] = w->alpha_pre[q];
    r.h_pre[q] = reinterpret_cast<float*>(ws + P.o_hpre) + (size_t)q * P.T * N;
  }
  r.idx = reinterpret_cast<int*>(ws + P.o_idx);
  r.p = reinterpret_cast<float*>(ws + P.o_p);
  r.z = reinterpret_cast<float*>(ws + P.o_z);
  if (flash4_route_p_applies(P)) {
    // the staged persistent projection, partials per (tile, slice)
    Flash4Route o;
    for (int q = 0; q < 4; ++q) {
      o.b_pre[q] = r.b_pre[q];
      o.a_pre[q] = r.a_pre[q];
      o.h_pre[q] = r.h_pre[q];
    }
    o.idx = r.idx; o.p = r.p; o.z = r.z;
    if (!launch_flash4_route_p(P, X, ws + P.o_wfull, part, o, st)) return false;
  } else {
    float* cs = reinterpret_cast<float*>(ws + P.o_colsum);
    flash_colsum_kernel<E, N><<<CSB, 256, 0, st>>>(reinterpret_cast<const TT*>(w->w_full), (long)N * P.C,
                                                   P.ncol_full, cs + N);
    flash_colsum_fin_kernel<N><<<1, 64, 0, st>>>(cs + N, cs);
    float* stats = reinterpret_cast<float*>(ws + P.o_stats);
    if (!launch_projection(P.dtype, P.NTF, X, (int)P.T, (long)N * P.C, ws + P.o_wfull, P.nkb_full, P.KS, part,
                           stats, st))
      return false;
    r.T = (int)P.T; r.m = P.m; r.KS = P.KS; r.NP = P.NTF * 16; r.n_el = (long)N * P.C;
    r.part = part; r.stats = stats; r.cs = cs; r.eps = P.eps_norm;
    flash_route_kernel<N, K, 4><<<(unsigned)((P.T + 255) / 256), 256, 0, st>>>(r);
  }

  FlashReadArgs d{};
  d.X = X; d.T = (int)P.T; d.C = P.C; d.K = P.K; d.idx = r.idx;
  d.out[0] = inp;
  for (int q = 1; q < 4; ++q) d.out[q] = static_cast<TT*>(bases) + (size_t)(q - 1) * P.T * P.C;
  for (int q = 0; q < 4; ++q) d.h_pre[q] = r.h_pre[q];
  const int nkbC = P.C / E::KB;
  if (flash_read_s_applies(P)) {
    if (!launch_flash_read_s(P, X, d.out, d.h_pre, d.idx, 4, st)) return false;
  } else {
    flash_read_kernel<E, N, 4, true><<<(unsigned)(P.ntiles * ((nkbC + TWV - 1) / TWV)), TNTHR, 0, st>>>(d);
  }

  // the first sublayer's post-map from the group-entry active rows
  float* part2 = reinterpret_cast<float*>(ws + P.o_part2);
  act_proj_launch<E, 1, K>(P, X, ws, reinterpret_cast<const uint4*>(ws + P.o_wq[0]), part2, st);
  AttnFinArgs f;
  f.T = (int)P.T; f.C = P.C; f.G = P.G2; f.part = part2;
  f.b_po = w->b_post[0]; f.a_po = w->alpha_post[0]; f.eps = P.eps_norm;
  f.h_post = reinterpret_cast<float*>(ws + P.o_hpost);
  flash_post_fin_kernel<K, 1, 1><<<(unsigned)((P.T + 255) / 256), 256, 0, st>>>(f);
  return true;
}

template <class E, int NT, int K>
void act_input_launch(const Plan& P, const void* X, void* inp, const void* base, const float* h_pre, const char* ws,
                      const uint4* wp, float* part, hipStream_t st) {
  ActInArgs a;
  a.X = X; a.inp = inp; a.base = base; a.T = (int)P.T; a.C = P.C; a.N = P.N; a.G = P.G2; a.ntiles = (int)P.ntiles;
  a.idx = reinterpret_cast<const int*>(ws + P.o_idx);
  a.h_pre = h_pre;
  a.wp = wp;
  a.part = part;
  dim3 grid((unsigned)((P.ntiles + 3) / 4), (unsigned)P.G2);
  flash_act_input_kernel<E, NT, K><<<grid, 256, 0, st>>>(a);
}

// Sublayer q (1..4): its write; then, for q < 4, the input of sublayer q + 1
// and its active maps (a post-map for sublayers 2 and 3, H_res and the
// post-map for the final MLP).
template <class E, int K, int KR>
bool flash4_post_launch(const Plan& P, const xhcf4_weights* w, int q, void* X, const void* out, const void* bases,
                        void* inp, char* ws, hipStream_t st) {
  using TT = typename E::T;
  if (q == 4) {
    xhc_weights wx{};
    wx.conv_w = w->conv_w[1];
    return launch_xhc_post(P, X, out, &wx, ws, st);
  }
  if (!launch_unmixed_write(P, q == 2 ? KR : 1, X, out, q == 2 ? w->conv_w[0] : nullptr, ws, st)) return false;
  const void* base = static_cast<const TT*>(bases) + (size_t)(q - 1) * P.T * P.C;
  const float* hp = reinterpret_cast<const float*>(ws + P.o_hpre) + (size_t)q * P.T * P.N;
  float* part2 = reinterpret_cast<float*>(ws + P.o_part2);
  AttnFinArgs f;
  f.T = (int)P.T; f.C = P.C; f.G = P.G2; f.part = part2; f.eps = P.eps_norm;
  f.h_post = reinterpret_cast<float*>(ws + P.o_hpost);
  const unsigned gt = (unsigned)((P.T + 255) / 256);
  if (q == 1) {   // next: the first MLP, unmixed, K_r components
    constexpr int NT2 = (K * KR + 15) / 16;
    act_input_launch<E, NT2, K>(P, X, inp, base, hp, ws, reinterpret_cast<const uint4*>(ws + P.o_wq[1]), part2, st);
    f.b_po = w->b_post[1]; f.a_po = w->alpha_post[1];
    flash_post_fin_kernel<K, KR, NT2><<<gt, 256, 0, st>>>(f);
    return true;
  }
  if (q == 2) {   // next: the second attention
    act_input_launch<E, 1, K>(P, X, inp, base, hp, ws, reinterpret_cast<const uint4*>(ws + P.o_wq[2]), part2, st);
    f.b_po = w->b_post[2]; f.a_po = w->alpha_post[2];
    flash_post_fin_kernel<K, 1, 1><<<gt, 256, 0, st>>>(f);
    return true;
  }
  // q == 3, next: the final MLP with its residual map
  constexpr int NTA = (K * K + K * KR + 15) / 16;
  act_input_launch<E, NTA, K>(P, X, inp, base, hp, ws, reinterpret_cast<const uint4*>(ws + P.o_wact), part2, st);
  return launch_act_fin(P, P.G2, part2, w->b_res, w->b_post[3], w->alpha_res, w->alpha_post[3],
                        reinterpret_cast<float*>(ws + P.o_hres), reinterpret_cast<float*>(ws + P.o_hpost), st);
}

template <class E>
bool flash4_pre_dispatch(const Plan& P, const xhcf4_weights* w, const void* X, void* inp, void* bases, char* ws,
                         hipStream_t st) {
  switch (P.N * 10 + P.K) {
    case 164: return flash4_pre_launch<E, 16, 4>(P, w, X, inp, bases, ws, st);
    case 84: return flash4_pre_launch<E, 8, 4>(P, w, X, inp, bases, ws, st);
    case 44: return flash4_pre_launch<E, 4, 4>(P, w, X, inp, bases, ws, st);
    case 11: return flash4_pre_launch<E, 1, 1>(P, w, X, inp, bases, ws, st);
    default: return false;
  }
}

template <class E>
bool flash4_post_dispatch(const Plan& P, const xhcf4_weights* w, int q, void* X, const void* out, const void* bases,
                          void* inp, char* ws, hipStream_t st) {
  switch (P.K * 10 + P.KR) {
    case 44: return flash4_post_launch<E, 4, 4>(P, w, q, X, out, bases, inp, ws, st);
    case 41: return flash4_post_launch<E, 4, 1>(P, w, q, X, out, bases, inp, ws, st);
    case 14: return flash4_post_launch<E, 1, 4>(P, w, q, X, out, bases, inp, ws, st);
    case 11: return flash4_post_launch<E, 1, 1>(P, w, q, X, out, bases, inp, ws, st);
    default: return false;
  }
}

}  // namespace

bool launch_xhcf4_pre(const Plan& P, const xhcf4_weights* w, const void* X, void* inp, void* bases, char* ws,
                      hipStream_t st) {
  return P.dtype == XHC_BF16 ? flash4_pre_dispatch<Bf16>(P, w, X, inp, bases, ws, st)
                             : flash4_pre_dispatch<F32>(P, w, X, inp, bases, ws, st);
}

bool launch_xhcf4_post(const Plan& P, const xhcf4_weights* w, int q, void* X, const void* out, const void* bases,
                       void* inp, char* ws, hipStream_t st) {
  return P.dtype == XHC_BF16 ? flash4_post_dispatch<Bf16>(P, w, q, X, out, bases, inp, ws, st)
                             : flash4_post_dispatch<F32>(P, w, q, X, out, bases, inp, ws, st);
}

bool launch_xhcf_pre(const Plan& P, const xhcf_weights* w, const void* X, void* inp_a, void* inp_m, char* ws,
                     hipStream_t st) {
  return P.dtype == XHC_BF16 ? flash_pre_dispatch<Bf16>(P, w, X, inp_a, inp_m, ws, st)
                             : flash_pre_dispatch<F32>(P, w, X, inp_a, inp_m, ws, st);
}

bool launch_xhcf_mid(const Plan& P, const xhcf_weights* w, void* X, const void* out_a, void* inp_m, char* ws,
                     hipStream_t st) {
  return P.dtype == XHC_BF16 ? flash_mid_dispatch<Bf16>(P, w, X, out_a, inp_m, ws, st)
                             : flash_mid_dispatch<F32>(P, w, X, out_a, inp_m, ws, st);
}

}  // namespace xhc
