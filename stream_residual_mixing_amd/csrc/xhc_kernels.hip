// libxhc kernels for gfx950.
//
// mHC pre stage (mapping generation + dense read):
//   pack_b      weights -> MFMA B fragments (once per call, a few MiB)
//   proj_gen    one pass over X: split-K bf16/f32 MFMA projection of the raw
//               (un-normalised) flattened state, plus sum x and sum x^2
//   mhc_read    per 16 tokens: RMS correction, H_pre / H_post, N x N
//               Sinkhorn, dense read -> inp
// (the xHC pre stage is the one-pass kernel of xhc_pre.hip)
// mHC post stage:
//   mhc_post    dense N x N mix + rank-1 write, in place
// (the xHC post stage is in xhc_post.hip)
//
// Normalisations are applied after the projection, from sum x and sum x^2,
// so no normalised state is ever materialised (xHC paper "xHC: Expanded
// Hyper-Connections", paragraph "Mapping generation").
#include "xhc_device.hpp"
#include "xhc_internal.hpp"

#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

// contraction blocks a proj_gen lane loads ahead (measured: 4 and 8 within
// 2% of each other, 16 slower)
#ifndef XHC_GEN_U
#define XHC_GEN_U 4
#endif

namespace xhc {

thread_local const char* g_launch_failure = nullptr;

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

  constexpr int U = XHC_GEN_U;
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
// mHC post kernel: block = 32 tokens x one slice of 256 threads x 4 channels.
// ---------------------------------------------------------------------------

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
    case 3: launch_gen<E, 3>(X, T, K, Wp, nkb, KS, part, stats, st); return true;
    case 5: launch_gen<E, 5>(X, T, K, Wp, nkb, KS, part, stats, st); return true;
    case 18: launch_gen<E, 18>(X, T, K, Wp, nkb, KS, part, stats, st); return true;
    default: return false;
  }
}

// ---------------------------------------------------------------------------
// Sums of x and x^2 over each token's flattened state (one wave per token,
// 16-byte loads, eight in flight per lane), for the RMSNorm of the wide mHC
// maps whose projection runs as a library GEMM.  stats[t] = (sum x, sum x^2).
// ---------------------------------------------------------------------------
template <class E>
__global__ __launch_bounds__(256) void mhc_sumsq_kernel(const typename E::T* __restrict__ X, int T, long NC,
                                                        float* __restrict__ stats) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const typename E::T* row = X + (size_t)t * NC;
  constexpr int U = 8;
  const long step = (long)WAVE * E::VEC;
  float s1 = 0.f, s2 = 0.f;
  long c = (long)lane * E::VEC;
  for (; c + (U - 1) * step < NC; c += U * step) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld16(row + c + u * step);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float f[E::VEC];
      E::unpack(v[u], f);
#pragma unroll
      for (int e = 0; e < E::VEC; ++e) { s1 += f[e]; s2 = fmaf(f[e], f[e], s2); }
    }
  }
  for (; c < NC; c += step) {
    float f[E::VEC];
    E::unpack(ld16(row + c), f);
#pragma unroll
    for (int e = 0; e < E::VEC; ++e) { s1 += f[e]; s2 = fmaf(f[e], f[e], s2); }
  }
  s1 = wave_sum(s1);
  s2 = wave_sum(s2);
  if (lane == 0) {
    stats[(size_t)t * 2] = s1;
    stats[(size_t)t * 2 + 1] = s2;
  }
}

// The library GEMM of the wide mHC projection: raw[t][0..ncol) = vec X_t . W
// (bf16 in, float out, rows of raw NP floats apart).  hipBLASLt is column-major,
// so it computes raw^T (ncol x T, ld NP) = W^T (ncol x NC, ld ncol) X^T (NC x T,
// ld NC), reading both operands in their row-major layout untransposed.  One
// handle per device and one algorithm per shape, chosen by the library's
// heuristic on first use and kept for the process.
struct LtShape {
  int dev;
  long T, NC, ncol, NP;
  bool operator<(const LtShape& o) const {
    return std::tie(dev, T, NC, ncol, NP) < std::tie(o.dev, o.T, o.NC, o.ncol, o.NP);
  }
};
struct LtPlan {
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
  hipblasLtMatmulAlgo_t algo{};
  size_t ws = 0;
};

static bool lt_gemm(const void* X, const void* W, float* raw, long T, long NC, long ncol, long NP, void* ws,
                    size_t ws_bytes, hipStream_t st) {
  static std::mutex mu;
  static hipblasLtHandle_t handles[64] = {};
  static std::map<LtShape, LtPlan> plans;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  std::lock_guard<std::mutex> lock(mu);
  if (!handles[dev] && hipblasLtCreate(&handles[dev]) != HIPBLAS_STATUS_SUCCESS) return false;
  const LtShape key{dev, T, NC, ncol, NP};
  auto it = plans.find(key);
  if (it == plans.end()) {
    LtPlan p;
    const hipblasOperation_t opn = HIPBLAS_OP_N;
    if (hipblasLtMatmulDescCreate(&p.op, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSA, &opn, sizeof opn) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSB, &opn, sizeof opn) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p.a, HIP_R_16BF, ncol, NC, ncol) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p.b, HIP_R_16BF, NC, T, NC) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p.d, HIP_R_32F, ncol, T, NP) != HIPBLAS_STATUS_SUCCESS)
      return false;
    hipblasLtMatmulPreference_t pref = nullptr;
    const uint64_t maxws = ws_bytes;
    hipblasLtMatmulHeuristicResult_t res[8];
    int n = 0;
    if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) return false;
    const bool ok = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &maxws,
                                                          sizeof maxws) == HIPBLAS_STATUS_SUCCESS &&
                    hipblasLtMatmulAlgoGetHeuristic(handles[dev], p.op, p.a, p.b, p.d, p.d, pref, 8, res, &n) ==
                        HIPBLAS_STATUS_SUCCESS &&
                    n > 0;
    hipblasLtMatmulPreferenceDestroy(pref);
    if (!ok) return false;
    p.algo = res[0].algo;
    p.ws = res[0].workspaceSize;
    it = plans.emplace(key, p).first;
  }
  const LtPlan& p = it->second;
  if (p.ws > ws_bytes) return false;
  const float one = 1.f, zero = 0.f;
  return hipblasLtMatmul(handles[dev], p.op, &one, W, p.a, X, p.b, &zero, raw, p.d, raw, p.d, &p.algo, ws, p.ws,
                         st) == HIPBLAS_STATUS_SUCCESS;
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
static bool mhc_pre_launch(const Plan& P, const void* X, void* inp, const xhc_weights* w, char* ws, hipStream_t st) {
  if (P.mhc_gemm) {
    const long NC = (long)P.N * P.C;
    mhc_sumsq_kernel<E><<<(unsigned)((P.T + 3) / 4), 256, 0, st>>>(reinterpret_cast<const typename E::T*>(X),
                                                                      (int)P.T, NC,
                                                                      reinterpret_cast<float*>(ws + P.o_stats));
    if (!lt_gemm(X, w->w_full, reinterpret_cast<float*>(ws + P.o_part), P.T, NC, P.ncol_full, (long)P.NTF * 16,
                 ws + P.o_gemm_ws, P.gemm_ws_bytes, st)) {
      g_launch_failure = "hipBLASLt GEMM of the full-state projection failed";
      return false;
    }
  } else {
    launch_pack<E>(w->w_full, P.nkb_full, P.ncol_full, P.NTF, ws + P.o_wfull, st);
    if (!gen_dispatch<E>(P.NTF, X, (int)P.T, (long)P.N * P.C, ws + P.o_wfull, P.nkb_full, P.KS,
                         reinterpret_cast<float*>(ws + P.o_part), reinterpret_cast<float*>(ws + P.o_stats), st))
      return false;
  }
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

bool launch_mhc_pre(const Plan& P, const void* X, void* inp, const xhc_weights* w, char* ws, hipStream_t st) {
  return P.dtype == XHC_BF16 ? mhc_pre_launch<Bf16>(P, X, inp, w, ws, st) : mhc_pre_launch<F32>(P, X, inp, w, ws, st);
}
bool launch_mhc_post(const Plan& P, void* X, const void* out, char* ws, hipStream_t st) {
  return P.dtype == XHC_BF16 ? mhc_post_launch<Bf16>(P, X, out, ws, st) : mhc_post_launch<F32>(P, X, out, ws, st);
}

// Packing and split-K projection for other launchers (xHC-Flash): W [nkb*KB]
// x [ncol] into NT-tile B fragments at out; X [T][K] . W -> part, stats.
void launch_pack_b(int dtype, const void* W, long nkb, int ncol, int NT, void* out, hipStream_t st) {
  if (dtype == XHC_BF16) launch_pack<Bf16>(W, nkb, ncol, NT, out, st);
  else launch_pack<F32>(W, nkb, ncol, NT, out, st);
}

bool launch_projection(int dtype, int NT, const void* X, int T, long K, const void* Wp, long nkb, int KS,
                       float* part, float* stats, hipStream_t st) {
  return dtype == XHC_BF16 ? gen_dispatch<Bf16>(NT, X, T, K, Wp, nkb, KS, part, stats, st)
                           : gen_dispatch<F32>(NT, X, T, K, Wp, nkb, KS, part, stats, st);
}

}  // namespace xhc
