// xHC before the sublayer, in one pass over the state (gfx950).
//
// The mapping generation of xHC needs a reduction over a token's whole
// flattened state (N*C values) before the dense read of that same state can
// start (xHC paper "xHC: Expanded Hyper-Connections", paragraphs "Mapping
// generation" and "Mapping application").  Reading X twice from HBM would
// cost 32 C-elements per token instead of 16, so here the work of a tile of
// 16 tokens is split over G workgroups by channel slice ("split-K"), and each
// workgroup keeps its slice of the tile (all N streams) in registers while
// the G partial projections are combined:
//
//   phase 1  load the slice (16-byte non-temporal loads straight into MFMA
//            A fragments), partial projection onto [W_r | W_pre] with bf16 (or
//            f32) MFMA, partial sums of x and x^2, partial column sums of W_r
//            (an MFMA with an all-ones A operand); publish the partial.
//   phase 2  the last workgroup of the tile to publish sums the G partials in
//            slice order (so every result is independent of arrival order),
//            applies the LayerNorm / RMSNorm corrections, computes router
//            logits, H_pre, the fixed + routed top-k, and releases the tile;
//            the others wait for that release.
//   phase 3  from the registers: dense read inp = sum_i H_pre[i] X_i, gather
//            of the k active rows, their sum of squares and partial active
//            projection onto [W_res | W_post]; publish; the last workgroup
//            to publish finishes RMSNorm, k x k Sinkhorn + row clamp and H_post.
//
// Workgroups take tiles in the order of a ticket drawn from a global counter,
// so a workgroup that waits only ever waits for workgroups that have already
// started; with room for G workgroups on the device at once every wait ends.
// Each wait is also bounded: past the bound the kernel records a status word
// and carries on (results are then invalid, and the host can see it).
#include "xhc_internal.hpp"
#include "xhc_tile.hpp"

namespace xhc {

namespace {

constexpr int NKW = PRE_NKW;  // contraction blocks per wave and stream
constexpr int WV = PRE_WV;    // waves per workgroup
constexpr int NTHR = WV * 64;
static_assert(WV == TWV, "tile workgroups are 8 waves");
// A wait gives up after this many ticks of the 100 MHz real-time counter (2 s).
constexpr uint64_t WAIT_LIMIT_TICKS = 200000000ull;

// Wait until *flag != 0 (one lane); bounded in time.  The polling loads are
// coherent but not acquiring (an acquire per poll would invalidate caches on
// every iteration); what the flag guards is then read with coherent loads.
__device__ __forceinline__ void wait_flag(int* flag, int* status) {
  const uint64_t start = wall_clock64();
  while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
    __builtin_amdgcn_s_sleep(2);
    if (wall_clock64() - start > WAIT_LIMIT_TICKS) {
      __hip_atomic_store(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
  }
}

}  // namespace

template <class E, int N, int K, int KR>
__global__ __launch_bounds__(NTHR, 4) void xhc_pre_fused_kernel(XhcPreArgs a) {
  using T = typename E::T;
  constexpr int NTF = (2 * N + 15) / 16;
  constexpr int NPF = NTF * 16;
  constexpr int NA = K * K + K * KR;
  constexpr int NTA = (NA + 15) / 16;
  constexpr int NPA = NTA * 16;
  constexpr int P1 = TM * NPF + 2 * TM + 16;
  constexpr int P2 = TM * NPA + TM;
  constexpr int PMAX = P1 > P2 ? P1 : P2;
  constexpr int KB = E::KB, VEC = E::VEC;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int C = a.C, G = a.G;
  const int nkbC = C / KB;

  __shared__ int s_msg;
  __shared__ float s_red[WV][PMAX];
  __shared__ float s_hpre[TM][N];
  __shared__ float s_z[TM][N];
  __shared__ int s_idx[TM][K];

  if (tid == 0) s_msg = __hip_atomic_fetch_add(a.sync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int ticket = s_msg;
  const int tile = ticket / G, slice = ticket % G;
  const int t0 = tile * TM;
  const int tok = t0 + r;
  const bool tvalid = tok < a.T;
  int* cnt1 = a.sync + 2;
  int* ready = cnt1 + a.ntiles;
  int* cnt2 = ready + a.ntiles;

  // ---------------------------------------------------------------- phase 1
  const int kb0 = slice * (WV * NKW) + wave * NKW;   // first contraction block of this wave (within C)
  static_assert(P1 % 2 == 0 && P2 % 2 == 0, "partials are read in pairs");
  const T* __restrict__ X = reinterpret_cast<const T*>(a.X);
  const T* xt = X + (size_t)(tvalid ? tok : 0) * N * C + VEC * g;
  u32x4_t xd[N][NKW];
  const u32x4_t zero = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int q = 0; q < NKW; ++q) {
      const int kb = kb0 + q;
      xd[i][q] = (tvalid && kb < nkbC) ? ld16v(xt + (size_t)i * C + kb * KB) : zero;
    }

  f32x4_t acc[NTF];
#pragma unroll
  for (int n = 0; n < NTF; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t acs = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float s1 = 0.f, s2 = 0.f;
  const u32x4_t ones = ones_frag<E>();
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int q = 0; q < NKW; ++q) {
      const int kb = kb0 + q;
      if (kb < nkbC) {
        float f[VEC];
        E::unpack(xd[i][q], f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) { s1 += f[e]; s2 = fmaf(f[e], f[e], s2); }
        const u32x4_t* wp = reinterpret_cast<const u32x4_t*>(a.wfull) + ((size_t)(i * nkbC + kb) * NTF) * WAVE + lane;
#pragma unroll
        for (int n = 0; n < NTF; ++n) acc[n] = E::mma(acc[n], xd[i][q], wp[n * WAVE]);
        acs = E::mma(acs, ones, wp[0]);
      }
    }
  s1 += __shfl_xor(s1, 16, WAVE);
  s1 += __shfl_xor(s1, 32, WAVE);
  s2 += __shfl_xor(s2, 16, WAVE);
  s2 += __shfl_xor(s2, 32, WAVE);
#pragma unroll
  for (int n = 0; n < NTF; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_red[wave][(4 * g + i) * NPF + n * 16 + r] = acc[n][i];
  if (g == 0) {
    s_red[wave][TM * NPF + 2 * r] = s1;
    s_red[wave][TM * NPF + 2 * r + 1] = s2;
    s_red[wave][TM * NPF + 2 * TM + r] = acs[0];
  }
  __syncthreads();
  if (wave == 0) {
    float* dst = a.part1 + (size_t)ticket * P1;
    for (int u = lane; u < P1; u += WAVE) st_co(dst + u, sum_waves(s_red, u));
    wait_mem();
    if (lane == 0) s_msg = __hip_atomic_fetch_add(cnt1 + tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const bool last1 = s_msg == G - 1;

  // ---------------------------------------------------------------- phase 2
  if (last1) {
    sum_slices<NTHR, CP_SC1>(a.part1 + (size_t)tile * G * P1, G, P1, P1, &s_red[1][0], tid);
    __syncthreads();
    const float* sm = &s_red[1][0];
    const float n_el = (float)N * (float)C;
    for (int u = tid; u < TM * N; u += NTHR) {
      const int tau = u / N, i = u % N;
      route_logits(sm[tau * NPF + i], sm[tau * NPF + N + i], sm[TM * NPF + 2 * tau], sm[TM * NPF + 2 * tau + 1],
                   sm[TM * NPF + 2 * TM + i], n_el, a.eps, a.a_pre, a.b_pre[i], t0 + tau < a.T, &s_z[tau][i],
                   &s_hpre[tau][i]);
      // kept for a backward: the raw pre-map logit and the token's sums
      if (t0 + tau < a.T) {
        float* gs = a.gstat + (size_t)(t0 + tau) * (N + 2);
        gs[i] = sm[tau * NPF + N + i];
        if (i == 0) {
          gs[N] = sm[TM * NPF + 2 * tau];
          gs[N + 1] = sm[TM * NPF + 2 * tau + 1];
        }
      }
    }
    __syncthreads();
    if (tid < TM) {
      float zt[N];
#pragma unroll
      for (int i = 0; i < N; ++i) zt[i] = s_z[tid][i];
      int sel[K];
      route_select<N, K>(zt, a.m, sel);
#pragma unroll
      for (int j = 0; j < K; ++j) s_idx[tid][j] = sel[j];
    }
    __syncthreads();
    if (wave == 0) {
      for (int u = lane; u < TM * N; u += WAVE) {
        const int tau = u / N, i = u % N, t = t0 + tau;
        if (t < a.T) {
          st_co(a.z + (size_t)t * N + i, s_z[tau][i]);
          st_co(a.h_pre + (size_t)t * N + i, s_hpre[tau][i]);
        }
      }
      for (int u = lane; u < TM * K; u += WAVE) {
        const int tau = u / K, j = u % K, t = t0 + tau;
        if (t < a.T) {
          const int sel = s_idx[tau][j];
          st_co(a.idx + (size_t)t * K + j, sel);
          st_co(a.p + (size_t)t * K + j, j < a.m ? 1.f : sigmoidf_(s_z[tau][sel]));
        }
      }
      wait_mem();
      if (lane == 0) __hip_atomic_store(ready + tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    if (wave == 0) {
      if (lane == 0) wait_flag(ready + tile, a.sync + 1);
      const int rows = a.T - t0 < TM ? a.T - t0 : TM;
      const __amdgpu_buffer_rsrc_t rh = make_rsrc(a.h_pre + (size_t)t0 * N, (uint32_t)(rows * N * 4));
      const __amdgpu_buffer_rsrc_t ri = make_rsrc(a.idx + (size_t)t0 * K, (uint32_t)(rows * K * 4));
      for (int u = lane; u < TM * N; u += WAVE) {
        const int tau = u / N, t = t0 + tau;
        s_hpre[tau][u % N] = t < a.T ? ld_co(rh, (uint32_t)(u * 4)) : 0.f;
      }
      for (int u = lane; u < TM * K; u += WAVE) {
        const int tau = u / K, j = u % K, t = t0 + tau;
        const int v = t < a.T ? ld_co_i(ri, (uint32_t)(u * 4)) : j;
        s_idx[tau][j] = v < 0 ? 0 : (v >= N ? N - 1 : v);
      }
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- phase 3
  // Gather + active projection first, so that the partial can be published
  // before this wave's stores of the sublayer input are in flight.
  int I[K];
#pragma unroll
  for (int j = 0; j < K; ++j) I[j] = s_idx[r][j];
  f32x4_t acc2[NTA];
#pragma unroll
  for (int n = 0; n < NTA; ++n) acc2[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < NKW; ++q) {
    const int kb = kb0 + q;
    if (kb < nkbC) {
#pragma unroll
      for (int j = 0; j < K; ++j) {
        u32x4_t v = xd[0][q];
#pragma unroll
        for (int i = 1; i < N; ++i) v = (I[j] == i) ? xd[i][q] : v;
        float f[VEC];
        E::unpack(v, f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) ss = fmaf(f[e], f[e], ss);
        const u32x4_t* wp = reinterpret_cast<const u32x4_t*>(a.wact) + ((size_t)(j * nkbC + kb) * NTA) * WAVE + lane;
#pragma unroll
        for (int n = 0; n < NTA; ++n) acc2[n] = E::mma(acc2[n], v, wp[n * WAVE]);
      }
    }
  }
  ss += __shfl_xor(ss, 16, WAVE);
  ss += __shfl_xor(ss, 32, WAVE);
  __syncthreads();   // s_red of phase 1 fully consumed
#pragma unroll
  for (int n = 0; n < NTA; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_red[wave][(4 * g + i) * NPA + n * 16 + r] = acc2[n][i];
  if (g == 0) s_red[wave][TM * NPA + r] = ss;
  __syncthreads();
  if (wave == 0) {
    float* dst = a.part2 + (size_t)ticket * P2;
    for (int u = lane; u < P2; u += WAVE) st_co(dst + u, sum_waves(s_red, u));
    wait_mem();
    if (lane == 0) s_msg = __hip_atomic_fetch_add(cnt2 + tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // dense read over all N streams -> sublayer input
  T* __restrict__ inp = reinterpret_cast<T*>(a.inp);
#pragma unroll
  for (int q = 0; q < NKW; ++q) {
    const int kb = kb0 + q;
    if (kb < nkbC) {
      float o[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[e] = 0.f;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const float hpi = s_hpre[r][i];
        float f[VEC];
        E::unpack(xd[i][q], f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = fmaf(hpi, f[e], o[e]);
      }
      if (tvalid) st16_nt(inp + (size_t)tok * C + kb * KB + VEC * g, E::packv(o));
    }
  }
  __syncthreads();
  if (s_msg != G - 1) return;

  // last workgroup of the tile: active maps (K lanes per token, one row each)
  sum_slices<NTHR, CP_SC1>(a.part2 + (size_t)tile * G * P2, G, P2, P2, &s_red[0][0], tid);
  __syncthreads();
  if (wave == 0) {
    constexpr int TPP = WAVE / K;
    constexpr int PASSES = (TM + TPP - 1) / TPP;
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      const int tau = pass * TPP + lane / K;
      const int row = lane % K;
      const int t = t0 + tau;
      const bool valid = tau < TM && t < a.T;
      const int tq = tau < TM ? tau : 0;
      const float rr = 1.f / sqrtf(s_red[0][TM * NPA + tq] / ((float)K * (float)C) + a.eps);
      float L[K];
#pragma unroll
      for (int b = 0; b < K; ++b) {
        const int col = row * K + b;
        L[b] = fmaf(a.a_res * s_red[0][tq * NPA + col], rr, a.b_res[col]);
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
              2.f * sigmoidf_(fmaf(a.a_post * s_red[0][tq * NPA + col], rr, a.b_post[row * KR + q]));
        }
      }
    }
  }
}

// Weight packing into MFMA B fragments and reset of the tile counters.
// Fragment (kb, nt, lane = 16 g + col) holds W[kb*KB + VEC*g + e][nt*16 + col]
// for e < VEC (zero beyond the logical width).
template <class E>
__global__ __launch_bounds__(256) void xhc_prep_kernel(const typename E::T* __restrict__ Wf, long nkbf, int ncf,
                                                       int NTF, uint4* __restrict__ outf,
                                                       const typename E::T* __restrict__ Wa, long nkba, int nca,
                                                       int NTA, uint4* __restrict__ outa, int* __restrict__ sync,
                                                       int nsync) {
  using T = typename E::T;
  const long f = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (f < nsync) sync[f] = 0;
  const long nf = nkbf * NTF * WAVE, na = nkba * NTA * WAVE;
  const T* W;
  long ff;
  int ncol, NT;
  uint4* out;
  if (f < nf) {
    W = Wf; ff = f; ncol = ncf; NT = NTF; out = outf;
  } else if (f < nf + na) {
    W = Wa; ff = f - nf; ncol = nca; NT = NTA; out = outa;
  } else {
    return;
  }
  const int lane = (int)(ff % WAVE);
  const long rest = ff / WAVE;
  const int nt = (int)(rest % NT);
  const long kb = rest / NT;
  const int g = lane >> 4, col = nt * 16 + (lane & 15);
  union { T v[E::VEC]; uint4 u; } frag;
#pragma unroll
  for (int e = 0; e < E::VEC; ++e) {
    const long row = kb * E::KB + E::VEC * g + e;
    frag.v[e] = col < ncol ? W[row * ncol + col] : T(0);
  }
  out[ff] = frag.u;
}

template <class E, int N, int K, int KR>
static void launch_fused(const Plan& P, const XhcPreArgs& a, hipStream_t st) {
  xhc_pre_fused_kernel<E, N, K, KR><<<(unsigned)(a.ntiles * a.G), NTHR, 0, st>>>(a);
}

template <class E>
static bool xhc_pre_fused_launch(const Plan& P, const void* X, void* inp, const xhc_weights* w, char* ws,
                                 hipStream_t st) {
  XhcPreArgs a;
  a.X = X; a.inp = inp; a.T = (int)P.T; a.C = P.C; a.m = P.m; a.G = P.G; a.ntiles = P.ntiles;
  a.wfull = reinterpret_cast<const uint4*>(ws + P.o_wfull);
  a.wact = reinterpret_cast<const uint4*>(ws + P.o_wact);
  a.b_pre = w->b_pre; a.b_res = w->b_res; a.b_post = w->b_post;
  a.a_pre = w->alpha_pre; a.a_res = w->alpha_res; a.a_post = w->alpha_post;
  a.eps = P.eps_norm; a.iters = P.iters;
  a.part1 = reinterpret_cast<float*>(ws + P.o_part);
  a.part2 = reinterpret_cast<float*>(ws + P.o_part2);
  a.sync = reinterpret_cast<int*>(ws + P.o_sync);
  a.idx = reinterpret_cast<int*>(ws + P.o_idx);
  a.p = reinterpret_cast<float*>(ws + P.o_p);
  a.h_pre = reinterpret_cast<float*>(ws + P.o_hpre);
  a.h_res = reinterpret_cast<float*>(ws + P.o_hres);
  a.h_post = reinterpret_cast<float*>(ws + P.o_hpost);
  a.z = reinterpret_cast<float*>(ws + P.o_z);
  a.gstat = reinterpret_cast<float*>(ws + P.o_gstat);

  const int nsync = 2 + 3 * P.ntiles;
  const long nfrag = (P.nkb_full * P.NTF + P.nkb_act * P.NTA) * WAVE;
  const long nthreads = nfrag > nsync ? nfrag : nsync;
  using TT = typename E::T;
  xhc_prep_kernel<E><<<(unsigned)((nthreads + 255) / 256), 256, 0, st>>>(
      reinterpret_cast<const TT*>(w->w_full), P.nkb_full, P.ncol_full, P.NTF, reinterpret_cast<uint4*>(ws + P.o_wfull),
      reinterpret_cast<const TT*>(w->w_act), P.nkb_act, P.ncol_act, P.NTA, reinterpret_cast<uint4*>(ws + P.o_wact),
      a.sync, nsync);

  const int key = P.N * 100 + P.K * 10 + P.KR;
  switch (key) {
    case 1641: launch_fused<E, 16, 4, 1>(P, a, st); return true;
    case 1644: launch_fused<E, 16, 4, 4>(P, a, st); return true;
    case 1621: launch_fused<E, 16, 2, 1>(P, a, st); return true;
    case 1624: launch_fused<E, 16, 2, 4>(P, a, st); return true;
    case 841: launch_fused<E, 8, 4, 1>(P, a, st); return true;
    case 844: launch_fused<E, 8, 4, 4>(P, a, st); return true;
    case 441: launch_fused<E, 4, 4, 1>(P, a, st); return true;
    case 444: launch_fused<E, 4, 4, 4>(P, a, st); return true;
    case 111: launch_fused<E, 1, 1, 1>(P, a, st); return true;
    case 114: launch_fused<E, 1, 1, 4>(P, a, st); return true;
    default: return false;
  }
}

template <class E>
static void pack_launch(const Plan* Pf, const xhc_weights* wf, char* wsf, const Plan* Pa, const xhc_weights* wa,
                        char* wsa, const Plan* Pz, char* wsz, hipStream_t st) {
  using TT = typename E::T;
  const long nkbf = Pf ? Pf->nkb_full : 0, nkba = Pa ? Pa->nkb_act : 0;
  const int NTF = Pf ? Pf->NTF : 1, NTA = Pa ? Pa->NTA : 1;
  const int nsync = Pz ? 2 + 3 * (int)Pz->ntiles : 0;
  const long nfrag = (nkbf * NTF + nkba * NTA) * WAVE;
  const long nthreads = nfrag > nsync ? nfrag : nsync;
  if (nthreads == 0) return;
  xhc_prep_kernel<E><<<(unsigned)((nthreads + 255) / 256), 256, 0, st>>>(
      Pf ? reinterpret_cast<const TT*>(wf->w_full) : nullptr, nkbf, Pf ? Pf->ncol_full : 0, NTF,
      Pf ? reinterpret_cast<uint4*>(wsf + Pf->o_wfull) : nullptr, Pa ? reinterpret_cast<const TT*>(wa->w_act) : nullptr,
      nkba, Pa ? Pa->ncol_act : 0, NTA, Pa ? reinterpret_cast<uint4*>(wsa + Pa->o_wact) : nullptr,
      Pz ? reinterpret_cast<int*>(wsz + Pz->o_sync) : nullptr, nsync);
}

bool launch_pack(const Plan* Pf, const xhc_weights* wf, char* wsf, const Plan* Pa, const xhc_weights* wa, char* wsa,
                 const Plan* Pz, char* wsz, hipStream_t st) {
  const int dt = Pf ? Pf->dtype : Pa ? Pa->dtype : Pz ? Pz->dtype : XHC_BF16;
  if (dt == XHC_BF16)
    pack_launch<Bf16>(Pf, wf, wsf, Pa, wa, wsa, Pz, wsz, st);
  else
    pack_launch<F32>(Pf, wf, wsf, Pa, wa, wsa, Pz, wsz, st);
  return true;
}

#ifndef XHC_PRE_VIA_CHAIN_MIN_T
#define XHC_PRE_VIA_CHAIN_MIN_T 4096
#endif
// Large bf16 batches at N = 16, k > 2, m = 2, C a multiple of 128: the
// routing pass and the last-sublayer pre pass of the chained calls (both
// staged through LDS) instead of the one-pass kernel above, whose
// workgroups wait for each other's routing partials.
static bool pre_via_chain(const Plan& P) {
  return P.dtype == XHC_BF16 && P.N == 16 && P.K > 2 && P.m == 2 && P.C % 128 == 0 &&
         P.T >= XHC_PRE_VIA_CHAIN_MIN_T;
}

bool launch_xhc_pre(const Plan& P, const void* X, void* inp, const xhc_weights* w, char* ws, hipStream_t st) {
  if (pre_via_chain(P))
    return launch_xhc_route(P, X, w, ws, st) && launch_xhc_pre_chained(P, w, nullptr, nullptr, X, inp, ws, nullptr, st);
  return P.dtype == XHC_BF16 ? xhc_pre_fused_launch<Bf16>(P, X, inp, w, ws, st)
                             : xhc_pre_fused_launch<F32>(P, X, inp, w, ws, st);
}

}  // namespace xhc
