// libxhc kernels for gfx950.
//
// mHC pre stage (mapping generation + dense read):
//   pack_b      weights -> MFMA B fragments (once per call, a few MiB)
//   proj_gen    one pass over X: split-K bf16/f32 MFMA projection of the raw
//               (un-normalised) flattened state, plus sum x and sum x^2
//   mhc_proj    the same for the wide maps (N >= 8, bf16: 2N + N^2 columns),
//               256 tokens per workgroup with the weights staged in LDS
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
#include "xhc_tile.hpp"

// contraction blocks a proj_gen lane loads ahead (measured: 4 and 8 within
// 2% of each other, 16 slower)
#ifndef XHC_GEN_U
#define XHC_GEN_U 4
#endif

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

#ifndef XHC_MHC_READ_NT
#define XHC_MHC_READ_NT 1
#endif
// a 16-byte load of state the dense read uses once (streaming: measured ~5%
// faster for the mHC read pass than the default policy)
__device__ __forceinline__ uint4 ld_x(const void* p) {
  if constexpr (XHC_MHC_READ_NT) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
  } else {
    return ld16(p);
  }
}

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

  // dense read: a wave takes one token at a time and its lanes cover 64
  // consecutive 16-byte pieces of each stream, so every load instruction reads
  // 1 KiB of contiguous state (whole 128-byte lines)
  constexpr int VEC = E::VEC;
  constexpr int U = 2;                       // channel chunks of 64 VEC in flight
  const int chunk = WAVE * VEC;
  for (int tau = wave; tau < RT; tau += 4) {
    const int t = t0 + tau;
    if (t >= a.T) break;
    float hp[N];
#pragma unroll
    for (int i = 0; i < N; ++i) hp[i] = s_hpre[tau][i];
    const T* xt = X + (size_t)t * N * C;
    for (int c0 = lane * VEC; c0 < C; c0 += U * chunk) {
      uint4 v[U][N];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < N; ++i)
          v[u][i] = c0 + u * chunk < C ? ld_x(xt + (size_t)i * C + c0 + u * chunk) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (c0 + u * chunk >= C) break;
        float o[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = 0.f;
#pragma unroll
        for (int i = 0; i < N; ++i) {
          float f[VEC];
          E::unpack(v[u][i], f);
#pragma unroll
          for (int e = 0; e < VEC; ++e) o[e] = fmaf(hp[i], f[e], o[e]);
        }
        st16(inp + (size_t)t * C + c0 + u * chunk, E::pack(o));
      }
    }
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
// mhc_proj: the wide mHC projection, raw[t][0..ncol) = vec X_t . W_full, with
// sum x and sum x^2, for bf16 state at N >= 8 (ncol = 2N + N^2: 288 columns
// at N = 16).  It is a real GEMM ([T x NC] . [NC x ncol], ~290 flop per byte
// of X at N = 16), so the weights must be reused across many tokens:
//   - a workgroup owns MP_TOK = 256 tokens and every column, over one of KS
//     contraction ranges; each wave owns MP_RT consecutive 16-row MFMA tiles
//     of them and holds their MP_RT x NT accumulators;
//   - the packed weight fragments of MP_KU contraction blocks at a time go
//     from global memory straight into LDS (double-buffered, one barrier per
//     stage) and are read by all eight waves; the state goes straight from
//     HBM into A fragments, one stage ahead;
//   - workgroup b takes range b mod KS, so the workgroups sharing an XCD (and
//     its L2) walk the same weight range.
// X is read once.  Partials per (range, token), summed by mhc_read.
// ---------------------------------------------------------------------------
#ifndef XHC_MHC_KU
#define XHC_MHC_KU 2   // measured: 2 best of 1, 2, 3, 4
#endif
#ifndef XHC_MHC_RT
#define XHC_MHC_RT 2
#endif
#ifndef XHC_MHC_BD
#define XHC_MHC_BD 4
#endif
#ifndef XHC_MHC_STAGED
#define XHC_MHC_STAGED 1   // the state staged through LDS, two stages ahead
#endif
#ifndef XHC_MHC_STATE_AUX
#define XHC_MHC_STATE_AUX 2   // cache policy of the staged state loads (whole 128-byte lines: streaming)
#endif
constexpr int MP_KU = XHC_MHC_KU;              // contraction blocks per LDS stage
constexpr int MP_BD = XHC_MHC_BD;              // weight fragments in registers (read ahead)
constexpr int MP_RT = XHC_MHC_RT;              // 16-token MFMA row tiles per wave
constexpr int MP_THREADS = 512 * 2 / MP_RT;    // 8 waves of 2 tiles or 4 waves of 4
constexpr int MP_TOK = MP_THREADS / 64 * 16 * MP_RT;   // 256 tokens per workgroup

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int NT>
__global__ __launch_bounds__(MP_THREADS, 1) void mhc_proj_kernel(const uint16_t* __restrict__ X, int T, long K,
                                                                 const uint4* __restrict__ Wp, long nkb, int KS,
                                                                 float* __restrict__ part, float* __restrict__ stats) {
  constexpr int CH = MP_KU * NT;                  // 1 KiB weight fragments per stage
  constexpr int NW = MP_THREADS / WAVE;
  // the two weight buffers are separate LDS arrays, so that the compiler
  // tells a read of one from the loads into the other
  __shared__ u32x4_t s_w0[MP_KU][NT][WAVE];
  __shared__ u32x4_t s_w1[MP_KU][NT][WAVE];
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = blockIdx.x % KS, tile = blockIdx.x / KS;
  const long kb0 = (long)ks * nkb / KS, kb1 = (long)(ks + 1) * nkb / KS;
  const int t0 = tile * MP_TOK;
  const int rows = T - t0 < MP_TOK ? T - t0 : MP_TOK;
  // the workgroup's rows only: loads past T read zeros
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(X + (size_t)t0 * K, (uint32_t)((size_t)rows * K * 2));
  const uint32_t voff0 = (uint32_t)(((size_t)(wave * 16 * MP_RT + r) * K + 8 * g) * 2);

  f32x4_t acc[MP_RT][NT];
  float s1[MP_RT], s2[MP_RT];   // token r of each tile, over this lane's 8 of 32 columns
#pragma unroll
  for (int h = 0; h < MP_RT; ++h) {
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[h][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    s1[h] = 0.f;
    s2[h] = 0.f;
  }

  // The weight fragments of the stage starting at kbs, straight from memory
  // into LDS buffer buf (each lane 16 bytes of a 1 KiB fragment), through a
  // resource over the packed weights: fragments past the last block read
  // zero.  Past this split's range the stage only loads what it will not use.
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(Wp, (uint32_t)((size_t)nkb * NT * WAVE * 16));
  // Fragment c = wave + NW q; a wave whose last q falls past CH loads the last
  // fragment again (the same bytes to the same place), so that every wave
  // issues the same, compile-time number of loads.
  auto load_w = [&](long kbs, auto bc) __attribute__((always_inline)) {
    u32x4_t* wb = decltype(bc)::value == 0 ? &s_w0[0][0][0] : &s_w1[0][0][0];
#pragma unroll
    for (int q = 0; q < (CH + NW - 1) / NW; ++q) {
      const int c = wave + NW * q < CH ? wave + NW * q : CH - 1;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr_t)(wb + (size_t)c * WAVE), 16,
                                               (int)(((kbs * NT + c) * WAVE + lane) * 16), 0, 0, 0);
    }
  };
  // A fragments of a stage; blocks past this split's range read zero (and
  // so add nothing to the sums and the MFMAs).  No load sits under a branch:
  // the compiler's memory-counter waits would then also cover the next
  // stage's loads.
  auto load_a = [&](long kbs, u32x4_t (&a)[MP_RT][MP_KU]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < MP_KU; ++k) {
      const uint32_t o = kbs + k < kb1 ? (uint32_t)((kbs + k) * 64) : OUT_OF_RANGE;
#pragma unroll
      for (int h = 0; h < MP_RT; ++h) a[h][k] = ld_b128(rx, voff0 + (uint32_t)(h * 16 * K * 2) + o, 0);
    }
  };
  // One stage: issue the next stage's weights (to the other buffer, last read
  // in the previous stage, before its barrier) and state, then the MFMAs of
  // this one.  Before the barrier each wave waits for its weight loads only;
  // the state loads issued after them stay in flight into the next stage.
  constexpr int WAIT_W = (MP_RT * MP_KU) | (0x7 << 4) | (0xF << 8);   // vmcnt(MP_RT * MP_KU)
  static_assert(MP_RT * MP_KU < 16, "the wait count fits the low vmcnt bits");
  auto stage = [&](long kbs, auto bc, const u32x4_t (&acur)[MP_RT][MP_KU], u32x4_t (&anext)[MP_RT][MP_KU])
      __attribute__((always_inline)) {
    constexpr int buf = decltype(bc)::value;
    const u32x4_t(&sw)[MP_KU][NT][WAVE] = buf == 0 ? s_w0 : s_w1;
    load_w(kbs + MP_KU, std::integral_constant<int, buf ^ 1>{});
    load_a(kbs + MP_KU, anext);
#pragma unroll
    for (int k = 0; k < MP_KU; ++k) {
#pragma unroll
      for (int h = 0; h < MP_RT; ++h) {
        float f[8];
        Bf16::unpack(acur[h][k], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s1[h] += f[e];
          s2[h] = fmaf(f[e], f[e], s2[h]);
        }
      }
      // weight fragments read MP_BD - 1 tiles ahead of their MFMAs, so the
      // LDS latency hides behind the MFMAs of the tiles before
      u32x4_t b[MP_BD];
#pragma unroll
      for (int q = 0; q < MP_BD - 1 && q < NT; ++q) b[q] = sw[k][q][lane];
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if (n + MP_BD - 1 < NT) b[(n + MP_BD - 1) % MP_BD] = sw[k][n + MP_BD - 1][lane];
#pragma unroll
        for (int h = 0; h < MP_RT; ++h) acc[h][n] = Bf16::mma(acc[h][n], acur[h][k], b[n % MP_BD]);
        __builtin_amdgcn_sched_barrier(0);   // keep each read ahead of the MFMAs before its use
      }
    }
    __builtin_amdgcn_s_waitcnt(WAIT_W);
    __syncthreads();
  };

  if constexpr (XHC_MHC_STAGED) {
    // The state through LDS: a stage's rows of the workgroup (256 tokens x
    // 2 blocks x 64 B) go from HBM into one slot of a two-stage ring with
    // buffer-to-LDS loads of 8 rows x 128 B.  A stage reads its A fragments
    // from its slot into registers first; once every wave is past those
    // reads the slot takes the state of the stage two on, while the other
    // slot's (issued a stage earlier) completes.  The slots are separate LDS
    // arrays, so the compiler tells a read of one from the loads into the
    // other, and the barriers are stage_barrier, without the release fence
    // that would wait for those loads.
    static_assert(MP_KU == 2 && NW * MP_RT * 16 == MP_TOK, "a stage is 256 rows x 128 B");
    constexpr int NDB = MP_TOK / 8;           // 1 KiB loads per stage
    constexpr int LPW = NDB / NW;             // per wave
    static_assert(NDB % NW == 0, "the loads of a stage split evenly over the waves");
    __shared__ u32x4_t s_a0[NDB][WAVE];
    __shared__ u32x4_t s_a1[NDB][WAVE];
    const int lr = lane >> 3, ls = lane & 7;
    // load d covers rows 8 d .. 8 d + 7 of the workgroup (half d mod 2 of
    // tile d / 2); lane l takes row 8 d + l / 8 and, at slot l mod 8, the
    // 16-byte chunk (l mod 8) xor ((row within the tile) / 2 mod 8) of its
    // 128 bytes (chunk c: block c / 4, lane group c mod 4).  Blocks past
    // this split's range read zero.
    auto dma_a = [&](long kbs, auto qc) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < LPW; ++u) {
        const int d = wave * LPW + u;
        const int rr = (d & 1) * 8 + lr, row = d * 8 + lr;
        const int c = ls ^ ((rr >> 1) & 7);
        const long blk = kbs + (c >> 2);
        const uint32_t off =
            blk < kb1 ? (uint32_t)((size_t)row * K * 2 + (size_t)blk * 64 + (size_t)(c & 3) * 16) : OUT_OF_RANGE;
        u32x4_t* dst = decltype(qc)::value == 0 ? &s_a0[d][0] : &s_a1[d][0];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_ptr_t)dst, 16, (int)off, 0, 0, XHC_MHC_STATE_AUX);
      }
    };
    // lane (g, r)'s fragment of tile h, block k: row r, chunk 4 k + g
    auto afrag = [&](const char* sa, int h, int k) __attribute__((always_inline)) {
      const int ti = wave * MP_RT + h;
      return *reinterpret_cast<const u32x4_t*>(sa + ti * 2048 + r * 128 + (((4 * k + g) ^ ((r >> 1) & 7)) << 4));
    };
    auto stage_s = [&](long kbs, auto qc) __attribute__((always_inline)) {
      constexpr int q = decltype(qc)::value;
      const char* sa = reinterpret_cast<const char*>(q == 0 ? &s_a0[0][0] : &s_a1[0][0]);
      const u32x4_t(&sw)[MP_KU][NT][WAVE] = q == 0 ? s_w0 : s_w1;
      u32x4_t acur[MP_RT][MP_KU];
#pragma unroll
      for (int h = 0; h < MP_RT; ++h)
#pragma unroll
        for (int k = 0; k < MP_KU; ++k) acur[h][k] = afrag(sa, h, k);
      stage_barrier<63>();   // every wave is past its reads of this slot
      load_w(kbs + MP_KU, std::integral_constant<int, q ^ 1>{});
      dma_a(kbs + 2 * MP_KU, qc);
#pragma unroll
      for (int k = 0; k < MP_KU; ++k) {
#pragma unroll
        for (int h = 0; h < MP_RT; ++h) {
          float f[8];
          Bf16::unpack(acur[h][k], f);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            s1[h] += f[e];
            s2[h] = fmaf(f[e], f[e], s2[h]);
          }
        }
        u32x4_t b[MP_BD];
#pragma unroll
        for (int qq = 0; qq < MP_BD - 1 && qq < NT; ++qq) b[qq] = sw[k][qq][lane];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          if (n + MP_BD - 1 < NT) b[(n + MP_BD - 1) % MP_BD] = sw[k][n + MP_BD - 1][lane];
#pragma unroll
          for (int h = 0; h < MP_RT; ++h) acc[h][n] = Bf16::mma(acc[h][n], acur[h][k], b[n % MP_BD]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // the next stage's weights (this stage's loads) and state (the
      // previous stage's) are in: all but this stage's state loads
      stage_barrier<LPW>();
    };
    load_w(kb0, Q0{});
    dma_a(kb0, Q0{});
    dma_a(kb0 + MP_KU, Q1{});
    stage_barrier<LPW>();
    // two stages per trip; a stage past the range reads zero fragments and
    // adds nothing
    for (long kbs = kb0; kbs < kb1; kbs += 2 * MP_KU) {
      stage_s(kbs, Q0{});
      stage_s(kbs + MP_KU, Q1{});
    }
    wait_vmcnt<0>();   // no load into LDS outlives the workgroup
  } else {
    u32x4_t a0[MP_RT][MP_KU], a1[MP_RT][MP_KU];
    load_w(kb0, Q0{});
    load_a(kb0, a0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (long kbs = kb0; kbs < kb1; kbs += 2 * MP_KU) {
      stage(kbs, Q0{}, a0, a1);
      if (kbs + MP_KU >= kb1) break;
      stage(kbs + MP_KU, Q1{}, a1, a0);
    }
  }
  constexpr int NP = NT * 16;
#pragma unroll
  for (int h = 0; h < MP_RT; ++h) {
    // the four lane groups of token r hold its four column groups
    s1[h] += __shfl_xor(s1[h], 16, WAVE);
    s1[h] += __shfl_xor(s1[h], 32, WAVE);
    s2[h] += __shfl_xor(s2[h], 16, WAVE);
    s2[h] += __shfl_xor(s2[h], 32, WAVE);
    const int tb = t0 + wave * 16 * MP_RT + h * 16;
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = tb + 4 * g + i;
        if (t < T) part[((size_t)ks * T + t) * NP + n * 16 + r] = acc[h][n][i];
      }
    if (g == 0 && tb + r < T) {
      stats[((size_t)ks * T + tb + r) * 2 + 0] = s1[h];
      stats[((size_t)ks * T + tb + r) * 2 + 1] = s2[h];
    }
  }
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
  launch_pack<E>(w->w_full, P.nkb_full, P.ncol_full, P.NTF, ws + P.o_wfull, st);
  if (P.mhc_wide) {
    const long ntile = (P.T + MP_TOK - 1) / MP_TOK;
    const unsigned grid = (unsigned)(ntile * P.KS);
    const uint16_t* Xb = reinterpret_cast<const uint16_t*>(X);
    const uint4* Wp = reinterpret_cast<const uint4*>(ws + P.o_wfull);
    float* part = reinterpret_cast<float*>(ws + P.o_part);
    float* stats = reinterpret_cast<float*>(ws + P.o_stats);
    const long K = (long)P.N * P.C;
    switch (P.NTF) {
      case 18: mhc_proj_kernel<18><<<grid, MP_THREADS, 0, st>>>(Xb, (int)P.T, K, Wp, P.nkb_full, P.KS, part, stats); break;
      case 5: mhc_proj_kernel<5><<<grid, MP_THREADS, 0, st>>>(Xb, (int)P.T, K, Wp, P.nkb_full, P.KS, part, stats); break;
      default: return false;
    }
  } else if (!gen_dispatch<E>(P.NTF, X, (int)P.T, (long)P.N * P.C, ws + P.o_wfull, P.nkb_full, P.KS,
                              reinterpret_cast<float*>(ws + P.o_part), reinterpret_cast<float*>(ws + P.o_stats), st)) {
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
