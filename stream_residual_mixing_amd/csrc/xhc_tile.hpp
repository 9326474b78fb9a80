// Building blocks of the tiled xHC kernels (gfx950): a tile is 16 tokens (the
// rows of an MFMA 16x16 block) times one channel slice; a workgroup is 8
// waves, each covering one contraction block of every stream.  Partial
// results of the slices of a tile are exchanged through memory.
#pragma once

#include "xhc_device.hpp"

namespace xhc {

constexpr int TM = 16;          // tokens per tile (MFMA rows)
constexpr int TWV = 8;          // waves per tile workgroup
constexpr int TNTHR = TWV * 64;

__device__ __forceinline__ u32x4_t ld16v(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ u32x4_t ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ void st16_nt(void* p, const u32x4_t& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

// Data exchanged between workgroups of one launch goes through
// device-coherent accesses: agent-scope atomic stores and loads (gfx950:
// global_store / global_load with the sc1 bit), which write through to, and
// read from, the level where all compute units agree.  A publisher stores its
// data this way, waits until every one of its memory operations has completed
// (s_waitcnt 0), and only then bumps the counter or sets the flag; a consumer
// polls the counter or flag, and reads the data with coherent loads issued
// after it has seen the flag.  This orders data before flag without an
// agent-scope release fence, which on this chip writes back the whole L2 and
// costs more than the rest of the kernel.
__device__ __forceinline__ void st_co(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_co(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Buffer resources (gfx9 V#: base, no stride, byte range): any read past the
// range returns zero instead of faulting, and independent loads through one
// are issued back to back.  Cache policy bits: sc1 (device-coherent, the same
// policy as the atomic loads above) and nt (streaming).  State reads use the
// default policy: a wave reads 64-byte halves of 128-byte lines whose other
// half a neighbouring wave reads moments later, and with nt the line tends to
// be gone by then (measured: the streaming hint made these kernels ~10%
// slower).
constexpr int CP_SC1 = 16;
constexpr int CP_NT = 2;
// A byte offset past any resource's range: loads from it return zero.
constexpr uint32_t OUT_OF_RANGE = 0x40000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
template <int AUX = 0>
__device__ __forceinline__ u32x4_t ld_b128(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff, (int)soff, AUX));
}
template <int AUX = 0>
__device__ __forceinline__ uint64_t ld_b64(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off) {
  return __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rs, (int)byte_off, 0, AUX));
}
__device__ __forceinline__ uint64_t ld_co64(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off) {
  return ld_b64<CP_SC1>(rs, byte_off);
}
__device__ __forceinline__ float ld_co(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (int)byte_off, 0, CP_SC1));
}
__device__ __forceinline__ int ld_co_i(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off) {
  return __builtin_bit_cast(int, __builtin_amdgcn_raw_buffer_load_b32(rs, (int)byte_off, 0, CP_SC1));
}

// Stores through a buffer resource: a store past its range is dropped.
// Kernels that prefetch across loop iterations store this way instead of
// under a branch: the compiler's memory-counter waits assume the fewest
// operations a branch may have issued, so a conditional store or load makes
// later waits cover the prefetched loads as well.
template <int AUX = 0>
__device__ __forceinline__ void st_b128(const u32x4_t& v, __amdgpu_buffer_rsrc_t rs, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rs, (int)voff, 0, AUX);
}
__device__ __forceinline__ void st_b32(float v, __amdgpu_buffer_rsrc_t rs, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, (int)voff, 0, 0);
}

// s_waitcnt vmcnt(n): at most n of this wave's vector memory operations
// still outstanding (they complete in issue order).
template <int NV>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(NV >= 0 && NV < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((NV & 15) | ((NV >> 4) << 14) | 0x0F70);
}
// Workgroup barrier of the passes that stage through LDS: this wave's LDS operations
// complete, at most NV of its vector memory operations outstanding (63: any
// number), then s_barrier.  It takes the place of __syncthreads, whose
// workgroup release fence also waits for every buffer-to-LDS load in flight,
// including those of tiles that no wave reads before a later barrier.  The
// empty asm statements keep the compiler from moving memory accesses across.
template <int NV>
__device__ __forceinline__ void stage_barrier() {
  static_assert(NV >= 0 && NV < 64, "vmcnt is 6 bits");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((NV & 15) | ((NV >> 4) << 14) | 0x0070);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait for all of this wave's outstanding memory operations.
__device__ __forceinline__ void wait_mem() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
}

// dst[u] = sum over s < G, in order s = 0, 1, ..., of src[s * stride + u], for
// u < n (n and stride even; two neighbouring elements per thread, read with
// one 8-byte load of policy AUX).  The loads of up to 16 slices are issued
// together, so the latency of fetching the partials is paid once per batch
// rather than once per slice.  NTHR threads take part.
template <int NTHR, int AUX>
__device__ __forceinline__ void sum_slices(const float* __restrict__ src, int G, int stride, int n,
                                           float* __restrict__ dst, int tid) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, (uint32_t)((size_t)G * stride * 4));
  for (int u = 2 * tid; u < n; u += 2 * NTHR) {
    float v0 = 0.f, v1 = 0.f;
    for (int s0 = 0; s0 < G; s0 += 16) {
      uint64_t x[16];
#pragma unroll
      for (int q = 0; q < 16; ++q)
        x[q] = s0 + q < G ? ld_b64<AUX>(rs, (uint32_t)(((s0 + q) * stride + u) * 4)) : 0ull;
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (s0 + q < G) {
          v0 += __uint_as_float((uint32_t)x[q]);
          v1 += __uint_as_float((uint32_t)(x[q] >> 32));
        }
    }
    dst[u] = v0;
    dst[u + 1] = v1;
  }
}

#ifndef XHC_FIN_AUX
#define XHC_FIN_AUX 2   // streaming loads of the slice partials in the finalize kernels (each read once; measured ~2% per chain step)
#endif
// v[0..1] += sum over s < G, in order s = 0, 1, ..., of the element pair at
// byte offset off + 4 s stride of the resource rs (whose range ends at slice
// G, so that slices past it read zero and add nothing; off = OUT_OF_RANGE
// adds zeros throughout).  The loads of SB slices go out unconditionally and
// together: with SB >= G the partials cost one memory round trip.
template <int SB>
__device__ __forceinline__ void add_slices2(__amdgpu_buffer_rsrc_t rs, int G, int stride, uint32_t off, float (&v)[2]) {
  for (int s0 = 0; s0 < G; s0 += SB) {
    uint64_t x[SB];
#pragma unroll
    for (int q = 0; q < SB; ++q) x[q] = ld_b64<XHC_FIN_AUX>(rs, off + (uint32_t)((s0 + q) * stride * 4));
#pragma unroll
    for (int q = 0; q < SB; ++q) {
      v[0] += __uint_as_float((uint32_t)x[q]);
      v[1] += __uint_as_float((uint32_t)(x[q] >> 32));
    }
  }
}

// Sum of the 8 per-wave partials of element u, in a fixed order.
template <int PM>
__device__ __forceinline__ float sum_waves(const float (&r)[TWV][PM], int u) {
  static_assert(TWV == 8, "fixed-order sum written for 8 waves");
  return ((r[0][u] + r[1][u]) + (r[2][u] + r[3][u])) + ((r[4][u] + r[5][u]) + (r[6][u] + r[7][u]));
}

// A fragment of 1.0 in every element (bf16 0x3f80, f32 0x3f800000)
template <class E> __device__ __forceinline__ u32x4_t ones_frag();
template <> __device__ __forceinline__ u32x4_t ones_frag<Bf16>() {
  return u32x4_t{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
}
template <> __device__ __forceinline__ u32x4_t ones_frag<F32>() {
  return u32x4_t{0x3f800000u, 0x3f800000u, 0x3f800000u, 0x3f800000u};
}

// Routing of a tile from its summed projection (one token per thread,
// tau < TM, i < N): LayerNorm-corrected router logits and H_pre.
//   raw   [TM][NPF]  columns 0..N-1: vec X . W_r, N..2N-1: vec X . W_pre
//   q1,q2 sum of x and of x^2 over the token's N*C elements
//   cs    column sums of W_r
// z = (raw_r - mu cs) / (sd + eps) (population sd), H_pre = sigmoid(alpha_pre
// raw_p / sqrt(mean x^2 + eps) + b_pre); padding tokens get H_pre = 0.
__device__ __forceinline__ void route_logits(float rr, float rp, float q1, float q2, float cs, float n_el,
                                             float eps, float a_pre, float b_pre, bool valid, float* z,
                                             float* hpre) {
  const float mu = q1 / n_el, nu = q2 / n_el;
  const float sd = sqrtf(fmaxf(nu - mu * mu, 0.f));
  const float rstd = 1.f / (sd + eps);
  const float rrms = 1.f / sqrtf(nu + eps);
  *z = (rr - mu * cs) * rstd;
  *hpre = valid ? sigmoidf_(fmaf(a_pre * rp, rrms, b_pre)) : 0.f;
}

// Fixed-m + routed top-(k-m) selection for one token: streams 0..m-1, then
// the k-m largest logits among streams m..N-1 in descending order, ties to the
// lower stream index.
template <int N, int K>
__device__ __forceinline__ void route_select(const float (&z)[N], int m, int (&sel)[K]) {
  uint32_t taken = 0;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    int s;
    if (j < m) {
      s = j;
    } else {
      int best = -1;
      float bz = 0.f;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const bool cand = (i >= m) && !((taken >> i) & 1u);
        if (cand && (best < 0 || z[i] > bz)) { best = i; bz = z[i]; }
      }
      s = best < 0 ? 0 : best;
    }
    taken |= 1u << s;
    sel[j] = s;
  }
}

}  // namespace xhc
