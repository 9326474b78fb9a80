// Device-side building blocks shared by the libxhc kernels (gfx950 only).
//
// Fragments: every global load or store of state data moves 16 bytes per
// lane (8 bf16 or 4 float).  The full-state and active-state projections
// run on MFMA 16x16 tiles with the state rows as the A operand (16 tokens
// per tile, one token per lane row) and the weights, pre-packed, as the B
// operand, so one 16-byte fragment of a state row is one MFMA step's worth
// of contraction for its lane group.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xhc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// 16-byte fragment as a native vector (register arrays of it stay in VGPRs)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}
// The same two roundings by gfx950's conversion instruction v_cvt_pk_bf16_f32
// (round to nearest even, NaN stays NaN; the same bits).  One instruction for
// two values, no branch for the NaN case; used by the persistent chained
// kernels, where it measured faster.  Not the default: in the one-pass pre
// kernel the compiler's register allocation then spilled.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2_cvt(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }

// ---------------------------------------------------------------------------
// Element types.  VEC = elements per 16-byte fragment; KB = contraction length
// covered by one fragment per lane group (4 lane groups x VEC).
// ---------------------------------------------------------------------------
struct Bf16 {
  using T = uint16_t;
  static constexpr int VEC = 8;
  static constexpr int KB = 32;
  __device__ static __forceinline__ void unpack(const uint4& v, float (&f)[8]) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  }
  __device__ static __forceinline__ uint4 pack(const float (&f)[8]) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                      pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
  }
  __device__ static __forceinline__ f32x4_t mma(f32x4_t acc, const uint4& a, const uint4& b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
  __device__ static __forceinline__ void unpack(const u32x4_t& v, float (&f)[8]) {
    f[0] = bf16_lo(v[0]); f[1] = bf16_hi(v[0]); f[2] = bf16_lo(v[1]); f[3] = bf16_hi(v[1]);
    f[4] = bf16_lo(v[2]); f[5] = bf16_hi(v[2]); f[6] = bf16_lo(v[3]); f[7] = bf16_hi(v[3]);
  }
  __device__ static __forceinline__ u32x4_t packv(const float (&f)[8]) {
    return u32x4_t{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                   pack_bf16x2(f[6], f[7])};
  }
  __device__ static __forceinline__ u32x4_t packv_cvt(const float (&f)[8]) {
    return u32x4_t{pack_bf16x2_cvt(f[0], f[1]), pack_bf16x2_cvt(f[2], f[3]), pack_bf16x2_cvt(f[4], f[5]),
                   pack_bf16x2_cvt(f[6], f[7])};
  }
  __device__ static __forceinline__ f32x4_t mma(f32x4_t acc, const u32x4_t& a, const u32x4_t& b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
};

struct F32 {
  using T = float;
  static constexpr int VEC = 4;
  static constexpr int KB = 16;
  __device__ static __forceinline__ void unpack(const uint4& v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ uint4 pack(const float (&f)[4]) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                      __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
  __device__ static __forceinline__ f32x4_t mma(f32x4_t acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
    return acc;
  }
  __device__ static __forceinline__ void unpack(const u32x4_t& v, float (&f)[4]) {
    f[0] = __uint_as_float(v[0]); f[1] = __uint_as_float(v[1]);
    f[2] = __uint_as_float(v[2]); f[3] = __uint_as_float(v[3]);
  }
  __device__ static __forceinline__ u32x4_t packv(const float (&f)[4]) {
    return u32x4_t{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
  }
  __device__ static __forceinline__ u32x4_t packv_cvt(const float (&f)[4]) { return packv(f); }
  __device__ static __forceinline__ f32x4_t mma(f32x4_t acc, const u32x4_t& a, const u32x4_t& b) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[s]), __uint_as_float(b[s]), acc, 0, 0, 0);
    return acc;
  }
};

// Small vectors of 4 channels used by the post kernels (native vector types,
// so that register arrays of them are not demoted to scratch memory).
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
template <class E> struct Quad;
template <> struct Quad<Bf16> {
  using V = u32x2_t;   // 4 bf16
  __device__ static __forceinline__ void unpack(const V& v, float (&f)[4]) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  }
  __device__ static __forceinline__ V pack(const float (&f)[4]) {
    return V{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])};
  }
};
template <> struct Quad<F32> {
  using V = f32x4_t;
  __device__ static __forceinline__ void unpack(const V& v, float (&f)[4]) {
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
  }
  __device__ static __forceinline__ V pack(const float (&f)[4]) {
    return V{f[0], f[1], f[2], f[3]};
  }
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// Sum over a full wave (64 lanes); every lane receives the same value.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// Sum / max over aligned groups of G lanes (G a power of two <= 64).  The
// xor butterfly gives every lane of a group the bitwise-same result.
template <int G> __device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = G / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
template <int G> __device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = G / 2; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

// Sinkhorn-Knopp on an R x R matrix held one row per lane in groups of R
// lanes: exponentiate after subtracting the matrix maximum, then `iters`
// times normalise columns, then rows (explainer "xHC: sixteen residual
// streams, four written at a time", section "mHC: keep the mixing doubly
// stochastic").  IEEE float division throughout.
template <int R>
__device__ __forceinline__ void sinkhorn_rows(float (&m)[R], int iters) {
  float mx = m[0];
#pragma unroll
  for (int b = 1; b < R; ++b) mx = fmaxf(mx, m[b]);
  mx = group_max<R>(mx);
#pragma unroll
  for (int b = 0; b < R; ++b) m[b] = expf(m[b] - mx);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int b = 0; b < R; ++b) m[b] = m[b] / group_sum<R>(m[b]);
    float rs = 0.f;
#pragma unroll
    for (int b = 0; b < R; ++b) rs += m[b];
#pragma unroll
    for (int b = 0; b < R; ++b) m[b] = m[b] / rs;
  }
}

}  // namespace xhc
