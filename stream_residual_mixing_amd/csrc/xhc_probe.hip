// Measurement helper: the achievable HBM read rate on this device.
//
// Not part of the layer.  bench.py times it next to the layer's kernels so
// that each kernel's rate can be compared with what a plain stream of 16-byte
// loads reaches on the same GPU.  Each thread reads 16-byte vectors with a
// grid-wide stride, UNROLL of them in flight, folds them into one word, and
// each workgroup writes one word so that no load can be removed.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "xhc.h"
#include "xhc_internal.hpp"

namespace xhc {

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
constexpr int PROBE_THREADS = 256;
constexpr int PROBE_UNROLL = 8;

template <bool NT>
__global__ __launch_bounds__(PROBE_THREADS) void probe_read_kernel(const v4u* __restrict__ src, size_t n,
                                                                  uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * PROBE_THREADS;
  size_t i = (size_t)blockIdx.x * PROBE_THREADS + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (PROBE_UNROLL - 1) * stride < n; i += PROBE_UNROLL * stride) {
    v4u v[PROBE_UNROLL];
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u)
      v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const v4u v = NT ? __builtin_nontemporal_load(src + i) : src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t s[PROBE_THREADS];
  s[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int t = 0; t < PROBE_THREADS; ++t) a ^= s[t];
    sink[blockIdx.x] = a;
  }
}

}  // namespace

bool launch_probe_read(const void* src, size_t bytes, uint32_t* sink, int mode, hipStream_t st) {
  const size_t n = bytes / 16;
  const unsigned grid = PROBE_SINK_WORDS;
  if (mode == 0)
    probe_read_kernel<false><<<grid, PROBE_THREADS, 0, st>>>(static_cast<const v4u*>(src), n, sink);
  else
    probe_read_kernel<true><<<grid, PROBE_THREADS, 0, st>>>(static_cast<const v4u*>(src), n, sink);
  return true;
}

}  // namespace xhc
