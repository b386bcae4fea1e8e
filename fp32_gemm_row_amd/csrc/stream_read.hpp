// Streaming-read ceiling: the plainest HBM-bound kernel, for measurement.
//
// Every float of X is read once with a 128-bit load and added into a per-lane
// sum; each workgroup writes the sum of its lanes to out[workgroup], so that
// no load is dead code. Over a buffer several times the size of the
// last-level cache (256 MB on MI355X) its rate is the read bandwidth a kernel
// that streams an operand once (the matrix-vector path) can reach in practice,
// against the 8 TB/s of the datasheet. The study notes "CUDA 学习笔记 Matrix
// Multiplication", section 2, bound the product's time by its bytes moved; this
// kernel measures what one byte of reading costs on this device.
//
// Grid-stride over float4 indices: workgroup b, thread t starts at b * 256 +
// t and steps by the grid's thread count, UNROLL loads issued before any is
// used. The loads are non-temporal (each float is read once), as in the
// matrix-vector kernel: over 1 GiB on MI355X ordinary loads reach about
// 6.4 TB/s, non-temporal ones about 7.1. The order of the additions does not
// matter (the sums are never checked beyond being finite).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgr {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;

typedef float sr_f32x4 __attribute__((ext_vector_type(4)));

// A non-temporal 128-bit load: the data streams through the caches (each
// float is read once), which on MI355X is the faster way to read HBM.
__device__ __forceinline__ float4 stream_load(const float4* p) {
  const sr_f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const sr_f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const float4* __restrict__ X, int64_t n4,
                                                                     float* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  float acc = 0.f;
  for (; i + (kStreamUnroll - 1) * stride < n4; i += kStreamUnroll * stride) {
    float4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = stream_load(X + i + u * stride);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
  }
  for (; i < n4; i += stride) {
    const float4 v = stream_load(X + i);
    acc += (v.x + v.y) + (v.z + v.w);
  }
  // the workgroup's sum: across each wave's lanes, then the four waves in LDS
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  __shared__ float wave_sum[kStreamThreads / 64];
  if ((threadIdx.x & 63) == 0) wave_sum[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kStreamThreads / 64; ++w) s += wave_sum[w];
    out[blockIdx.x] = s;
  }
}

}  // namespace fgr
