// Second pass of a reduction split across workgroups: C[i] = the sum over p
// of W[p][i], where W holds `parts` partial copies of C back to back. Bound by
// HBM: (parts + 1) x 4 bytes moved per output.
//
// A workgroup of 256 threads covers 256 / slices outputs (vectors of VW
// floats); the `slices` threads of an output each add a contiguous run of
// parts, [parts s / slices, parts (s + 1) / slices), in part order, four
// loads in flight, and the run sums are then added in slice order through
// LDS. The order is fixed by (parts, slices), so the result is the same on
// every run; on integer-valued data every order gives the exact sum.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_mfma.hpp"  // grouped_tile

namespace fgr {

constexpr int kReduceThreads = 256;
constexpr int kReduceMaxSlices = 16;

template <class V>
__device__ __forceinline__ V add_vec(V a, V b) {
  if constexpr (std::is_same<V, float4>::value) return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
  else return a + b;
}

// VW = 4: n % 4 == 0 and W, C 16-byte aligned. slices: a power of two in
// [1, 16], at most parts (every run holds at least one part).
template <int VW>
__global__ __launch_bounds__(kReduceThreads) void reduce_parts_kernel(const float* __restrict__ W,
                                                                      float* __restrict__ C, int64_t n,
                                                                      int parts, int slices) {
  typedef typename std::conditional<VW == 4, float4, float>::type V;
  __shared__ V run_sum[kReduceThreads];
  const int64_t nv = n / VW;
  const V* w = reinterpret_cast<const V*>(W);
  V* c = reinterpret_cast<V*>(C);
  const int opw = kReduceThreads / slices;  // outputs per workgroup
  const int o = threadIdx.x % opw;
  const int s = threadIdx.x / opw;
  const int64_t i = (int64_t)blockIdx.x * opw + o;
  if (i < nv) {
    const int p0 = parts * s / slices;
    const int p1 = parts * (s + 1) / slices;
    V acc = w[(int64_t)p0 * nv + i];
    int p = p0 + 1;
    for (; p + 4 <= p1; p += 4) {
      const V a = w[(int64_t)p * nv + i];
      const V b = w[(int64_t)(p + 1) * nv + i];
      const V d = w[(int64_t)(p + 2) * nv + i];
      const V e = w[(int64_t)(p + 3) * nv + i];
      acc = add_vec(add_vec(add_vec(add_vec(acc, a), b), d), e);
    }
    for (; p < p1; ++p) acc = add_vec(acc, w[(int64_t)p * nv + i]);
    run_sum[threadIdx.x] = acc;
  }
  __syncthreads();
  if (s == 0 && i < nv) {
    V r = run_sum[o];
    for (int q = 1; q < slices; ++q) r = add_vec(r, run_sum[q * opw + o]);
    c[i] = r;
  }
}

// The same for partial tiles in compact slots: tiles [first, first + count)
// of a tiles_m x tiles_n grid of BT x BT tiles in the grouped order, part p of
// tile t in slot p count + t (BT x BT floats, row stride BT). Block (x, t)
// covers 256 elements of tile t; each thread adds the parts of one element
// in part order, four loads in flight, and stores it if it lies in C.
template <int BT>
__global__ __launch_bounds__(kReduceThreads) void reduce_tiles_kernel(const float* __restrict__ W,
                                                                      float* __restrict__ C, int M, int K,
                                                                      int parts, int tiles_m, int tiles_n,
                                                                      int group, int first, int count) {
  static_assert(BT * BT % kReduceThreads == 0, "whole blocks per tile");
  const int t = blockIdx.y;
  const int e = blockIdx.x * kReduceThreads + threadIdx.x;
  int tm, tn;
  grouped_tile(first + t, tiles_m, tiles_n, group, tm, tn);
  const int row = tm * BT + e / BT;
  const int col = tn * BT + e % BT;
  if (row >= M || col >= K) return;
  const int64_t stride = (int64_t)count * BT * BT;
  const float* w = W + (int64_t)t * BT * BT + e;
  float acc = w[0];
  int p = 1;
  for (; p + 4 <= parts; p += 4) {
    const float a = w[p * stride], b = w[(p + 1) * stride], d = w[(p + 2) * stride], f = w[(p + 3) * stride];
    acc = (((acc + a) + b) + d) + f;
  }
  for (; p < parts; ++p) acc += w[p * stride];
  C[(int64_t)row * K + col] = acc;
}

}  // namespace fgr
