// Second pass of a reduction split across workgroups: C[i] = W[0][i] +
// W[1][i] + ... + W[parts - 1][i], added in part order (so the result does not
// depend on which workgroup finished first). W holds `parts` partial copies of
// C back to back. Bound by HBM: parts + 1 floats moved per output.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgr {

constexpr int kReduceThreads = 256;

// VW = 4: n % 4 == 0 and W, C 16-byte aligned
template <int VW>
__global__ __launch_bounds__(kReduceThreads) void reduce_parts_kernel(const float* __restrict__ W,
                                                                      float* __restrict__ C, int64_t n,
                                                                      int parts) {
  typedef typename std::conditional<VW == 4, float4, float>::type V;
  const int64_t nv = n / VW;
  const V* w = reinterpret_cast<const V*>(W);
  V* c = reinterpret_cast<V*>(C);
  const int64_t stride = (int64_t)gridDim.x * kReduceThreads;
  for (int64_t i = (int64_t)blockIdx.x * kReduceThreads + threadIdx.x; i < nv; i += stride) {
    V s = w[i];
    for (int p = 1; p < parts; ++p) {
      const V v = w[p * nv + i];
      if constexpr (VW == 4) {
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
      } else {
        s += v;
      }
    }
    c[i] = s;
  }
}

}  // namespace fgr
