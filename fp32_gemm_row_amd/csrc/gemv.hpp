// Matrix-vector shaped product (M == 1): C[0,k] = sum_n A[0,n] * B[n,k].
//
// The pages give no kernel for this shape; it is legal (1 <= M in the LeetGPU
// "Constraints") and the LeetGPU "Example 2" is one. With a single output row
// there is nothing to reuse from B: each element of B is used once, so the
// kernel is bound by streaming B (N*K floats) from HBM, at 0.5 FLOP per byte.
//
// Design: workgroup w owns the 32 output columns [32w, 32w+32) - one 128-byte
// segment of every row of B - and the whole reduction for them. Its threads
// split the rows of B: LPR lanes cover the 32 columns of one row (8 lanes x
// float4 on the 128-bit path, 32 lanes x float on the 32-bit path) and the
// RPI = NT / LPR row groups walk rows r, r + RPI, r + 2 RPI, ...; the loop is
// unrolled so that each lane keeps UNROLL independent loads in flight (with
// NT = 1024 and UNROLL = 8 a workgroup has 1024 rows = 128 KiB of B in
// flight). A is staged through LDS in chunks of up to 8192 elements. The row
// groups' partial sums are first added across the lanes of each wave (lanes
// that share columns differ by multiples of LPR), then across waves in LDS.
// No atomics and no workspace: the result is deterministic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgr {

constexpr int kGemvCols = 32;       // output columns per workgroup
constexpr int kGemvAChunk = 8192;   // elements of A staged in LDS at a time

template <int VW, int NT, int UNROLL>
__global__ __launch_bounds__(NT) void gemv_kernel(const float* __restrict__ A,
                                                  const float* __restrict__ B,
                                                  float* __restrict__ C, int N, int K) {
  constexpr int LPR = kGemvCols / VW;  // lanes per row segment
  constexpr int RPI = NT / LPR;        // rows in flight per workgroup step
  constexpr int WAVES = NT / 64;
  static_assert(VW == 1 || VW == 4, "vector width");
  static_assert(NT % 64 == 0 && 64 % LPR == 0, "waves must hold whole row segments");

  __shared__ float a_s[kGemvAChunk];
  __shared__ float part[WAVES][kGemvCols];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int cl = tid % LPR;  // column lane
  const int rl = tid / LPR;  // row group
  const int col = blockIdx.x * kGemvCols + cl * VW;
  const bool col_ok = col < K;  // VW == 4: K % 4 == 0, so all four columns are in

  float acc[VW];
#pragma unroll
  for (int e = 0; e < VW; ++e) acc[e] = 0.f;

  for (int nb = 0; nb < N; nb += kGemvAChunk) {
    const int len = (N - nb) < kGemvAChunk ? (N - nb) : kGemvAChunk;
    __syncthreads();  // the previous chunk of A has been read by every thread
    for (int i = tid; i < len; i += NT) a_s[i] = A[nb + i];
    __syncthreads();
    if (col_ok) {
      const float* bp = B + (int64_t)nb * K + col;
#pragma unroll UNROLL
      for (int r = rl; r < len; r += RPI) {
        const float a = a_s[r];
        if constexpr (VW == 4) {
          const float4 v = *reinterpret_cast<const float4*>(bp + (int64_t)r * K);
          acc[0] += a * v.x;
          acc[1] += a * v.y;
          acc[2] += a * v.z;
          acc[3] += a * v.w;
        } else {
          acc[0] += a * bp[(int64_t)r * K];
        }
      }
    }
  }

  // lanes cl, cl + LPR, cl + 2 LPR, ... of a wave hold the same columns
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < VW; ++e) acc[e] += __shfl_xor(acc[e], off);
  if (lane < LPR) {
#pragma unroll
    for (int e = 0; e < VW; ++e) part[wave][cl * VW + e] = acc[e];
  }
  __syncthreads();
  if (tid < kGemvCols) {
    const int c = blockIdx.x * kGemvCols + tid;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) s += part[w][tid];
    if (c < K) C[c] = s;
  }
}

}  // namespace fgr
