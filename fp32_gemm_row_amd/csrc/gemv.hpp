// Matrix-vector and skinny products (M <= 8): C[m,k] = sum_n A[m,n] * B[n,k].
//
// The pages give no kernel for this shape; it is legal (1 <= M in the LeetGPU
// "Constraints") and the LeetGPU "Example 2" is one. With one (or a few)
// output rows there is (almost) nothing to reuse from B: each element of B is
// used M times, so the kernel is bound by streaming B (N*K floats) from HBM,
// at 0.5 * M FLOP per byte.
//
// Design: workgroup w owns the 32 output columns [32w, 32w+32) - one 128-byte
// segment of every row of B (16 columns, 64 bytes, where K is too small to
// give every CU a 32-column block) - and the whole reduction for them, for all MR
// (>= M) rows of A. Its threads split the rows of B: LPR lanes cover the 32
// columns of one row (8 lanes x float4 on the 128-bit path, 32 lanes x float
// on the 32-bit path) and the RPI = NT / LPR row groups walk rows r, r + RPI,
// r + 2 RPI, ...; each lane loads UNROLL rows before it uses them (UNROLL
// loads in flight per lane). With one row of A (M == 1) each lane reads its
// A[n] straight from global memory beside its row of B (measured at
// 1 x 8192 x 8192: 43.0 us against 45.9 with A staged first). With more
// rows, A is staged through LDS, row-major, AF elements at a time (AF / MR
// reduction indices of every row); rows of A past M are staged as zeros and
// their outputs are not stored. The row groups' partial sums are first added across the lanes of
// each wave (lanes that share columns differ by multiples of LPR), then across
// waves in LDS, in wave order. No atomics: the result is deterministic, and
// for M == 1 the reduction order is that of MR == 1 for every MR. When K has
// too few 32-column blocks to occupy the CUs, the rows of B are also split
// into parts over a second grid dimension (below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_mfma.hpp"  // xcd_remap
#include "timestamps.hpp"

namespace fgr {

constexpr int kGemvCols = 32;        // output columns per workgroup
constexpr int kGemvMaxRows = 8;      // largest M the kernel takes
constexpr int kGemvAFloats = 16384;  // elements of A staged in LDS at a time (all rows)

typedef float f32x4 __attribute__((ext_vector_type(4)));

// One row segment of B. Every element of B is read once, so the loads are
// non-temporal: they stream through the caches without displacing lines that
// are reused (A). (For a plain streaming read on MI355X, non-temporal loads
// reach about 7.1 TB/s against about 6.4 for ordinary ones; here the gain is
// within the noise.)
template <int VW>
__device__ __forceinline__ void load_row(const float* p, float (&v)[VW]) {
  if constexpr (VW == 4) {
    const f32x4 q = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    v[0] = q.x;
    v[1] = q.y;
    v[2] = q.z;
    v[3] = q.w;
  } else {
    v[0] = __builtin_nontemporal_load(p);
  }
}

// acc[m][e] += A[m][r] * v[e] for the MR staged rows of A
template <int VW, int MR, int CHUNK>
__device__ __forceinline__ void fma_row(float (&acc)[MR][VW], const float* a_s, int r, const float (&v)[VW]) {
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    const float a = a_s[m * CHUNK + r];
#pragma unroll
    for (int e = 0; e < VW; ++e) acc[m][e] += a * v[e];
  }
}

// Split across workgroups (parts > 1): workgroup row blockIdx.y = part owns
// the reduction indices [N part / parts, N (part + 1) / parts) and writes its
// partial rows to W + part M K instead of C; a second kernel adds the parts in
// order (for K too small to give every CU its 32 columns).
template <int VW, int NT, int UNROLL, int MR, int AF = kGemvAFloats, int COLS = kGemvCols>
__global__ __launch_bounds__(NT) void gemv_kernel(const float* __restrict__ A,
                                                  const float* __restrict__ B,
                                                  float* __restrict__ C, int M, int N, int K, int parts,
                                                  float* __restrict__ W) {
  constexpr int LPR = COLS / VW;          // lanes per row segment
  constexpr int RPI = NT / LPR;           // rows in flight per workgroup step
  constexpr int WAVES = NT / 64;
  constexpr int CHUNK = AF / MR;          // reduction indices per staged chunk of A
  static_assert(VW == 1 || VW == 4, "vector width");
  static_assert(NT % 64 == 0 && 64 % LPR == 0, "waves must hold whole row segments");
  static_assert(MR >= 1 && MR <= kGemvMaxRows && AF % MR == 0 && (AF / MR) % RPI == 0, "rows per workgroup");

  __shared__ float a_s[MR == 1 ? 1 : MR * CHUNK];  // [m][n - nb] (M > 1: A is staged)
  __shared__ float part[WAVES][MR][COLS];

  TsMarks ts;  // measurement build only (timestamps.hpp)
  ts.start();
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int cl = tid % LPR;  // column lane
  const int rl = tid / LPR;  // row group
  // column block: consecutive blocks on one XCD (with 16-column blocks two
  // of them share each 128-byte line of B, which its L2 then fetches once)
  const int cb = xcd_remap(blockIdx.x, gridDim.x);
  const int col = cb * COLS + cl * VW;
  const bool col_ok = col < K;  // VW == 4: K % 4 == 0, so all four columns are in

  float acc[MR][VW];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int e = 0; e < VW; ++e) acc[m][e] = 0.f;

  const int n_lo = (int)((int64_t)N * blockIdx.y / parts);
  const int n_hi = (int)((int64_t)N * (blockIdx.y + 1) / parts);
  float* const Out = parts > 1 ? W + (int64_t)blockIdx.y * M * K : C;
  if constexpr (MR == 1) {
    // One row of A: each lane reads A[n] for its own rows of B straight from
    // global memory (4N bytes that every workgroup reads, so they stay in
    // L2), beside its load of the row of B. Nothing is staged and no barrier
    // holds back the stream of B at the start. The rows are visited in the
    // same order as on the staged path, so the sums are the same.
    if (col_ok) {
      const float* bp = B + (int64_t)n_lo * K + col;
      const float* ap = A + n_lo;
      const int len = n_hi - n_lo;
      for (int r = rl; r < len; r += RPI) {
        float v[VW];
        load_row<VW>(bp + (int64_t)r * K, v);
        const float a = ap[r];
#pragma unroll
        for (int e = 0; e < VW; ++e) acc[0][e] += a * v[e];
      }
    }
  } else {
    for (int nb = n_lo; nb < n_hi; nb += CHUNK) {
      const int len = (n_hi - nb) < CHUNK ? (n_hi - nb) : CHUNK;
      __syncthreads();  // the previous chunk of A has been read by every thread
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const bool row_ok = m < M;
        const float* ar = A + (int64_t)(row_ok ? m : 0) * N + nb;
        for (int i = tid; i < len; i += NT) a_s[m * CHUNK + i] = row_ok ? ar[i] : 0.f;
      }
      __syncthreads();
      if (col_ok) {
        const float* bp = B + (int64_t)nb * K + col;
        // UNROLL rows of B are loaded before any is used, so that each lane
        // keeps UNROLL loads in flight whatever MR is
        int r = rl;
        for (; r + (UNROLL - 1) * RPI < len; r += UNROLL * RPI) {
          float v[UNROLL][VW];
#pragma unroll
          for (int u = 0; u < UNROLL; ++u) load_row<VW>(bp + (int64_t)(r + u * RPI) * K, v[u]);
#pragma unroll
          for (int u = 0; u < UNROLL; ++u) fma_row<VW, MR, CHUNK>(acc, a_s, r + u * RPI, v[u]);
        }
        for (; r < len; r += RPI) {
          float v[VW];
          load_row<VW>(bp + (int64_t)r * K, v);
          fma_row<VW, MR, CHUNK>(acc, a_s, r, v);
        }
      }
    }
  }

  ts.loop_done();
  // lanes cl, cl + LPR, cl + 2 LPR, ... of a wave hold the same columns
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int e = 0; e < VW; ++e) acc[m][e] += __shfl_xor(acc[m][e], off);
  if (lane < LPR) {
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int e = 0; e < VW; ++e) part[wave][m][cl * VW + e] = acc[m][e];
  }
  __syncthreads();
  for (int t = tid; t < MR * COLS; t += NT) {
    const int m = t / COLS;
    const int cc = t % COLS;
    const int c = cb * COLS + cc;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) s += part[w][m][cc];
    if (m < M && c < K) Out[(int64_t)m * K + c] = s;
  }
  ts.finish();
}

}  // namespace fgr
