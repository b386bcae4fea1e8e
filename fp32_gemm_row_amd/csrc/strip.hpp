// The narrow column strip of a product, on the vector ALUs.
//
// When K is a few columns past a multiple of 64 (K = 64 q + w, 1 <= w <= 8)
// and the q full column blocks of 64 x 64 tiles give every CU at most one
// tile, the last w columns would otherwise cost a whole extra column of
// mostly-padding tiles, i.e. a second partial wave of tiles. Instead the
// k-split kernel's launch holds, after its tiles' workgroups, workgroups that
// run strip_rows: C[m, c0 + j] = sum over n of A[m,n] B[n, c0 + j], c0 = 64
// q, j < w, each a plain FP32 dot product (the per-output loop of the LeetGPU
// write-up's naive kernel, section "V0", spread over a wave's lanes). Two
// workgroups fit a CU, so these run beside the tiles, whose matrix cores they
// leave alone.
//
// A workgroup takes four rows of A, one per wave. It stages B's strip (rows
// nb .. nb + len - 1, columns c0 .. K - 1, column by column) in the LDS it is
// given, read once for its four rows; lane l then takes reduction
// indices nb + 4 l + 256 u .. + 3 of its row (one 16-byte load each, for
// which 4-byte alignment suffices), keeping w partial sums. The
// lanes' sums are added across the wave (xor shuffles: every lane ends with
// the same bits) and lane j stores column c0 + j. Every loop issues its loads
// (kStripLoads per thread, or more) before it uses any of them: one at a time,
// each use would wait out a full memory round trip before the next load.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_mfma.hpp"

namespace fgr {

constexpr int kStripMax = 8;    // widest strip (columns)
constexpr int kStripRows = 4;   // rows of A per workgroup (one per wave of 256 threads)
constexpr int kStripLoads = 8;  // loads each thread keeps in flight

// Rows kStripRows b .. kStripRows b + 3 of the strip (rows past M idle but
// take part in the barriers). stage: lds_floats floats of LDS, 16-byte
// aligned, at least 68 kStripMax, overwritten.
__device__ __forceinline__ void strip_rows(const float* __restrict__ A, const float* __restrict__ B,
                                           float* __restrict__ C, int M, int N, int K, int c0, int b, float* stage,
                                           int lds_floats) {
  const int tid = threadIdx.x;
  const int m = b * kStripRows + (tid >> 6);
  const int lane = tid & 63;
  const bool row_ok = m < M;
  const int w = K - c0;  // 1 .. kStripMax
  // B's strip is staged column by column: rows nb .. nb + len - 1 of column
  // c0 + j at stage[j * pitch + (n - nb)], zeros after them up to a multiple
  // of 4 rows, so that a lane reads its four consecutive rows of a column
  // with one 16-byte LDS read, the lanes' reads side by side (no bank
  // conflicts; row-major staging put the lanes 4 w floats apart, a 32-way
  // conflict at w = 8). pitch = 4 mod 64 spreads the staging writes of the
  // columns over the banks.
  const int pitch = (((lds_floats / w) - 4) & ~63) + 4;  // rows of B's strip staged at a time
  const float* a = A + (int64_t)(row_ok ? m : 0) * N;
  float acc[kStripMax];
#pragma unroll
  for (int j = 0; j < kStripMax; ++j) acc[j] = 0.f;
  constexpr int kRowQuads = kStripLoads / 2;  // 16-byte loads of A per lane per round
  for (int nb = 0; nb < N; nb += pitch) {
    const int len = N - nb < pitch ? N - nb : pitch;
    const int len4 = (len + 3) & ~3;
    __syncthreads();  // the previous chunk has been read by every wave
    const int total = len4 * w;
    for (int i0 = tid; i0 < total; i0 += 64 * kStripRows * kStripLoads) {
      float v[kStripLoads];
#pragma unroll
      for (int u = 0; u < kStripLoads; ++u) {
        const int i = i0 + u * 64 * kStripRows;
        const int n = i / w;
        v[u] = i < total && n < len ? B[(int64_t)(nb + n) * K + c0 + (i - n * w)] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kStripLoads; ++u) {
        const int i = i0 + u * 64 * kStripRows;
        const int n = i / w;
        if (i < total) stage[(i - n * w) * pitch + n] = v[u];
      }
    }
    __syncthreads();
    if (row_ok) {
      // lane l: elements n = nb + 4 l + 256 u .. n + 3 of its row, one 16-byte
      // load each (4-byte alignment suffices), element by element at the end
      for (int n0 = nb + 4 * lane; n0 < nb + len; n0 += 256 * kRowQuads) {
        float4 v[kRowQuads];
#pragma unroll
        for (int u = 0; u < kRowQuads; ++u) {
          const int n = n0 + 256 * u;
          if (n + 3 < nb + len) {
            v[u] = load_dwords<float4>(a + n);
          } else {
            float e[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) e[q] = n + q < nb + len ? a[n + q] : 0.f;
            v[u] = make_float4(e[0], e[1], e[2], e[3]);
          }
        }
#pragma unroll
        for (int u = 0; u < kRowQuads; ++u) {
          const int r = n0 + 256 * u - nb;  // a multiple of 4
          if (r < len) {
#pragma unroll
            for (int j = 0; j < kStripMax; ++j)
              if (j < w) {
                const float4 bq = *reinterpret_cast<const float4*>(stage + j * pitch + r);
                acc[j] += ((v[u].x * bq.x + v[u].y * bq.y) + v[u].z * bq.z) + v[u].w * bq.w;
              }
          }
        }
      }
    }
  }
  if (!row_ok) return;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)
#pragma unroll
    for (int j = 0; j < kStripMax; ++j) acc[j] += __shfl_xor(acc[j], off);
  float mine = 0.f;
#pragma unroll
  for (int j = 0; j < kStripMax; ++j)
    if (lane == j) mine = acc[j];
  if (lane < w) C[(int64_t)m * K + c0 + lane] = mine;
}

}  // namespace fgr
