// FP32 GEMM on the vector ALUs (no matrix cores): C[M,K] = A[M,N] x B[N,K],
// row-major. This is the register-tiled line that "LeetGPU |
// 02_Matrix_Multiplication" develops on CUDA cores (sections "V1:
// Two-Dimensional Thread Tiling", "V2: Vectorized float4 Transfers", "V2
// Control: Vectorized Single Buffer (128 x 128)" and "V3: Register Prefetch
// and Double-Buffered Shared Memory"), re-designed for CDNA4 wave64, as an
// A/B reference against the MFMA kernels:
//
//  * a workgroup of 256 threads (four waves) owns a 128 x 128 tile of C and
//    the whole reduction; thread (ty, tx) of the 16 x 16 thread grid owns an
//    8 x 8 micro-tile as four 4 x 4 blocks: rows 4ty + i and 64 + 4ty + i,
//    columns 4tx + j and 64 + 4tx + j (i, j < 4);
//  * per reduction index n the thread reads 8 values of A and 8 of B from LDS
//    (four 128-bit reads) and does the 64 FMAs of their outer product into
//    64 FP32 accumulators (the outer-product view of the V1 2-D section);
//  * the reduction advances in chunks of BK: the next chunk of A and B is
//    loaded into registers (128-bit loads, 32-bit when rows are not 16-byte
//    aligned) while the current one is consumed from LDS, then written to the
//    other of two LDS buffers - one barrier per chunk (the V3 section's
//    register prefetch and double buffer);
//  * A is stored k-major in LDS (As[n][m], pitch BM + 4) so that the 4 rows
//    of a block are one 128-bit read; B row-major (Bs[n][k], pitch BN). In a
//    wave the 16 lanes of one thread row read the same A address (broadcast)
//    and the 16 thread columns read 256 contiguous bytes of B: no bank
//    conflicts on the reads;
//  * out-of-range rows, columns and reduction indices are zero-filled and
//    never loaded; stores are guarded by row < M, col < K.
//
// Plain (unpacked) FP32 FMAs only (v_fmac_f32; packed FP32 ops are disabled
// for the whole library). Each output is a single FMA chain over n = 0, 1,
// ..., N-1 in order. 8-deep chunks: the compiler hoists a chunk's LDS reads
// ahead of its FMAs (214 VGPRs, two waves per SIMD); 16-deep ones pushed it
// past 256 VGPRs into AGPR copies.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_mfma.hpp"  // xcd_remap, grouped_tile

namespace fgr {

constexpr int kValuBM = 128;
constexpr int kValuBN = 128;
constexpr int kValuThreads = 256;

template <int BK_, bool VEC_>
struct ValuConfig {
  static constexpr int BM = kValuBM, BN = kValuBN, BK = BK_;
  static constexpr bool VEC = VEC_;
  static constexpr int kPitchA = BM + 4;             // floats per k-row of As
  static constexpr int kAQuads = BK / 4;             // 4-float pieces per row of the A chunk
  static constexpr int kALoads = BM * BK / 4 / kValuThreads;  // per thread and chunk
  static constexpr int kBLoads = BK * BN / 4 / kValuThreads;
  static_assert(BK % 4 == 0 && kALoads >= 1 && kBLoads >= 1, "chunk shape");
};

template <class T>
__global__ __launch_bounds__(kValuThreads) void gemm_valu_kernel(const float* __restrict__ A,
                                                                 const float* __restrict__ B,
                                                                 float* __restrict__ C, int M, int N, int K,
                                                                 int tiles_m, int tiles_n, int group) {
  constexpr int BM = T::BM, BN = T::BN, BK = T::BK, PA = T::kPitchA;
  __shared__ __attribute__((aligned(16))) float As[2][BK * PA];
  __shared__ __attribute__((aligned(16))) float Bs[2][BK * BN];

  const int tid = threadIdx.x;
  const int tx = tid % 16;
  const int ty = tid / 16;

  int tm, tn;
  grouped_tile(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, group, tm, tn);
  const int m0 = tm * BM;
  const int k0 = tn * BN;

  // Load slots. A: slot f covers row f / kAQuads of the chunk, reduction
  // offsets 4 (f % kAQuads) .. +3; B: row f / (BN / 4), columns 4 (f % (BN / 4)) .. +3.
  const float* a_src[T::kALoads];
  bool a_row_ok[T::kALoads];
  int a_n[T::kALoads], a_m[T::kALoads];
#pragma unroll
  for (int j = 0; j < T::kALoads; ++j) {
    const int f = tid + j * kValuThreads;
    a_m[j] = f / T::kAQuads;
    a_n[j] = 4 * (f % T::kAQuads);
    a_row_ok[j] = m0 + a_m[j] < M;
    a_src[j] = A + (int64_t)(a_row_ok[j] ? m0 + a_m[j] : 0) * N + a_n[j];
  }
  const float* b_src[T::kBLoads];
  int b_n[T::kBLoads], b_k[T::kBLoads];
#pragma unroll
  for (int j = 0; j < T::kBLoads; ++j) {
    const int f = tid + j * kValuThreads;
    b_n[j] = f / (BN / 4);
    b_k[j] = 4 * (f % (BN / 4));
    b_src[j] = B + (k0 + b_k[j]);
  }

  float4 ra[T::kALoads], rb[T::kBLoads];
  // chunk starting at reduction index n0 into registers, zero outside the matrix
  auto load_chunk = [&](int n0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < T::kALoads; ++j) {
      const int n = n0 + a_n[j];
      if constexpr (T::VEC) {
        // N % 4 == 0: the four indices are all inside or all outside
        ra[j] = a_row_ok[j] && n < N ? *reinterpret_cast<const float4*>(a_src[j] + n0)
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
      } else {
        const float* p = a_src[j] + n0;
        ra[j].x = a_row_ok[j] && n < N ? p[0] : 0.f;
        ra[j].y = a_row_ok[j] && n + 1 < N ? p[1] : 0.f;
        ra[j].z = a_row_ok[j] && n + 2 < N ? p[2] : 0.f;
        ra[j].w = a_row_ok[j] && n + 3 < N ? p[3] : 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < T::kBLoads; ++j) {
      const int n = n0 + b_n[j];
      const int k = k0 + b_k[j];
      const float* p = b_src[j] + (int64_t)(n < N ? n : 0) * K;
      if constexpr (T::VEC) {
        // K % 4 == 0: the four columns are all inside or all outside
        rb[j] = n < N && k < K ? *reinterpret_cast<const float4*>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
      } else {
        rb[j].x = n < N && k < K ? p[0] : 0.f;
        rb[j].y = n < N && k + 1 < K ? p[1] : 0.f;
        rb[j].z = n < N && k + 2 < K ? p[2] : 0.f;
        rb[j].w = n < N && k + 3 < K ? p[3] : 0.f;
      }
    }
  };
  auto store_chunk = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < T::kALoads; ++j) {
      float* d = As[buf] + a_n[j] * PA + a_m[j];
      d[0] = ra[j].x;
      d[PA] = ra[j].y;
      d[2 * PA] = ra[j].z;
      d[3 * PA] = ra[j].w;
    }
#pragma unroll
    for (int j = 0; j < T::kBLoads; ++j)
      *reinterpret_cast<float4*>(Bs[buf] + b_n[j] * BN + b_k[j]) = rb[j];
  };

  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

  const int nchunks = (N + BK - 1) / BK;
  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    if (c + 1 < nchunks) load_chunk((c + 1) * BK);
    const float* as = As[buf];
    const float* bs = Bs[buf];
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      const float4 a0 = *reinterpret_cast<const float4*>(as + kk * PA + 4 * ty);
      const float4 a1 = *reinterpret_cast<const float4*>(as + kk * PA + 64 + 4 * ty);
      const float4 b0 = *reinterpret_cast<const float4*>(bs + kk * BN + 4 * tx);
      const float4 b1 = *reinterpret_cast<const float4*>(bs + kk * BN + 64 + 4 * tx);
      const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    if (c + 1 < nchunks) {
      // the other buffer was last read in chunk c - 1, before the barrier
      // that ended it
      store_chunk(buf ^ 1);
      __syncthreads();
    }
  }

  // rows 4ty + i (i < 4) and 64 + 4ty + i; columns 4tx + j and 64 + 4tx + j
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = m0 + (i < 4 ? 4 * ty + i : 64 + 4 * ty + i - 4);
    if (row >= M) continue;
    float* crow = C + (int64_t)row * K;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int col = k0 + 64 * h + 4 * tx;
      if constexpr (T::VEC) {
        if (col < K)
          *reinterpret_cast<float4*>(crow + col) =
              make_float4(acc[i][4 * h], acc[i][4 * h + 1], acc[i][4 * h + 2], acc[i][4 * h + 3]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (col + j < K) crow[col + j] = acc[i][4 * h + j];
      }
    }
  }
}

}  // namespace fgr
