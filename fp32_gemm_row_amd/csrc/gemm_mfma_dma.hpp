// FP32 MFMA GEMM for whole tiles, fed by direct global->LDS loads.
//
// Same product, tiling and operand layout as gemm_mfma.hpp, for rows that are
// 16-byte aligned (N % 4 == 0, K % 4 == 0, aligned bases) and N >= 64. Every
// reduction chunk but the first is copied from global memory straight into
// LDS with global_load_lds_dwordx4 (16 bytes per lane, written to LDS at the
// M0 base + 16 * lane), the gfx950 counterpart of the cp.async copies of the
// LeetGPU write-up's section "V4: Hardware-Asynchronous cp.async Pipeline".
// That data never passes through VGPRs, so the copies do not compete with the
// MFMAs for register-file bandwidth, and no LDS write instructions are issued.
//
// Ragged edges. Rows of A beyond M and columns of B beyond K only feed
// outputs that are never stored, so their copies read a clamped in-bounds
// address (the last row / last column quad) and the epilogue guards the
// stores. Reduction indices beyond N would feed real outputs and must be
// zero: the chunks are aligned to the END of the reduction (chunk c covers
// n in [N - BK*(T - c), N - BK*(T - c) + BK), T = ceil(N / BK)), so that only
// chunk 0 can reach below n = 0; chunk 0 is loaded through registers with
// every element outside [0, N) set to zero (the zero padding of the study
// notes' section 4) and written to LDS in the same layout.
//
// LDS layout (two stages, each a separate LDS object so that the compiler can
// tell reads of one stage from copies into the other):
//   A stage: BM rows x BK floats, unpadded; row r holds its BK/4 quads in the
//     order q ^ swz(r), swz(r) = (r mod 8) ^ (bit 3 of r). One copy
//     instruction fills 8 consecutive rows (BK = 32). The MFMA operand read of
//     lane (i, g) fetches quad 2h + g of row i; over any 8 consecutive rows
//     from a multiple of 8, and over 16 from a multiple of 16, the swizzle
//     sends these reads to distinct 16-byte bank groups (32 or 64 banks).
//   B stage: BK rows x BN floats, row-major; one copy instruction per row.
#pragma once

#include "gemm_mfma.hpp"

namespace fgr {

typedef __attribute__((address_space(3))) void lds_void_t;

template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct DmaConfig {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static constexpr int kThreads = WM * WN * 64;
  static constexpr int kWaves = WM * WN;
  static constexpr int kWaveM = BM / WM;
  static constexpr int kWaveN = BN / WN;
  static constexpr int kRB = kWaveM / 32;
  static constexpr int kCB = kWaveN / 32;
  static constexpr int kQuads = BK / 4;                   // quads per A row
  static constexpr int kRowsPerCopy = 64 / kQuads;        // A rows per copy instruction
  static constexpr int kACopies = BM / kRowsPerCopy / kWaves;  // per wave per chunk
  static constexpr int kBCopies = BK / kWaves;            // B rows per wave per chunk
  static constexpr int kAStage = BM * BK;                 // floats
  static constexpr int kBStage = BK * BN;

  static_assert(BN == 256, "one B copy instruction covers a 256-float row");
  static_assert(BK == 32, "the A swizzle is written for 8 quads per row");
  static_assert(kCB == 2 || kCB == 4, "B operands are read as 2 or 4 adjacent floats");
  static_assert(kWaveM % 32 == 0 && kWaveN % 32 == 0, "wave tile must be a multiple of 32x32");
  static_assert(BM % (kRowsPerCopy * kWaves) == 0 && BK % kWaves == 0, "copies split evenly over waves");
  static_assert(4 * 2 * (kAStage + kBStage) <= 160 * 1024, "LDS budget of a gfx950 workgroup");
};

__device__ __forceinline__ int a_swizzle(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// 16 bytes per lane from global memory into LDS at lds + 16 * lane (lds is
// wave-uniform). A plain device function: the builtin has no host form.
__device__ __forceinline__ void copy16_to_lds(const float* g, float* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds, 16, 0, 0);
}

template <class T>
__global__ __launch_bounds__(T::kThreads) void gemm_mfma_dma_kernel(
    const float* __restrict__ A, const float* __restrict__ B, float* __restrict__ C, int M, int N,
    int K, int tiles_m, int tiles_n, int group) {
  constexpr int BM = T::BM, BK = T::BK, WN = T::WN;
  constexpr int H = BK / 8;
  __shared__ __attribute__((aligned(1024))) float As0[T::kAStage];
  __shared__ __attribute__((aligned(1024))) float As1[T::kAStage];
  __shared__ __attribute__((aligned(1024))) float Bs0[T::kBStage];
  __shared__ __attribute__((aligned(1024))) float Bs1[T::kBStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform (scalar): the LDS destination of a copy goes to M0
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int li = lane & 31;
  const int lg = lane >> 5;

  int tm, tn;
  grouped_tile(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, group, tm, tn);
  const int m0 = tm * BM;
  const int k0 = tn * T::BN;

  // Copy sources for this lane. A copy j of this wave fills rows
  // [R, R + 8), R = 8 * (wave * kACopies + j): lane L lands in row R + L / 8
  // at stored position L % 8, which holds quad (L % 8) ^ swz(row). Rows past
  // M read row M - 1 instead (their outputs are not stored).
  const float* a_src[T::kACopies];
  int a_dst[T::kACopies];  // LDS float offset of the copy's 1 KiB block
  int a_quad[T::kACopies];
#pragma unroll
  for (int j = 0; j < T::kACopies; ++j) {
    const int blk = wave * T::kACopies + j;
    const int r = blk * T::kRowsPerCopy + lane / T::kQuads;
    const int q = (lane % T::kQuads) ^ a_swizzle(r);
    const int row = m0 + r < M ? m0 + r : M - 1;
    a_src[j] = A + (int64_t)row * N + 4 * q;
    a_dst[j] = blk * 256;
    a_quad[j] = q;
  }
  // B copy j of this wave fills chunk row wave * kBCopies + j; lane L copies
  // columns 4L .. 4L + 3 (past K: the last quad instead, not stored).
  const float* b_src[T::kBCopies];
  int b_dst[T::kBCopies];
  const int b_col = k0 + 4 * lane < K ? k0 + 4 * lane : K - 4;
#pragma unroll
  for (int j = 0; j < T::kBCopies; ++j) {
    const int r = wave * T::kBCopies + j;
    b_src[j] = B + (int64_t)r * K + b_col;
    b_dst[j] = r * T::BN;
  }

  auto copy_chunk = [&](int n0, float* As, float* Bs) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < T::kACopies; ++j)
      copy16_to_lds(a_src[j] + n0, As + a_dst[j]);
#pragma unroll
    for (int j = 0; j < T::kBCopies; ++j)
      copy16_to_lds(b_src[j] + (int64_t)n0 * K, Bs + b_dst[j]);
  };
  // The first chunk (n0 <= 0): the same placement through registers, with
  // every element whose n lies outside [0, N) replaced by zero. N % 4 == 0 and
  // n0 % 4 == 0, so a quad is wholly inside or wholly outside.
  auto load_first_chunk = [&](int n0, float* As, float* Bs) __attribute__((always_inline)) {
    float4 va[T::kACopies], vb[T::kBCopies];
    bool oka[T::kACopies], okb[T::kBCopies];
#pragma unroll
    for (int j = 0; j < T::kACopies; ++j) {
      const int n = n0 + 4 * a_quad[j];
      oka[j] = n >= 0 && n < N;
      va[j] = *reinterpret_cast<const float4*>(oka[j] ? a_src[j] + n0 : A);
    }
#pragma unroll
    for (int j = 0; j < T::kBCopies; ++j) {
      const int n = n0 + wave * T::kBCopies + j;
      okb[j] = n >= 0 && n < N;
      vb[j] = *reinterpret_cast<const float4*>(okb[j] ? b_src[j] + (int64_t)n0 * K : B);
    }
#pragma unroll
    for (int j = 0; j < T::kACopies; ++j)
      *reinterpret_cast<float4*>(As + a_dst[j] + 4 * lane) = mask_quad(va[j], oka[j] ? 0xfu : 0u);
#pragma unroll
    for (int j = 0; j < T::kBCopies; ++j)
      *reinterpret_cast<float4*>(Bs + b_dst[j] + 4 * lane) = mask_quad(vb[j], okb[j] ? 0xfu : 0u);
  };

  struct Frag {
    float4 a[T::kRB];
    float b[T::kCB][4];
  };
  // Row of A block i read by this lane, and its swizzle (the same for every
  // block: blocks start at multiples of 32 and the swizzle reads bits 0-3).
  const int a_row0 = wm * T::kWaveM + li;
  const int a_swz = a_swizzle(a_row0);
  // Output columns inside the wave tile are interleaved across the MFMA
  // column blocks: lane column li of block j is column kCB * li + j, so one
  // lane's B operands for all blocks are kCB consecutive floats of a row (one
  // 64-bit LDS read for two blocks). Every output keeps its own column of B,
  // so the product is unchanged; the epilogue writes with the same mapping.
  const int b_frag = 4 * lg * T::BN + wn * T::kWaveN + T::kCB * li;
  auto read_frag = [&](Frag& f, const float* As, const float* Bs, int h) __attribute__((always_inline)) {
    const int q = (2 * h + lg) ^ a_swz;
#pragma unroll
    for (int i = 0; i < T::kRB; ++i)
      f.a[i] = *reinterpret_cast<const float4*>(As + (a_row0 + 32 * i) * BK + 4 * q);
    const float* Bh = Bs + b_frag + 8 * h * T::BN;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (T::kCB == 2) {
        const float2 v = *reinterpret_cast<const float2*>(Bh + t * T::BN);
        f.b[0][t] = v.x;
        f.b[1][t] = v.y;
      } else {
        const float4 v = *reinterpret_cast<const float4*>(Bh + t * T::BN);
        f.b[0][t] = v.x;
        f.b[1][t] = v.y;
        f.b[2][t] = v.z;
        f.b[3][t] = v.w;
      }
    }
  };

  f32x16 acc[T::kRB][T::kCB];
#pragma unroll
  for (int i = 0; i < T::kRB; ++i)
#pragma unroll
    for (int j = 0; j < T::kCB; ++j) acc[i][j] = f32x16{};

  auto mma = [&](const Frag& f) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < T::kRB; ++i)
#pragma unroll
        for (int j = 0; j < T::kCB; ++j) {
          const float av = t == 0 ? f.a[i].x : t == 1 ? f.a[i].y : t == 2 ? f.a[i].z : f.a[i].w;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, f.b[j][t], acc[i][j], 0, 0, 0);
        }
  };

  constexpr int kMfmas = T::kRB * T::kCB * 4;
  constexpr int kReads = T::kRB + 2 * T::kCB;

  // One chunk held in (As, Bs); the copy of the next chunk into (Asn, Bsn) is
  // issued first, spread over the first half-step. The barrier before the
  // last half-step waits for this wave's copies (the compiler's vmcnt(0) of
  // __syncthreads), so after it the next chunk is complete in LDS; it also
  // releases (As, Bs) for the copy that the following chunk issues.
  Frag f[2];
  auto steps = [&](const float* As, const float* Bs) __attribute__((always_inline)) {
    static_for<0, H - 1>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      read_frag(f[(h + 1) & 1], As, Bs, h + 1);
      mma(f[h & 1]);
      sched_interleave<kMfmas, 0, 0, kReads>();
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // a chunk followed by another (at n_next): copy that one first, then compute
  auto chunk_more = [&](int n_next, const float* As, const float* Bs, float* Asn, float* Bsn) __attribute__((always_inline)) {
    copy_chunk(n_next, Asn, Bsn);
    steps(As, Bs);
    __syncthreads();
    read_frag(f[H & 1], Asn, Bsn, 0);
    mma(f[(H - 1) & 1]);
    sched_interleave<kMfmas, 0, 0, kReads>();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto chunk_last = [&](const float* As, const float* Bs) __attribute__((always_inline)) {
    steps(As, Bs);
    mma(f[(H - 1) & 1]);
  };

  // nchunks >= 2 chunks, aligned to the end of the reduction; chunk 0 may
  // reach below n = 0. The loop takes chunks in pairs (stage 0, then stage
  // 1) and ends with the pair (nchunks - 2, nchunks - 1); with an odd count,
  // chunk 0 goes to stage 1 and is computed ahead of the pairs.
  const int nchunks = (N + BK - 1) / BK;
  const int n_first = N - BK * nchunks;  // in (-BK, 0]
  int c = 0;
  if (nchunks & 1) {
    load_first_chunk(n_first, As1, Bs1);
    __syncthreads();
    read_frag(f[0], As1, Bs1, 0);
    chunk_more(n_first + BK, As1, Bs1, As0, Bs0);
    c = 1;
  } else {
    load_first_chunk(n_first, As0, Bs0);
    __syncthreads();
    read_frag(f[0], As0, Bs0, 0);
  }
  for (; c + 2 < nchunks; c += 2) {
    chunk_more(n_first + BK * (c + 1), As0, Bs0, As1, Bs1);
    chunk_more(n_first + BK * (c + 2), As1, Bs1, As0, Bs0);
  }
  chunk_more(N - BK, As0, Bs0, As1, Bs1);
  chunk_last(As1, Bs1);

  // Epilogue. Offsets are 32-bit from the tile's corner, a wave-uniform base,
  // which keeps the address arithmetic small. K % 4 == 0 and a lane's kCB
  // adjacent columns start at a multiple of kCB, so they are wholly inside or
  // outside.
  float* const Ct = C + (int64_t)m0 * K + k0;
  const int col = wn * T::kWaveN + T::kCB * li;
  const bool col_ok = k0 + col < K;
#pragma unroll
  for (int i = 0; i < T::kRB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * T::kWaveM + i * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
      if (col_ok && m0 + row < M) {
        float* dst = Ct + (uint32_t)row * (uint32_t)K + (uint32_t)col;
        if constexpr (T::kCB == 2)
          *reinterpret_cast<float2*>(dst) = make_float2(acc[i][0][r], acc[i][1][r]);
        else
          *reinterpret_cast<float4*>(dst) = make_float4(acc[i][0][r], acc[i][1][r], acc[i][2][r], acc[i][3][r]);
      }
    }
}

}  // namespace fgr
