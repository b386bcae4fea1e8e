// FP32 MFMA GEMM for shapes with few output tiles: the reduction is split
// across the waves of a workgroup.
//
// When M x K holds too few tiles to occupy the 256 CUs (the ragged 1023-size
// problem has 272 tiles of 64 x 64, a 256-cube only 16), a workgroup's waves
// would each own a 32 x 32 corner of a small tile and spend most of their time
// at barriers. Here every wave of the workgroup computes the WHOLE BM x BN
// tile, each over its own share of the reduction index n (the ceil(N / BK)
// chunks dealt to the workgroup's S waves in turn: wave w takes chunks w,
// w + S, ..., so that the waves load neighbouring pieces of the same rows of A
// at about the same time). A wave
// stages its own chunks through its own region of LDS, so the main loop has no
// barrier at all: LDS operations of one wave complete in order, which is the
// only ordering its private staging needs. At the end the S partial tiles are
// written to LDS and added in wave order (0, 1, ..., S - 1), so the result is
// deterministic; no workspace and no atomics.
//
// This is the pages' output-parallel decomposition ("LeetGPU |
// 02_Matrix_Multiplication", V0 "Approach": outputs are independent, each
// reduction belongs to one thread or tile) kept at workgroup level, with the
// reduction of each tile shared by the workgroup's waves.
//
// Tail mode (sub > 0): the workgroups cover big square tiles of sub*BM, the
// logical big tiles [first, first + gridDim.x / sub^2) of a tiles_m x tiles_n
// grid walked in the grouped order, each cut into sub x sub tiles of BM x BN.
// This spreads the few 256 x 256 tiles of a last, partial wave of the
// direct-copy kernel over every CU.
//
// Within a wave: the same MFMA operand layout, zero padding and LDS pitch as
// gemm_mfma.hpp (v_mfma_f32_32x32x2_f32, reduction index 8h + 4g + t of a
// chunk for half-wave g at step (h, t)); output columns are interleaved across
// the kCB column blocks (lane column li of block j is column kCB * li + j) so
// that one lane's B operands for all blocks are adjacent in LDS.
#pragma once

#include "gemm_mfma.hpp"

namespace fgr {

template <int BM_, int BN_, int BK_, int S_>
struct SplitConfig {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, S = S_;
  static constexpr int kThreads = S * 64;
  static constexpr int kRB = BM / 32;
  static constexpr int kCB = BN / 32;
  static constexpr int kLdA = BK + 4;  // padded A pitch (floats)
  static constexpr int kLdB = BN;
  static constexpr int kAQuads = BK / 4;
  static constexpr int kBQuads = BN / 4;
  static constexpr int kAPerLane = BM * BK / 4 / 64;  // float4 loads per lane per chunk
  static constexpr int kBPerLane = BK * BN / 4 / 64;
  static constexpr int kStage = BM * kLdA + BK * kLdB;  // floats, one wave, one stage
  static constexpr int kLdsFloats =
      (2 * S * kStage > S * BM * BN) ? 2 * S * kStage : S * BM * BN;

  static_assert(BM % 32 == 0 && BN % 32 == 0, "tile must be a multiple of 32x32");
  static_assert(kCB == 1 || kCB == 2 || kCB == 4, "B operands are read as 1, 2 or 4 floats");
  static_assert(BK % 16 == 0, "BK must be a multiple of 16 (an even number of half-steps)");
  static_assert(BM * BK % 256 == 0 && BK * BN % 256 == 0, "chunks split evenly over a wave");
  static_assert(64 % kAQuads == 0 && 64 % kBQuads == 0, "a lane keeps its column quad");
  static_assert(kLdsFloats * 4 <= 160 * 1024, "LDS budget of a gfx950 workgroup");
  static_assert(BM * BN % kThreads == 0, "the final sum splits evenly over threads");
};

template <int CB>
struct FloatVec;
template <>
struct FloatVec<1> {
  typedef float type;
};
template <>
struct FloatVec<2> {
  typedef float2 type;
};
template <>
struct FloatVec<4> {
  typedef float4 type;
};

__device__ __forceinline__ float vec_get(float v, int) { return v; }
__device__ __forceinline__ float vec_get(float2 v, int i) { return i == 0 ? v.x : v.y; }
__device__ __forceinline__ float vec_get(float4 v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <class T, bool VEC>
__global__ __launch_bounds__(T::kThreads) void gemm_mfma_split_kernel(
    const float* __restrict__ A, const float* __restrict__ B, float* __restrict__ C, int M, int N,
    int K, int tiles_m, int tiles_n, int group, int first, int sub) {
  constexpr int BM = T::BM, BN = T::BN, BK = T::BK, S = T::S;
  static_assert(BM == BN, "tail mode cuts square big tiles");
  constexpr int H = BK / 8;
  __shared__ __attribute__((aligned(16))) float lds[T::kLdsFloats];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31;
  const int lg = lane >> 5;

  int tm, tn, m0, k0;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  if (sub == 0) {
    grouped_tile(logical, tiles_m, tiles_n, group, tm, tn);
    m0 = tm * BM;
    k0 = tn * BN;
  } else {
    const int per = sub * sub;
    grouped_tile(first + logical / per, tiles_m, tiles_n, group, tm, tn);
    const int w = logical % per;
    m0 = (tm * sub + w / sub) * BM;
    k0 = (tn * sub + w % sub) * BN;
    if (m0 >= M || k0 >= K) return;  // a piece of a partial big tile: no outputs
  }

  // this wave's share of the reduction: chunks wave, wave + S, wave + 2S, ...
  // (dealt in turn, so that the waves load neighbouring pieces of the same
  // rows of A at about the same time)
  const int nchunks = (N + BK - 1) / BK;
  const int nmine = nchunks > wave ? (nchunks - wave + S - 1) / S : 0;

  float* const stage0 = lds + wave * 2 * T::kStage;

  // Per-lane load slots (a wave loads whole chunks by itself).
  const float* a_ptr[T::kAPerLane];
  bool a_row_ok[T::kAPerLane];
  int a_col[T::kAPerLane];
  int a_lds[T::kAPerLane];
#pragma unroll
  for (int i = 0; i < T::kAPerLane; ++i) {
    const int f = lane + 64 * i;
    const int r = f / T::kAQuads;
    const int q = f % T::kAQuads;
    a_row_ok[i] = m0 + r < M;
    a_col[i] = 4 * q;
    a_ptr[i] = A + (int64_t)(a_row_ok[i] ? m0 + r : 0) * N + 4 * q;
    a_lds[i] = r * T::kLdA + 4 * q;
  }
  const float* b_ptr[T::kBPerLane];
  int b_row[T::kBPerLane];
  int b_lds[T::kBPerLane];
  const int b_col = k0 + 4 * (lane % T::kBQuads);
#pragma unroll
  for (int i = 0; i < T::kBPerLane; ++i) {
    const int f = lane + 64 * i;
    const int r = f / T::kBQuads;
    b_row[i] = r;
    b_ptr[i] = B + (int64_t)r * K + b_col;
    b_lds[i] = BM * T::kLdA + r * T::kLdB + 4 * (f % T::kBQuads);
  }

  // On the 32-bit path a lane's elements are placed so that consecutive lanes
  // take consecutive columns: A element i of a lane is row ea_r0 + i * 64 / BK,
  // column lane % BK of the chunk (likewise for B with BN), so each 32-bit
  // load instruction reads whole row segments.
  constexpr int kARowStep = 64 / BK;
  constexpr int kBRowStep = 64 / BN;
  static_assert(64 % BK == 0 && 64 % BN == 0, "element slots keep one column");
  const int ea_r0 = lane / BK, ea_c = lane % BK;
  const int eb_r0 = lane / BN, eb_c = lane % BN;
  const float* const ea_base = A + (int64_t)(m0 + ea_r0 < M ? m0 + ea_r0 : 0) * N + ea_c;
  const float* const eb_base = B + (int64_t)eb_r0 * K + k0 + eb_c;

  float4 ra[T::kAPerLane], rb[T::kBPerLane];
  unsigned oka[T::kAPerLane], okb[T::kBPerLane];
  auto load_chunk = [&](int c) {
    const int n0 = c * BK;
    if constexpr (VEC) {
#pragma unroll
      for (int i = 0; i < T::kAPerLane; ++i)
        ra[i] = load_quad<VEC>(a_ptr[i] + n0, A, a_row_ok[i], n0 + a_col[i], N, oka[i]);
#pragma unroll
      for (int i = 0; i < T::kBPerLane; ++i)
        rb[i] = load_quad<VEC>(b_ptr[i] + (int64_t)n0 * K, B, n0 + b_row[i] < N, b_col, K, okb[i]);
    } else {
      const bool a_col_in = n0 + ea_c < N;
#pragma unroll
      for (int s = 0; s < T::kAPerLane; ++s) {
        float x[4];
        unsigned ok = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * s + e;
          const bool in = a_col_in && m0 + ea_r0 + i * kARowStep < M;
          ok |= in ? 1u << e : 0u;
          x[e] = *(in ? ea_base + (int64_t)i * kARowStep * N + n0 : A);
        }
        ra[s] = make_float4(x[0], x[1], x[2], x[3]);
        oka[s] = ok;
      }
      const bool b_col_in = k0 + eb_c < K;
#pragma unroll
      for (int s = 0; s < T::kBPerLane; ++s) {
        float x[4];
        unsigned ok = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * s + e;
          const bool in = b_col_in && n0 + eb_r0 + i * kBRowStep < N;
          ok |= in ? 1u << e : 0u;
          x[e] = *(in ? eb_base + ((int64_t)n0 + i * kBRowStep) * K : B);
        }
        rb[s] = make_float4(x[0], x[1], x[2], x[3]);
        okb[s] = ok;
      }
    }
  };
  auto store_chunk = [&](float* st) {
    if constexpr (VEC) {
#pragma unroll
      for (int i = 0; i < T::kAPerLane; ++i)
        *reinterpret_cast<float4*>(st + a_lds[i]) = mask_quad(ra[i], oka[i]);
#pragma unroll
      for (int i = 0; i < T::kBPerLane; ++i)
        *reinterpret_cast<float4*>(st + b_lds[i]) = mask_quad(rb[i], okb[i]);
    } else {
#pragma unroll
      for (int s = 0; s < T::kAPerLane; ++s) {
        const float4 v = mask_quad(ra[s], oka[s]);
        const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) st[(ea_r0 + (4 * s + e) * kARowStep) * T::kLdA + ea_c] = x[e];
      }
#pragma unroll
      for (int s = 0; s < T::kBPerLane; ++s) {
        const float4 v = mask_quad(rb[s], okb[s]);
        const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          st[BM * T::kLdA + (eb_r0 + (4 * s + e) * kBRowStep) * T::kLdB + eb_c] = x[e];
      }
    }
  };

  typedef typename FloatVec<T::kCB>::type BVec;
  struct Frag {
    float4 a[T::kRB];
    float b[T::kCB][4];
  };
  const int a_frag = li * T::kLdA + 4 * lg;
  const int b_frag = BM * T::kLdA + 4 * lg * T::kLdB + T::kCB * li;
  auto read_frag = [&](Frag& f, const float* st, int h) {
#pragma unroll
    for (int i = 0; i < T::kRB; ++i)
      f.a[i] = *reinterpret_cast<const float4*>(st + a_frag + i * 32 * T::kLdA + 8 * h);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const BVec v = *reinterpret_cast<const BVec*>(st + b_frag + (8 * h + t) * T::kLdB);
#pragma unroll
      for (int j = 0; j < T::kCB; ++j) f.b[j][t] = vec_get(v, j);
    }
  };

  f32x16 acc[T::kRB][T::kCB];
#pragma unroll
  for (int i = 0; i < T::kRB; ++i)
#pragma unroll
    for (int j = 0; j < T::kCB; ++j) acc[i][j] = f32x16{};

  auto mma = [&](const Frag& f) {
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

  // Per-wave pipeline over its chunks: the wave's j-th chunk sits in stage
  // j % 2 of the wave's region; the next chunk is loaded into registers at the
  // top of the current one and written to the other stage before its last
  // half-step (the reads of that stage for chunk j - 1 were issued earlier by
  // this same wave, and LDS serves one wave's operations in order).
  if (nmine > 0) {
    Frag f[2];
    load_chunk(wave);
    store_chunk(stage0);
    read_frag(f[0], stage0, 0);
    int s = 0;
    for (int j = 0; j + 1 < nmine; ++j) {
      const float* st = stage0 + s * T::kStage;
      float* nx = stage0 + (s ^ 1) * T::kStage;
      load_chunk(wave + S * (j + 1));
      static_for<0, H - 1>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        read_frag(f[(h + 1) & 1], st, h + 1);
        mma(f[h & 1]);
        __builtin_amdgcn_sched_barrier(0);
      });
      store_chunk(nx);
      read_frag(f[H & 1], nx, 0);
      mma(f[(H - 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      s ^= 1;
    }
    const float* st = stage0 + s * T::kStage;
    static_for<0, H - 1>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      read_frag(f[(h + 1) & 1], st, h + 1);
      mma(f[h & 1]);
      __builtin_amdgcn_sched_barrier(0);
    });
    mma(f[(H - 1) & 1]);
  }

  // Partial tiles to LDS (the staging is no longer needed once every wave is
  // past this barrier), then the S partials of each element added in wave
  // order and stored with consecutive threads on consecutive columns.
  __syncthreads();
  float* const part = lds + wave * BM * BN;
#pragma unroll
  for (int i = 0; i < T::kRB; ++i)
#pragma unroll
    for (int j = 0; j < T::kCB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
        part[row * BN + T::kCB * li + j] = acc[i][j][r];
      }
  __syncthreads();
#pragma unroll
  for (int e = tid; e < BM * BN; e += T::kThreads) {
    const int row = e / BN;
    const int col = e % BN;
    float s = lds[e];
#pragma unroll
    for (int w = 1; w < S; ++w) s += lds[w * BM * BN + e];
    if (m0 + row < M && k0 + col < K) C[(int64_t)(m0 + row) * K + k0 + col] = s;
  }
}

}  // namespace fgr
