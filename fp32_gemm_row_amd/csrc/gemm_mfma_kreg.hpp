// FP32 MFMA k-split tiles whose operands go straight from global memory into
// the MFMA operand registers: the form for rows that are not 16-byte aligned.
//
// The k-split kernel (gemm_mfma_ksplit.hpp) stages every chunk through LDS
// with global->LDS copies. Those copies move 16 bytes per lane only from
// 16-byte aligned addresses; with N or K not a multiple of 4 the rows of A or
// B start at arbitrary 4-byte boundaries and the copies fall back to 4 bytes
// per lane, so a chunk of a 64x64 tile takes 16 copy instructions per wave and
// the copies, not the matrix cores, set the pace. Here each lane instead
// loads exactly the operands its MFMAs take, in their register layout:
//
//   A: the four reduction indices 4 lg .. 4 lg + 3 of the chunk for row li
//      (+ 32 i): one 16-byte load per MFMA block row;
//   B: reduction index 4 lg + t, the kCB adjacent output columns kCB li ..
//      kCB li + kCB - 1 of lane column li (the interleaved output columns of
//      the k-split kernel): one kCB-float load per t.
//
// On gfx9-family GPUs a global load of two or four dwords needs only dword
// alignment, so these loads need nothing beyond the 4-byte alignment every
// float has; the compiler emits global_load_dwordx4 / dwordx2 for them. A
// 64x64 chunk is then 6 load instructions per wave and no LDS traffic at all.
// The operand registers of D chunks rotate as a ring: the loads of chunk j +
// D - 1 are issued before chunk j's MFMAs, and the compiler's wait counts hold
// the MFMAs of a chunk until its own loads are back.
//
// Everything else is the k-split kernel's: the tile and part decomposition,
// the chunks dealt to the four waves in turn (wave w takes chunks w, w + 4, ...
// of its part), 8-deep chunks aligned to the end of the reduction so that
// only chunk 0 reaches below n = 0 (loaded element by element with zero
// fill), and the four partial tiles added in wave order through LDS. With the
// same chunk order and MFMA order per wave the results are bitwise those of the
// k-split kernel.
#pragma once

#include "gemm_mfma.hpp"
#include "gemm_mfma_split.hpp"
#include "strip.hpp"

namespace fgr {

// BM x BM tiles (32 or 64); D chunks of operands in registers; STRIP as in
// KsplitConfig (the column strip on the vector ALUs in the same launch).
template <int BM_, int D_, bool STRIP_ = false>
struct KregConfig {
  static constexpr int BM = BM_, BN = BM_, BK = 8, D = D_;
  static constexpr bool kStrip = STRIP_;
  static constexpr bool kPaddedA = false;  // reads the caller's A: lda = N, pad = 0
  static constexpr bool kReg = true;
  static constexpr int kWaves = 4;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kRB = BM / 32, kCB = BN / 32;
  static constexpr int kSlices = kRB * kCB;  // MFMA blocks of a tile
  static constexpr int kPartial = BM * BN;   // floats of one wave's partial tile
  static constexpr int kLds = kWaves * kPartial;
  static_assert(BM == 32 || BM == 64, "32x32 or 64x64 tiles (four 128x128 partials exceed the LDS)");
  static_assert(D >= 2 && D <= 4, "two to four chunks in registers");
  static_assert(!STRIP_ || BM == 64, "the strip goes with 64x64 tiles");
  static_assert(kLds * 4 <= 160 * 1024, "LDS budget of a gfx950 workgroup");
};

template <class T>
__global__ __launch_bounds__(T::kThreads) void gemm_mfma_kreg_kernel(
    const float* __restrict__ A, const float* __restrict__ B, float* __restrict__ C, int M, int N, int K,
    int tiles_m, int tiles_n, int group, int parts, float* __restrict__ W, int first, int compact, int nfull,
    int /*lda*/, int /*pad*/) {
  constexpr int BK = T::BK, BN = T::BN, D = T::D, kRB = T::kRB, kCB = T::kCB;
  __shared__ __attribute__((aligned(1024))) float red[T::kLds];

  // workgroups past the tiles (STRIP): four rows of the column strip each
  const int gx = T::kStrip ? tiles_m * tiles_n : (int)gridDim.x;
  if constexpr (T::kStrip) {
    if ((int)blockIdx.x >= gx) {
      strip_rows(A, B, C, M, N, K, tiles_n * BN, (int)blockIdx.x - gx, red, T::kLds);
      return;
    }
  }

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int li = lane & 31;
  const int lg = lane >> 5;

  // Tiles and parts exactly as in the k-split kernel: the first nfull
  // workgroups take whole tiles [first, first + nfull) into C; the others
  // take the tiles after them, each split over `parts` workgroups (logical id
  // part * ntiles + tile) writing partial tiles to W.
  const bool whole = (int)blockIdx.x < nfull;
  const int grid = whole ? nfull : gx - nfull;
  const int logical = xcd_remap(whole ? (int)blockIdx.x : (int)blockIdx.x - nfull, grid);
  const int kparts = whole ? 1 : parts;
  const int ntiles = grid / kparts;
  const int part = logical / ntiles;
  const int tl = logical - part * ntiles;
  int tm, tn;
  grouped_tile(first + (whole ? 0 : nfull) + tl, tiles_m, tiles_n, group, tm, tn);
  const int m0 = tm * T::BM;
  const int k0 = tn * BN;

  const int nchunks = (N + BK - 1) / BK;
  const int n_first = N - BK * nchunks;  // in (-BK, 0]
  const int pc0 = (int)((int64_t)nchunks * part / kparts);
  const int pn = (int)((int64_t)nchunks * (part + 1) / kparts) - pc0;
  const int nmine = pn > wave ? (pn - wave + T::kWaves - 1) / T::kWaves : 0;
  auto chunk_n0 = [&](int j) __attribute__((always_inline)) {
    return n_first + BK * (pc0 + wave + T::kWaves * j);
  };

  // A: row li + 32 i of the tile (rows past M read row M - 1, never stored),
  // from reduction index 4 lg of each chunk.
  const float* pa[kRB];
#pragma unroll
  for (int i = 0; i < kRB; ++i) {
    const int r = m0 + li + 32 * i;
    pa[i] = A + (int64_t)(r < M ? r : M - 1) * N + 4 * lg;
  }
  // B: the lane's kCB columns from bc, read from bce = bc clamped so that
  // the load stays inside the row (K >= kCB); a lane whose first column is
  // the row's last (bc = K - 1 with kCB = 2) takes it from the load's second
  // element. Columns past K are read but never stored.
  const int bc = k0 + kCB * li;
  const int bce = bc + kCB <= K ? bc : K - kCB;
  const bool shifted = bc != bce;
  const float* pb = B + (int64_t)(4 * lg) * K + bce;
  typedef typename FloatVec<kCB>::type BVec;

  // a chunk's operands as loaded: B's stay raw vectors until the MFMAs take
  // them (choosing the shifted element at load time would wait for the load)
  struct Frag {
    float4 a[kRB];
    BVec b[4];
  };
  // chunk starting at reduction index n0 >= 0
  auto load = [&](Frag& f, int n0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kRB; ++i) f.a[i] = load_dwords<float4>(pa[i] + n0);
    const float* p = pb + (int64_t)n0 * K;
#pragma unroll
    for (int t = 0; t < 4; ++t) f.b[t] = load_dwords<BVec>(p + (int64_t)t * K);
  };
  // chunk 0 of the reduction (n0 = n_first < 0): element by element, zero
  // below n = 0 (loads there read the matrix's first element instead)
  auto load_first = [&](Frag& f, int n0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kRB; ++i) {
      float e[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool ok = n0 + 4 * lg + q >= 0;
        const float v = *(ok ? pa[i] + n0 + q : A);
        e[q] = ok ? v : 0.f;
      }
      f.a[i] = make_float4(e[0], e[1], e[2], e[3]);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bool ok = n0 + 4 * lg + t >= 0;
      const BVec v = load_dwords<BVec>(ok ? pb + (int64_t)(n0 + t) * K : B + bce);
      f.b[t] = ok ? v : BVec{};
    }
  };
  // operand of column block j at reduction offset t
  auto b_of = [&](const Frag& f, int j, int t) __attribute__((always_inline)) {
    if constexpr (kCB == 2) return j == 0 ? (shifted ? f.b[t].y : f.b[t].x) : f.b[t].y;
    else return f.b[t];
  };

  f32x16 acc[kRB][kCB];
#pragma unroll
  for (int i = 0; i < kRB; ++i)
#pragma unroll
    for (int j = 0; j < kCB; ++j) acc[i][j] = f32x16{};
  auto mma = [&](const Frag& f) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < kRB; ++i)
#pragma unroll
        for (int j = 0; j < kCB; ++j) {
          const float av = t == 0 ? f.a[i].x : t == 1 ? f.a[i].y : t == 2 ? f.a[i].z : f.a[i].w;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b_of(f, j, t), acc[i][j], 0, 0, 0);
        }
  };

  // The ring: chunk j's operands in f[j % D]. Chunks 0 .. D - 2 first; then
  // each step issues chunk j + D - 1's loads and runs chunk j's MFMAs. Loads
  // past the wave's last chunk repeat it (never used), so that every step
  // issues the same loads and the compiler's wait counts stay exact (a load
  // issued on some paths only makes it wait for every load in flight); the
  // last nmine % D chunks, already loaded, run after the whole groups of D.
  Frag f[D];
  const int j_last = nmine - 1;
  if (nmine > 0) {
    // chunks 1 .. : the wave's chunk j, or its last chunk repeated (at n0 >= 0
    // even when that is chunk 0, whose plain loads would reach below row 0)
    auto n0_of = [&](int j) __attribute__((always_inline)) {
      const int n0 = chunk_n0(j < j_last ? j : j_last);
      return n0 > 0 ? n0 : 0;
    };
    if (chunk_n0(0) < 0) load_first(f[0], chunk_n0(0));
    else load(f[0], chunk_n0(0));
    static_for<1, D - 1>([&](auto dc) { load(f[decltype(dc)::value], n0_of(decltype(dc)::value)); });
    const int whole_end = nmine - nmine % D;
    for (int c = 0; c < whole_end; c += D) {
      static_for<0, D>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        load(f[(k + D - 1) % D], n0_of(c + k + D - 1));
        __builtin_amdgcn_sched_barrier(0);
        mma(f[k]);
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    // the last nmine - whole_end < D chunks, nested so that every path
    // updates the accumulators in place
    auto rest = [&](auto kc, auto& self) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      if constexpr (k < D - 1) {
        if (whole_end + k < nmine) {
          mma(f[k]);
          self(std::integral_constant<int, k + 1>{}, self);
        }
      }
    };
    rest(std::integral_constant<int, 0>{}, rest);
  }

  // The four partial tiles through LDS, each wave's at red + wave kPartial:
  // slice s (MFMA block i = s / kCB, j = s % kCB, 16 accumulators of every
  // lane) at s * 1024, lane-major as float4. Then each wave adds its share of
  // the tile over the partials in wave order, ((p0 + p1) + p2) + p3.
  float* mine = red + wave * T::kPartial;
#pragma unroll
  for (int s = 0; s < T::kSlices; ++s)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(mine + s * 1024 + 256 * q + 4 * lane) =
          make_float4(acc[s / kCB][s % kCB][4 * q], acc[s / kCB][s % kCB][4 * q + 1],
                      acc[s / kCB][s % kCB][4 * q + 2], acc[s / kCB][s % kCB][4 * q + 3]);
  __syncthreads();

  float* Ct;
  uint32_t ldc;  // row stride; row * ldc is formed in 64 bits (K may pass 2^25)
  if (kparts == 1) {
    Ct = C + (int64_t)m0 * K + k0;
    ldc = (uint32_t)K;
  } else if (compact) {
    Ct = W + ((int64_t)part * ntiles + tl) * (T::BM * BN);
    ldc = BN;
  } else {
    Ct = W + (int64_t)part * M * K + (int64_t)m0 * K + k0;
    ldc = (uint32_t)K;
  }
  // the partial sums of accumulator group q (4 accumulators) of slice s
  auto sum4 = [&](int s, int q) __attribute__((always_inline)) {
    float4 v = *reinterpret_cast<const float4*>(red + s * 1024 + 256 * q + 4 * lane);
#pragma unroll
    for (int p = 1; p < T::kWaves; ++p) {
      const float4 w = *reinterpret_cast<const float4*>(red + p * T::kPartial + s * 1024 + 256 * q + 4 * lane);
      v = make_float4(v.x + w.x, v.y + w.y, v.z + w.z, v.w + w.w);
    }
    return v;
  };
  if constexpr (kCB == 2) {
    // 64x64: wave w takes block row i = w / 2, both column blocks, and
    // accumulator groups q = 2 (w % 2), 2 (w % 2) + 1 (rows 16 (w % 2) ..
    // + 15 of the block row's 32 in the MFMA's order): lane column li holds
    // output columns 2 li and 2 li + 1, stored together
    const int i = wave >> 1;
    const int col = 2 * li;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int q = 2 * (wave & 1) + qq;
      const float4 v0 = sum4(2 * i, q), v1 = sum4(2 * i + 1, q);
      const float e0[4] = {v0.x, v0.y, v0.z, v0.w}, e1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int row = i * 32 + 8 * q + 4 * lg + k;
        if (m0 + row >= M) continue;
        float* dst = Ct + (uint64_t)row * ldc + (uint32_t)col;
        if (k0 + col + 1 < K) store_dwords<float2>(dst, make_float2(e0[k], e1[k]));
        else if (k0 + col < K) *dst = e0[k];
      }
    }
  } else {
    // 32x32: one slice; wave w stores accumulator group q = w
    const int q = wave;
    const float4 v = sum4(0, q);
    const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int row = 8 * q + 4 * lg + k;
      if (k0 + li < K && m0 + row < M) Ct[(uint64_t)row * ldc + (uint32_t)li] = e[k];
    }
  }
}

}  // namespace fgr
