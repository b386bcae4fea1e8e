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
#include "timestamps.hpp"

namespace fgr {

// BM x BM tiles (32, 64 or 128); D chunks of operands in registers; STRIP as
// in KsplitConfig (the column strip on the vector ALUs in the same launch).
// BUF: the chunk loads go through buffer resources with fixed 32-bit lane
// offsets, for shapes whose offsets fit 32 bits. Measured on MI355X (us per
// call, buffer against 64-bit addresses): at 128x128 0.5-1.2% faster on every
// shape tried (2047^3 126.3 vs 127.4, 8191 x 1023 x 8191 1055 vs 1068, 3501 x
// 2001 x 3501 393 vs 397); at 64x64 faster on a few (1023 x 1025 x 1027 22.9
// vs 23.2) but 5-7% slower on others (3001^3 464 vs 440, 3001 x 1001 x 3001
// 169 vs 158), so only 128x128 tiles take it.
// The four partial tiles pass through LDS all at once, or at BM = 128 half a
// tile at a time (four whole partials would need 256 KB).
template <int BM_, int D_, bool STRIP_ = false, bool BUF_ = false>
struct KregConfig {
  static constexpr int BM = BM_, BN = BM_, BK = 8, D = D_;
  static constexpr bool kStrip = STRIP_;
  static constexpr bool kBuf = BUF_;  // buffer loads (ksplit_offsets_fit(BM, N, K)), else 64-bit addresses
  static constexpr bool kReg = true;
  static constexpr int kWaves = 4;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kRB = BM / 32, kCB = BN / 32;
  static constexpr int kSlices = kRB * kCB;  // MFMA blocks of a tile
  static constexpr int kPartial = BM * BN;   // floats of one wave's partial tile
  static constexpr int kAtOnce = BM == 128 ? 2 : 4;  // whole partials' worth of LDS
  static constexpr int kLds = kAtOnce * kPartial;
  // a wave's share of the reduced tile (32x32, 64x64): kPairs (MFMA block,
  // accumulator group) pairs
  static constexpr int kPairs = kSlices * 4 / kWaves;
  static_assert(BM == 32 || BM == 64 || BM == 128, "32x32, 64x64 or 128x128 tiles");
  static_assert(D >= 2 && D <= 4, "two to four chunks in registers");
  static_assert(!STRIP_ || BM == 64, "the strip goes with 64x64 tiles");
  static_assert(kLds * 4 <= 160 * 1024, "LDS budget of a gfx950 workgroup");
};

// The B columns of lane column li in the tile that starts at column k0, kcb
// adjacent columns per lane (K >= kcb): the lane loads (and computes)
// columns first .. first + kcb - 1, where first is its own first column k0 +
// kcb li, or K - kcb where that would run past K; it stores those from its own
// first column on, i.e. the last kcb - skip of them (none when all of its own
// columns lie past K). The stored columns of the tile's lanes are then each
// column of [k0, min(k0 + 32 kcb, K)) exactly once, and no load leaves [0, K).
struct KregCols {
  int first;
  int skip;
};
__host__ __device__ __forceinline__ KregCols kreg_cols(int k0, int li, int K, int kcb) {
  const int own = k0 + kcb * li;
  const int first = own + kcb <= K ? own : K - kcb;
  return {first, own - first};
}

template <class T>
__global__ __launch_bounds__(T::kThreads) void gemm_mfma_kreg_kernel(
    const float* __restrict__ A, const float* __restrict__ B, float* __restrict__ C, int M, int N, int K,
    int tiles_m, int tiles_n, int group, int parts, float* __restrict__ W, int first, int compact, int nfull) {
  constexpr int BK = T::BK, BN = T::BN, D = T::D, kRB = T::kRB, kCB = T::kCB;
  __shared__ __attribute__((aligned(1024))) float red[T::kLds];

  TsMarks ts;  // measurement build only (timestamps.hpp)
  ts.start();
  // workgroups past the tiles (STRIP): four rows of the column strip each
  const int gx = T::kStrip ? tiles_m * tiles_n : (int)gridDim.x;
  if constexpr (T::kStrip) {
    if ((int)blockIdx.x >= gx) {
      strip_rows(A, B, C, M, N, K, tiles_n * BN, (int)blockIdx.x - gx, red, T::kLds);
      ts.loop_done();
      ts.finish(1);
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
  // B: the lane's kCB adjacent columns (kreg_cols: at the right edge the kCB
  // columns ending at K, of which it stores only its own)
  const KregCols cols = kreg_cols(k0, li, K, kCB);
  const int bce = cols.first;
  const int shift = cols.skip;  // 0 but at the right edge
  const float* pb = B + (int64_t)(4 * lg) * K + bce;
  typedef typename FloatVec<kCB>::type BVec;

  // a chunk's operands, in the registers the MFMAs read
  struct Frag {
    float4 a[kRB];
    BVec b[4];
  };
  // BUF: A through a buffer over the tile's rows (a_voff fixed, 4 n0 bytes
  // scalar), B through a buffer over the chunk's 8 rows (b_voff fixed, row t
  // of the lane's four t K 4 bytes scalar)
  const int tile_rows = M - m0 < T::BM ? M - m0 : T::BM;
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A + (int64_t)m0 * N, (uint32_t)tile_rows * (uint32_t)N * 4u);
  uint32_t a_voff[kRB];
#pragma unroll
  for (int i = 0; i < kRB; ++i) a_voff[i] = (uint32_t)(pa[i] - (A + (int64_t)m0 * N)) * 4u;
  const uint32_t b_voff = (uint32_t)(pb - B) * 4u;
  // chunk starting at reduction index n0 >= 0
  auto load = [&](Frag& f, int n0) __attribute__((always_inline)) {
    if constexpr (T::kBuf) {
#pragma unroll
      for (int i = 0; i < kRB; ++i)
        f.a[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, a_voff[i], (uint32_t)n0 * 4u, 0));
      const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(B + (int64_t)n0 * K, (uint32_t)K * 32u);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t soff = (uint32_t)t * (uint32_t)K * 4u;
        if constexpr (kCB == 4)
          f.b[t] = __builtin_bit_cast(BVec, __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, b_voff, soff, 0));
        else if constexpr (kCB == 2)
          f.b[t] = __builtin_bit_cast(BVec, __builtin_amdgcn_raw_buffer_load_b64(b_rsrc, b_voff, soff, 0));
        else
          f.b[t] = __builtin_bit_cast(BVec, __builtin_amdgcn_raw_buffer_load_b32(b_rsrc, b_voff, soff, 0));
      }
    } else {
#pragma unroll
      for (int i = 0; i < kRB; ++i) f.a[i] = load_dwords<float4>(pa[i] + n0);
      const float* p = pb + (int64_t)n0 * K;
#pragma unroll
      for (int t = 0; t < 4; ++t) f.b[t] = load_dwords<BVec>(p + (int64_t)t * K);
    }
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
  // Operand of column block j at reduction offset t. At 64x64, block 0's
  // operand is passed through a VALU move first: with the MFMAs reading both
  // B operands straight from the registers the loads wrote, two waves per
  // SIMD ran about 30% slower (measured on MI355X, 2047^3: 183 against 141 us
  // with the move; moving both operands: 142; reordering the MFMAs instead:
  // 183). The same move cost 3-8% at 32x32 and 4% at 128x128 (one wave per
  // SIMD), which go without it. The asm keeps the compiler from folding the
  // move away; since the compiler does not take the asm for a vector-ALU
  // write, the asm itself carries the two wait states that an MFMA reading a
  // register needs after such a write (the compiler, counting the asm as one,
  // would leave a single one, and the MFMA could read the register's
  // previous value).
  auto b_of = [&](const Frag& f, int j, int t) __attribute__((always_inline)) {
    float v;
    if constexpr (kCB == 1) {
      v = f.b[t];
    } else if constexpr (kCB == 2) {
      v = j == 0 ? f.b[t].x : f.b[t].y;
      if (j == 0) asm volatile("v_mov_b32 %0, %1\n\ts_nop 1" : "=v"(v) : "v"(v));
    } else {
      v = j == 0 ? f.b[t].x : j == 1 ? f.b[t].y : j == 2 ? f.b[t].z : f.b[t].w;
    }
    return v;
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

  // The ring: the wave's chunk j has its operands in f[(j + D - lead) % D],
  // lead = nmine % D. Chunks 0 .. D - 2 are loaded first; then each step
  // issues chunk j + D - 1's loads and runs chunk j's MFMAs. The lead chunks
  // run before the loop, so that the loop runs whole groups of D from f[0]:
  // one loop and no chunk under a condition, so the accumulators stay in
  // place. Loads past the wave's last chunk repeat it (never used), so that
  // every step issues the same loads and the compiler's wait counts stay exact
  // (a load issued on some paths only makes it wait for every load in flight).
  Frag f[D];
  const int j_last = nmine - 1;
  if (nmine > 0) {
    // chunks 1 .. : the wave's chunk j, or its last chunk repeated (at n0 >= 0
    // even when that is chunk 0, whose plain loads would reach below row 0)
    auto n0_of = [&](int j) __attribute__((always_inline)) {
      const int n0 = chunk_n0(j < j_last ? j : j_last);
      return n0 > 0 ? n0 : 0;
    };
    auto step = [&](auto kc, int j) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;  // slot of chunk j
      load(f[(k + D - 1) % D], n0_of(j + D - 1));
      __builtin_amdgcn_sched_barrier(0);
      mma(f[k]);
      __builtin_amdgcn_sched_barrier(0);
    };
    const int lead = nmine % D;
    static_for<0, D>([&](auto rc) {
      constexpr int R = decltype(rc)::value;
      if (lead == R) {
        constexpr int s0 = (D - R) % D;  // slot of chunk 0
        if (chunk_n0(0) < 0) load_first(f[s0], chunk_n0(0));
        else load(f[s0], chunk_n0(0));
        static_for<1, D - 1>([&](auto dc) {
          constexpr int d = decltype(dc)::value;
          load(f[(s0 + d) % D], n0_of(d));
        });
        static_for<0, R>([&](auto kc) {
          constexpr int k = decltype(kc)::value;
          step(std::integral_constant<int, (s0 + k) % D>{}, k);
        });
      }
    });
    for (int c = lead; c < nmine; c += D)
      static_for<0, D>([&](auto kc) { step(kc, c + decltype(kc)::value); });
  }

  ts.loop_done();
  // The four partial tiles are added in wave order, ((p0 + p1) + p2) + p3,
  // through LDS: kAtOnce of them at a time, wave w's in slot w % kAtOnce
  // (slice s = MFMA block i = s / kCB, j = s % kCB: 16 accumulators of every
  // lane, at s * 1024, lane-major as float4). Each wave adds up its share of
  // the tile, kPairs (slice, accumulator group q) pairs:
  //   32x32: group q = w;
  //   64x64: block row i = w / 2, both column blocks, groups 2 (w % 2) and
  //          2 (w % 2) + 1 (pair u: j = u % 2, q = 2 (w % 2) + u / 2).
  // 128x128 tiles reduce half a tile at a time after the store set-up below.
  auto pair_of = [&](int u, int& sl, int& q) __attribute__((always_inline)) {
    if constexpr (T::BM == 32) {
      sl = 0;
      q = wave;
    } else {
      sl = 2 * (wave >> 1) + (u & 1);
      q = 2 * (wave & 1) + (u >> 1);
    }
  };
  float4 sum[T::kPairs];
  if constexpr (T::kAtOnce == 4) {
#pragma unroll
    for (int ph = 0; ph < T::kWaves / T::kAtOnce; ++ph) {
      if (ph > 0) __syncthreads();  // the last phase's partials have been read
      if (wave / T::kAtOnce == ph) {
        float* mine = red + (wave % T::kAtOnce) * T::kPartial;
#pragma unroll
        for (int sl = 0; sl < T::kSlices; ++sl)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4*>(mine + sl * 1024 + 256 * q + 4 * lane) =
                make_float4(acc[sl / kCB][sl % kCB][4 * q], acc[sl / kCB][sl % kCB][4 * q + 1],
                            acc[sl / kCB][sl % kCB][4 * q + 2], acc[sl / kCB][sl % kCB][4 * q + 3]);
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < T::kPairs; ++u) {
        int sl, q;
        pair_of(u, sl, q);
#pragma unroll
        for (int p = 0; p < T::kAtOnce; ++p) {
          const float4 v = *reinterpret_cast<const float4*>(red + p * T::kPartial + sl * 1024 + 256 * q + 4 * lane);
          sum[u] = ph == 0 && p == 0 ? v : make_float4(sum[u].x + v.x, sum[u].y + v.y, sum[u].z + v.z, sum[u].w + v.w);
        }
      }
    }
  }

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
  // Row r of accumulator group q, element k: 8 q + 4 lg + k of its block
  // row; the lane's columns are bce .. bce + kCB - 1, of which it stores
  // those from bc on (all of them, in one store, but at the right edge).
  auto comp = [](const float4& v, int k) __attribute__((always_inline)) {
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
  };
  const int col = bce - k0;  // negative (down to 1 - kCB) at the right edge
  const bool whole_cols = shift == 0;
  auto store_row = [&](int row, const float (&e)[kCB]) __attribute__((always_inline)) {
    if (m0 + row >= M) return;
    // signed: with col < 0 only the elements j >= shift, at or past the
    // row's column 0 of the tile, are written
    float* dst = Ct + (int64_t)row * (int64_t)ldc + col;
    if (whole_cols) {
      if constexpr (kCB == 4) store_dwords<float4>(dst, make_float4(e[0], e[1], e[2], e[3]));
      else if constexpr (kCB == 2) store_dwords<float2>(dst, make_float2(e[0], e[1]));
      else *dst = e[0];
    } else {
#pragma unroll
      for (int j = 0; j < kCB; ++j)
        if (j >= shift) dst[j] = e[j];
    }
  };

  if constexpr (T::BM == 32) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float e[1] = {comp(sum[0], k)};
      store_row(8 * wave + 4 * lg + k, e);
    }
  } else if constexpr (T::BM == 64) {
    const int i = wave >> 1;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float e[2] = {comp(sum[2 * qq], k), comp(sum[2 * qq + 1], k)};
        store_row(i * 32 + 8 * (2 * (wave & 1) + qq) + 4 * lg + k, e);
      }
  } else {
    // 128x128: the tile in two halves of 8 MFMA blocks (block rows 2h and
    // 2h + 1), all four partials of a half at once (4 x 32 KiB). Wave w's
    // share of half h: block row 2h + w / 2, column blocks 2 (w % 2) and
    // 2 (w % 2) + 1, every accumulator group; a lane stores its two adjacent
    // columns of those blocks together. (Two whole partials at a time instead
    // needed a running sum, or adds into a wave's accumulators, kept across a
    // barrier: 12 to 16 VGPRs spilled.)
    constexpr int kHalf = T::kSlices / 2;  // MFMA blocks per half
    auto half_slot = [&](int p) __attribute__((always_inline)) { return red + p * (kHalf * 1024); };
    const int j0 = 2 * (wave & 1);  // the share's first column block
    auto add4 = [](float4 x, float4 y) __attribute__((always_inline)) {
      return make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
    };
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h > 0) __syncthreads();  // the first half has been read
      float* mine = half_slot(wave);
#pragma unroll
      for (int b = 0; b < kHalf; ++b) {
        const int sl = kHalf * h + b;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float4*>(mine + b * 1024 + 256 * q + 4 * lane) =
              make_float4(acc[sl / kCB][sl % kCB][4 * q], acc[sl / kCB][sl % kCB][4 * q + 1],
                          acc[sl / kCB][sl % kCB][4 * q + 2], acc[sl / kCB][sl % kCB][4 * q + 3]);
      }
      __syncthreads();
      const int br = 2 * h + (wave >> 1);  // block row
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 v[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int b = 4 * (wave >> 1) + j0 + jj;  // block inside the half
          auto at = [&](int p) __attribute__((always_inline)) {
            return *reinterpret_cast<const float4*>(half_slot(p) + b * 1024 + 256 * q + 4 * lane);
          };
          v[jj] = add4(add4(add4(at(0), at(1)), at(2)), at(3));
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int row = 32 * br + 8 * q + 4 * lg + k;
          if (m0 + row >= M) continue;
          float* dst = Ct + (int64_t)row * (int64_t)ldc + col + j0;
          const float e0 = comp(v[0], k), e1 = comp(v[1], k);
          if (whole_cols) {
            store_dwords<float2>(dst, make_float2(e0, e1));
          } else {
            if (j0 >= shift) dst[0] = e0;
            if (j0 + 1 >= shift) dst[1] = e1;
          }
        }
      }
    }
  }
  ts.finish();
}

}  // namespace fgr
