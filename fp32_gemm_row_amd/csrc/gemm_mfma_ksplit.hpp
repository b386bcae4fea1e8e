// FP32 MFMA GEMM for mid-size and small shapes: output tiles whose reduction
// is split over the four waves of a workgroup ("k-split"), each wave fed by
// its own direct global->LDS copies.
//
// Between the few-tile shapes and the whole-device shapes of gemm_mfma_dma.hpp
// (at least one 256x256 tile per CU) lie shapes such as 2048^3 or a
// (1024, 6144, 4096) row shard: 64 tiles of 256x256, 256 of 128x128, 1024 of
// 64x64. Each wave of a workgroup computes the WHOLE tile over every fourth
// reduction chunk (wave w takes chunks w, w + 4, ...: the four waves then
// read neighbouring 32-byte pieces of the same 128-byte lines of A at about
// the same time), so a tile keeps a CU's four matrix cores busy with a
// quarter of the outputs a whole-device tile needs. At the end the four
// partial tiles are added in wave order (0, 1, 2, 3) through LDS, each wave
// summing and storing its share of the tile: deterministic, no workspace, no
// atomics.
//
// This file is the form whose operands go through LDS: each wave copies its
// own A (BM x BK) and B (BK x BN) chunks with buffer_load ... lds (16 bytes
// per lane for 16-byte aligned rows, 4 bytes otherwise) into its own ring of S
// LDS stages and waits only on its own copies (s_waitcnt vmcnt): the main
// loop has no barrier. It serves 64x64 and 32x32 tiles whose rows of A, B
// and C are all 16-byte aligned, and the skinny 32x128 tiles. 128x128 tiles,
// and 64x64 and 32x32 tiles with unaligned rows, load their operands straight
// into registers instead (gemm_mfma_kreg.hpp, the same decomposition), which
// was measured faster there.
//
// This keeps the output-parallel decomposition of the LeetGPU write-up
// (section "V0", "Approach": outputs independent, each owned with its whole
// reduction by one block) at workgroup level; only the waves inside the
// workgroup share a tile's reduction.
//
// Chunks are BK = 8 deep (one MFMA step: reduction index 4g + t of a chunk for
// half-wave g at MFMA t), aligned to the END of the reduction as in the
// direct-copy kernel, so that only chunk 0 can reach below n = 0; each wave
// loads its first chunk through registers with zero fill (only wave 0's first
// chunk is chunk 0). With N >= 64 every wave owns at least two chunks, so a
// copy clamped to a wave's last chunk never reads chunk 0.
//
// LDS: stage s of every wave is a separate LDS object per operand (so that the
// compiler can tell a stage's reads from the copies into another), each holding
// the four waves' pieces. A rows are 8 floats (two quads) stored in the order
// q ^ swz(r), swz(r) = bit 2 ^ bit 3 of r: the 128-bit operand reads of 8
// consecutive rows from a multiple of 8 (32 banks), and of 16 from a multiple
// of 16 (64 banks), hit distinct 16-byte bank groups. B is row-major, BM
// floats per row. A copy fills 64 (4-byte copies) or 256 consecutive floats of
// a wave's piece; a lane's source address is free, so the layout is the same
// for both copy widths.
#pragma once

#include "gemm_mfma.hpp"
#include "gemm_mfma_dma.hpp"
#include "gemm_mfma_split.hpp"
#include "strip.hpp"

namespace fgr {

// BM x BN tiles: 64 x 64, 32 x 32, or the skinny 32 x 128 tile (few output
// rows, wide column blocks of B per workgroup). VA / VB: 16-byte copies of A / B
// (their rows 16-byte aligned), else 4-byte copies. STRIP: the launch also
// holds, after the tiles' workgroups, workgroups that compute the narrow
// column strip [tiles_n * BN, K) of C on the vector ALUs (strip.hpp).
template <int BM_, int S_, bool VA_, int BN_ = BM_, bool VB_ = VA_, bool STRIP_ = false>
struct KsplitConfig {
  static constexpr int BM = BM_, BN = BN_, BK = 8, S = S_;
  static constexpr bool kStrip = STRIP_;
  static constexpr bool VA = VA_, VB = VB_;
  static constexpr bool kReg = false;  // operands through LDS (gemm_mfma_kreg.hpp: through registers)
  static constexpr int kWaves = 4;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kRB = BM / 32, kCB = BN / 32;
  static constexpr int kACopyFloats = VA ? 4 : 1;  // floats per lane per copy
  static constexpr int kBCopyFloats = VB ? 4 : 1;
  static constexpr int kABlock = 64 * kACopyFloats;  // floats one copy fills
  static constexpr int kBBlock = 64 * kBCopyFloats;
  static constexpr int kPieceA = BM * BK;          // floats of one wave's A stage
  static constexpr int kPieceB = BK * BN;          // floats of one wave's B stage
  static constexpr int kACopies = kPieceA / kABlock;  // per wave per chunk
  static constexpr int kBCopies = kPieceB / kBBlock;
  static constexpr int kCopies = kACopies + kBCopies;
  static constexpr int kStageA = kWaves * kPieceA;  // floats of one LDS stage object of A
  static constexpr int kStageB = kWaves * kPieceB;
  // the reduction: a slice is one MFMA block's 16 accumulators of every lane
  static constexpr int kSlices = kRB * kCB;
  static constexpr int kSlicesPerObjA = kStageA / 1024;
  static constexpr int kSlicesPerObjB = kStageB / 1024;
  static constexpr int kSlicesPerWave = kSlices >= kWaves ? kSlices / kWaves : 1;

  static_assert((BM == BN && (BM == 32 || BM == 64)) || (BM == 32 && BN == 128), "64x64, 32x32 or 32x128 tiles");
  static_assert(kPieceA % kABlock == 0 && kPieceB % kBBlock == 0 && BN % kBCopyFloats == 0,
                "copies cover whole pieces");
  static_assert(S == 2 || S == 4, "an even ring depth: stage and operand buffer cycle together");
  static_assert(!STRIP_ || (BM == 64 && BN == 64), "the strip goes with 64x64 tiles");
  static_assert(kCopies * (S - 2) <= 63, "the wait count fits the vmcnt field");
  static_assert(S * (kStageA + kStageB) * 4 <= 160 * 1024, "LDS budget of a gfx950 workgroup");
  static_assert(kSlices <= S * kSlicesPerObjA && kSlices <= S * kSlicesPerObjB,
                "a partial tile fits in the stage objects of either operand");
};

__host__ __device__ __forceinline__ int a_swizzle2(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }

// Column (inside the 8-deep chunk) of the A element a copy puts at float
// position pos of a wave's A piece: row pos / 8, stored slot (pos % 8) / 4,
// which holds quad slot ^ a_swizzle2(row).
__host__ __device__ __forceinline__ int ksplit_a_col(int pos) {
  return 4 * (((pos % 8) / 4) ^ a_swizzle2(pos / 8)) + pos % 4;
}

// Float offset, in a wave's A piece, of quad g of row li (li < 32; rows li +
// 32 i sit 32 * 8 * i floats further on with the same swizzle).
__host__ __device__ __forceinline__ int ksplit_a_read(int li, int g) { return li * 8 + 4 * (g ^ a_swizzle2(li)); }

// A BYTES-wide copy per lane into LDS at lds + BYTES * lane, from a buffer
// resource (scalar registers) at soff + voff bytes, as in the direct-copy
// kernel: no vector address arithmetic per copy. The LDS destination is
// passed as an opaque wave-uniform integer: the compiler then cannot
// attribute the copy to one LDS object and does not pair it with the operand
// reads (which keep their objects), so it inserts no wait of its own before
// those reads. The kernel counts the copies in flight and waits for them
// itself (s_waitcnt vmcnt), the only way its reads are ordered after the
// copies they need.
template <int BYTES>  // 16 or 4
__device__ __forceinline__ void copy_to_lds_counted(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff,
                                                    float* lds) {
  uint32_t a = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)lds);
  asm volatile("" : "+s"(a));
  static_assert(BYTES == 16 || BYTES == 4, "16- or 4-byte copies");
  if constexpr (BYTES == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(uintptr_t)a, 16, voff, soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(uintptr_t)a, 4, voff, soff, 0, 0);
}

// Scheduling hints for NO memory instructions among MFMAS MFMAs, when there
// are MFMAs enough to interleave them one by one (else the default order).
template <int MASK, int MFMAS, int NO>
__device__ __forceinline__ void sched_spread() {
  if constexpr (NO > 0 && MFMAS >= NO) {
    sched_pairs<MASK, MFMAS / NO, NO>();
    if constexpr (MFMAS % NO) __builtin_amdgcn_sched_group_barrier(kSchedMfma, MFMAS % NO, 0);
  }
}

template <class T>
__global__ __launch_bounds__(T::kThreads) void gemm_mfma_ksplit_kernel(
    const float* __restrict__ A, const float* __restrict__ B, float* __restrict__ C, int M, int N,
    int K, int tiles_m, int tiles_n, int group, int parts, float* __restrict__ W, int first, int compact,
    int nfull) {
  constexpr int S = T::S, BK = T::BK, BN = T::BN;
  __shared__ __attribute__((aligned(1024))) float As0[T::kStageA];
  __shared__ __attribute__((aligned(1024))) float As1[T::kStageA];
  __shared__ __attribute__((aligned(1024))) float As2[T::kStageA];
  __shared__ __attribute__((aligned(1024))) float As3[T::kStageA];
  __shared__ __attribute__((aligned(1024))) float Bs0[T::kStageB];
  __shared__ __attribute__((aligned(1024))) float Bs1[T::kStageB];
  __shared__ __attribute__((aligned(1024))) float Bs2[T::kStageB];
  __shared__ __attribute__((aligned(1024))) float Bs3[T::kStageB];
  auto a_stage = [&](auto sc) __attribute__((always_inline)) -> float* {
    constexpr int s = decltype(sc)::value;
    if constexpr (s == 0) return As0;
    else if constexpr (s == 1) return As1;
    else if constexpr (s == 2) return As2;
    else return As3;
  };
  auto b_stage = [&](auto sc) __attribute__((always_inline)) -> float* {
    constexpr int s = decltype(sc)::value;
    if constexpr (s == 0) return Bs0;
    else if constexpr (s == 1) return Bs1;
    else if constexpr (s == 2) return Bs2;
    else return Bs3;
  };

  TsMarks ts;  // measurement build only (timestamps.hpp)
  ts.start();
  // workgroups past the tiles (STRIP): four rows of the column strip each,
  // staging B's strip in the first A stage object
  const int gx = T::kStrip ? tiles_m * tiles_n : (int)gridDim.x;
  if constexpr (T::kStrip) {
    if ((int)blockIdx.x >= gx) {
      strip_rows(A, B, C, M, N, K, tiles_n * BN, (int)blockIdx.x - gx, As0, T::kStageA);
      ts.loop_done();
      ts.finish(1);
      return;
    }
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31;
  const int lg = lane >> 5;
  const int piece_a = wave * T::kPieceA;  // this wave's offset inside every A stage object
  const int piece_b = wave * T::kPieceB;  // and B stage object

  // The launch covers tiles [first, first + nfull + ntiles) of the grouped
  // order. The first nfull workgroups take whole tiles [first, first + nfull)
  // (their whole reduction, results to C). The other gridDim.x - nfull take
  // the ntiles tiles after them, each split across workgroups when parts > 1:
  // parts x ntiles workgroups, logical id = part * ntiles + tile, so that
  // after the XCD renumbering the tiles of one part, which read the same
  // reduction range of A and B, run on the same XCD and share its L2. Part p
  // owns the chunks [nchunks p / parts, nchunks (p + 1) / parts) and writes
  // its partial tile to the workspace W instead of C: at its place in a copy
  // of C (W + p M K, row stride K) or, compact, to slot p ntiles + tile (BM x
  // BN floats, row stride BN); a second kernel adds the parts. Whole and split
  // tiles in one grid run side by side (two workgroups fit a CU): a last
  // partial wave of tiles then spreads over every CU next to the full wave
  // instead of running after it. At least 8 chunks per part give every wave
  // >= 2 of the part's chunks (dealt as below).
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
  // The part's chunks are dealt to the waves in turn: this wave's j-th chunk
  // is pc0 + wave + kWaves j, so that the four waves copy the four 32-byte
  // pieces of the same 128-byte lines of A at about the same time (with a
  // contiguous range per wave each line was fetched four times, chunks apart).
  const int nmine = pn > wave ? (pn - wave + T::kWaves - 1) / T::kWaves : 0;
  const int j_last = nmine - 1;
  auto chunk_n0 = [&](int j) __attribute__((always_inline)) {
    return n_first + BK * (pc0 + wave + T::kWaves * j);
  };

  // Copy j of a wave fills floats [j * kABlock, (j + 1) * kABlock) of its A
  // piece; lane L the kACopyFloats floats at position p = j * kABlock + L *
  // kACopyFloats (likewise for B).
  // In A, p is row p / 8, stored slot (p % 8) / 4, element p % 4, and the slot
  // holds quad slot ^ swz(row): the lane copies that quad's element (the whole
  // quad with 16-byte copies). Rows past M read row M - 1 (not stored).
  auto a_row_of = [&](int j) __attribute__((always_inline)) {
    return (j * T::kABlock + lane * T::kACopyFloats) / BK;
  };
  static_assert(BK == 8, "ksplit_a_col and ksplit_a_read are written for 8-deep chunks");
  auto a_col_of = [&](int j) __attribute__((always_inline)) {
    return ksplit_a_col(j * T::kABlock + lane * T::kACopyFloats);
  };
  auto a_ptr_of = [&](int j) __attribute__((always_inline)) {
    const int r = a_row_of(j);
    const int row = m0 + r < M ? m0 + r : M - 1;
    return A + (int64_t)row * N + a_col_of(j);
  };
  auto b_row_of = [&](int j) __attribute__((always_inline)) {
    return (j * T::kBBlock + lane * T::kBCopyFloats) / BN;
  };
  auto b_ptr_of = [&](int j) __attribute__((always_inline)) {
    const int c = k0 + (j * T::kBBlock + lane * T::kBCopyFloats) % BN;
    return B + (int64_t)b_row_of(j) * K + (c < K ? c : K - T::kBCopyFloats);
  };
  // a_src / b_src: the lane's sources in the wave's first chunk (loaded
  // through registers). The copies of later chunks read a buffer over the
  // tile's rows of A at a_off + 4 n0 bytes, and a buffer over rows [n0, n0 +
  // BK) of B at b_off (32-bit offsets: BM N and BK K floats at most 2^32
  // bytes, which the host checks).
  const int tile_rows = M - m0 < T::BM ? M - m0 : T::BM;
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A + (int64_t)m0 * N, (uint32_t)tile_rows * (uint32_t)N * 4u);
  const float* a_src[T::kACopies];
  uint32_t a_off[T::kACopies];
  int a_dst[T::kACopies], a_col[T::kACopies];
#pragma unroll
  for (int j = 0; j < T::kACopies; ++j) {
    a_dst[j] = piece_a + j * T::kABlock;
    a_src[j] = a_ptr_of(j);
    a_off[j] = (uint32_t)(a_src[j] - (A + (int64_t)m0 * N)) * 4u;
    a_col[j] = a_col_of(j);
  }
  // In B, p is row p / BN, column p % BN (columns past K read the last column,
  // or the last quad with 16-byte copies; not stored).
  const float* b_src[T::kBCopies];
  uint32_t b_off[T::kBCopies];
  int b_dst[T::kBCopies];
#pragma unroll
  for (int j = 0; j < T::kBCopies; ++j) {
    b_dst[j] = piece_b + j * T::kBBlock;
    b_src[j] = b_ptr_of(j);
    b_off[j] = (uint32_t)(b_src[j] - B) * 4u;
  }

  auto copy_chunk = [&](int j, float* As, float* Bs) __attribute__((always_inline)) {
    const int n0 = chunk_n0(j);
    const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(B + (int64_t)n0 * K, (uint32_t)(BK * K) * 4u);
#pragma unroll
    for (int j = 0; j < T::kACopies; ++j)
      copy_to_lds_counted<4 * T::kACopyFloats>(a_rsrc, a_off[j], (uint32_t)n0 * 4u, As + a_dst[j]);
#pragma unroll
    for (int j = 0; j < T::kBCopies; ++j) copy_to_lds_counted<4 * T::kBCopyFloats>(b_rsrc, b_off[j], 0u, Bs + b_dst[j]);
  };

  struct Frag {
    float4 a[T::kRB];
    float b[T::kCB][4];
  };
  // Operand read offsets, each one integer from the stage's start: a longer
  // chain of address steps hides the stage object from the compiler, which
  // then waits for every copy in flight before the read. A: quad lg of row li
  // (+ 32 i), stored at position lg ^ swz(li) (the same swizzle for every i).
  const int a_frag = piece_a + ksplit_a_read(li, lg);
  // lane column li of MFMA column block j is output column kCB li + j (see the
  // direct-copy kernel): one read gives a lane's B operands of all blocks
  const int b_frag = piece_b + 4 * lg * BN + T::kCB * li;
  typedef typename FloatVec<T::kCB>::type BVec;
  auto read_frag = [&](Frag& f, const float* As, const float* Bs) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < T::kRB; ++i)
      f.a[i] = *reinterpret_cast<const float4*>(As + a_frag + 32 * BK * i);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const BVec v = *reinterpret_cast<const BVec*>(Bs + b_frag + t * BN);
#pragma unroll
      for (int j = 0; j < T::kCB; ++j) f.b[j][t] = vec_get(v, j);
    }
  };

  f32x16 acc[T::kRB][T::kCB];
#pragma unroll
  for (int i = 0; i < T::kRB; ++i)
#pragma unroll
    for (int j = 0; j < T::kCB; ++j) acc[i][j] = f32x16{};
  // the MFMAs of reduction offsets t in [t0, t1) of a chunk
  auto mma = [&](const Frag& f, int t0, int t1) __attribute__((always_inline)) {
#pragma unroll
    for (int t = t0; t < t1; ++t)
#pragma unroll
      for (int i = 0; i < T::kRB; ++i)
#pragma unroll
        for (int j = 0; j < T::kCB; ++j) {
          const float av = t == 0 ? f.a[i].x : t == 1 ? f.a[i].y : t == 2 ? f.a[i].z : f.a[i].w;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, f.b[j][t], acc[i][j], 0, 0, 0);
        }
  };
  constexpr int kMfmasT = T::kRB * T::kCB;  // MFMAs per reduction offset t
  constexpr int kReads = T::kRB + 4;

  Frag f[2];
  // Ring fill with the wave's first chunk in stage OFF: that chunk through
  // registers (zero where n < 0), the next S - 2 copied into the stages after it.
  auto fill = [&](auto offc) __attribute__((always_inline)) {
    constexpr int OFF = decltype(offc)::value;
    constexpr int X = OFF & 1;  // operand buffer of the chunk in stage OFF
    using S0 = std::integral_constant<int, OFF>;
    const int n0 = chunk_n0(0);
    typedef typename std::conditional<T::VA, float4, float>::type CopyTA;
    typedef typename std::conditional<T::VB, float4, float>::type CopyTB;
    CopyTA va[T::kACopies];
    CopyTB vb[T::kBCopies];
    bool oka[T::kACopies], okb[T::kBCopies];
#pragma unroll
    for (int j = 0; j < T::kACopies; ++j) {
      oka[j] = n0 + a_col[j] >= 0;
      va[j] = *reinterpret_cast<const CopyTA*>(oka[j] ? a_src[j] + n0 : A);
    }
#pragma unroll
    for (int j = 0; j < T::kBCopies; ++j) {
      okb[j] = n0 + b_row_of(j) >= 0;
      vb[j] = *reinterpret_cast<const CopyTB*>(okb[j] ? b_src[j] + (int64_t)n0 * K : B);
    }
    static_for<1, S - 1>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      using Sj = std::integral_constant<int, (OFF + j) % S>;
      copy_chunk(min(j, j_last), a_stage(Sj{}), b_stage(Sj{}));
    });
    auto zero_out = [](auto v, bool ok) __attribute__((always_inline)) {
      if constexpr (std::is_same<decltype(v), float4>::value) return mask_quad(v, ok ? 0xfu : 0u);
      else return ok ? v : 0.f;
    };
#pragma unroll
    for (int j = 0; j < T::kACopies; ++j)
      *reinterpret_cast<CopyTA*>(a_stage(S0{}) + a_dst[j] + T::kACopyFloats * lane) = zero_out(va[j], oka[j]);
#pragma unroll
    for (int j = 0; j < T::kBCopies; ++j)
      *reinterpret_cast<CopyTB*>(b_stage(S0{}) + b_dst[j] + T::kBCopyFloats * lane) = zero_out(vb[j], okb[j]);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
    __builtin_amdgcn_sched_barrier(0);
    read_frag(f[X], a_stage(S0{}), b_stage(S0{}));
  };

  // Chunk c in stage s, one MFMA step; f[X] holds its operands on entry, and
  // f[X ^ 1] receives chunk c + 1's. The copy of chunk c + S - 1 (clamped to
  // the wave's last chunk) goes to the stage chunk c - 1 used; chunk c + 1's
  // copies were issued S - 2 chunks ago.
  auto chunk = [&](auto sc, auto xc, int c) __attribute__((always_inline)) {
    constexpr int s = decltype(sc)::value, X = decltype(xc)::value;
    using Sn = std::integral_constant<int, (s + 1) % S>;
    using Sp = std::integral_constant<int, (s + S - 1) % S>;
    // t = 0: the copies among its MFMAs
    copy_chunk(min(c + S - 1, j_last), a_stage(Sp{}), b_stage(Sp{}));
    mma(f[X], 0, 1);
    sched_spread<kSchedVmemRead, kMfmasT, T::kCopies>();
    __builtin_amdgcn_sched_barrier(0);
    // chunk c + 1 has landed in LDS: its operand reads among the MFMAs of t = 1..3
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(T::kCopies * (S - 2)));
    __builtin_amdgcn_sched_barrier(0);
    read_frag(f[X ^ 1], a_stage(Sn{}), b_stage(Sn{}));
    mma(f[X], 1, 4);
    sched_spread<kSchedDsRead, 3 * kMfmasT, kReads>();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Chunk k of a group of S uses stage k and operand buffer k & 1 (S is
  // even, so a group always starts with buffer 0). The wave's (count mod S)
  // leading chunks run in stages S - r .. S - 1 so that the loop below starts
  // at stage 0 with whole groups; one loop, so the accumulators stay in place.
  const int lead = nmine % S;
  static_for<0, S>([&](auto rc) {
    constexpr int R = decltype(rc)::value;
    if (lead == R) {
      fill(std::integral_constant<int, (S - R) % S>{});
      static_for<0, R>([&](auto kc) {
        constexpr int k = S - R + decltype(kc)::value;
        chunk(std::integral_constant<int, k>{}, std::integral_constant<int, k & 1>{}, k - (S - R));
      });
    }
  });
  for (int c = lead; c < nmine; c += S)
    static_for<0, S>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      chunk(std::integral_constant<int, k>{}, std::integral_constant<int, k & 1>{}, c + k);
    });
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));  // stray copies past the wave's last chunk
  ts.loop_done();

  // The four partial tiles are added in wave order, ((p0 + p1) + p2) + p3,
  // through LDS (the staging is free once every wave is past the first
  // barrier), two partials at a time, in the stage objects of A (waves 0, 2)
  // or of B (waves 1, 3). Slice t of a partial (MFMA block i = t / kCB,
  // j = t % kCB: 16 accumulators of every lane) lives in object
  // t / kSlicesPerObjA (or B), lane-major as float4. Wave w sums and stores slices
  // [w kSlicesPerWave, (w + 1) kSlicesPerWave).
  constexpr int kSPW = T::kSlicesPerWave;
  auto slice_ptr = [&](auto tc, bool use_b) __attribute__((always_inline)) -> float* {
    constexpr int t = decltype(tc)::value;
    using OA = std::integral_constant<int, t / T::kSlicesPerObjA>;
    using OB = std::integral_constant<int, t / T::kSlicesPerObjB>;
    return (use_b ? b_stage(OB{}) + (t % T::kSlicesPerObjB) * 1024 : a_stage(OA{}) + (t % T::kSlicesPerObjA) * 1024) +
           4 * lane;
  };
  auto put = [&](bool use_b) __attribute__((always_inline)) {
    static_for<0, T::kSlices>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      float* p = slice_ptr(tc, use_b);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(p + 256 * q) =
            make_float4(acc[t / T::kCB][t % T::kCB][4 * q], acc[t / T::kCB][t % T::kCB][4 * q + 1],
                        acc[t / T::kCB][t % T::kCB][4 * q + 2], acc[t / T::kCB][t % T::kCB][4 * q + 3]);
    });
  };
  float sum[kSPW][16];
  // sum (+)= this wave's slices of the partial in the A (use_b false) or B objects
  auto take = [&](bool use_b, bool first) __attribute__((always_inline)) {
    static_for<0, T::kSlices>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      if (wave != t / kSPW) return;
      const float* p = slice_ptr(tc, use_b);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(p + 256 * q);
        const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) sum[t % kSPW][4 * q + k] = first ? e[k] : sum[t % kSPW][4 * q + k] + e[k];
      }
    });
  };
  __syncthreads();
  if (wave == 0) put(false);
  if (wave == 1) put(true);
  __syncthreads();
  take(false, true);
  take(true, false);
  __syncthreads();
  if (wave == 2) put(false);
  if (wave == 3) put(true);
  __syncthreads();
  take(false, false);
  take(true, false);

  if (wave * kSPW >= T::kSlices) return;  // small tiles: fewer slices than waves
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
#pragma unroll
  for (int u = 0; u < kSPW; ++u) {
    const int t = wave * kSPW + u;
    const int i = t / T::kCB, j = t % T::kCB;
    const int col = T::kCB * li + j;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int row = i * 32 + 8 * (rr / 4) + 4 * lg + (rr % 4);
      if (k0 + col < K && m0 + row < M) Ct[(uint64_t)row * ldc + (uint32_t)col] = sum[u][rr];
    }
  }
  ts.finish();  // wave 0 always stores, so thread 0 gets here
}

}  // namespace fgr
