// FP32 MFMA GEMM for whole-device shapes, fed by direct global->LDS copies
// through a ring of S LDS stages.
//
// Same product, output tiling and operand layout as gemm_mfma.hpp, for
// N >= 64. Every reduction chunk but the first is copied from global memory
// straight into LDS with buffer_load_dwordx4 ... lds (16 bytes per lane,
// written to LDS at the M0 base + 16 * lane) when rows are 16-byte aligned
// (N % 4 == 0, K % 4 == 0, aligned bases), else with buffer_load_dword ...
// lds (4 bytes per lane, four times as many copies, the same LDS layout), the
// gfx950 counterpart of the cp.async copies of the LeetGPU write-up's section
// "V4: Hardware-Asynchronous cp.async Pipeline". The data never passes
// through VGPRs, so the copies take no register-file bandwidth from the MFMAs
// and no LDS write instructions are issued. The write-up's Triton solution
// runs a 3-stage software pipeline; here the ring has S stages (3..5) of
// BK = 16 reduction indices.
//
// Copy addressing. A copy's source is a buffer resource in scalar registers
// (A: the workgroup's rows of A; B: the chunk's 16 rows of B, rebuilt per
// chunk), a per-lane 32-bit byte offset fixed for the whole loop, and for A a
// scalar offset that advances with the chunk. A copy is thus one instruction
// with no vector address arithmetic; with 64-bit per-lane addresses (one
// vector add per copy in the loop) the timed shape 8192 x 6144 x 4096 ran
// 1.6% slower (2743 against 2699 us). The 32-bit offsets bound the shapes this
// kernel takes: 256 rows of A span at most 2^32 bytes (N <= kDmaMaxN) and 16
// rows of B too (K <= kDmaMaxK); the host routes larger ones elsewhere.
//
// Pipeline. Chunk c lives in stage (c + off) mod S. While chunk c is
// multiplied, this wave copies chunk c + S - 1 into the stage that chunk c - 1
// used; that stage was released by the barrier before chunk c - 1's last
// step. Before the last step of chunk c (which reads the first operands of
// chunk c + 1) each wave waits until at most the copies of the S - 2 newer
// chunks are in flight (s_waitcnt vmcnt), then the workgroup meets at one
// s_barrier, so every wave's copies of chunk c + 1 have landed. A chunk's
// copies thus have about S - 2 chunks of MFMA work to arrive, and the barrier
// no longer waits on memory latency. Copies past the last chunk re-read the
// last chunk into a stage that is never read again, which keeps the wait
// counts the same in every chunk.
//
// Ragged edges. Rows of A beyond M and columns of B beyond K only feed
// outputs that are never stored, so their copies read a clamped in-bounds
// address (the last row / last column quad) and the epilogue guards the
// stores. Reduction indices beyond N would feed real outputs and must be
// zero: the chunks are aligned to the END of the reduction (chunk c covers
// n in [N - BK*(T - c), N - BK*(T - c) + BK), T = ceil(N / BK)), so that only
// chunk 0 can reach below n = 0; chunk 0 is loaded through registers with
// every element outside [0, N) set to zero (the zero padding of the study
// notes' section 4) and written to LDS in the same layout. N >= 64 keeps
// T >= 2, so a clamped copy never reads chunk 0.
//
// LDS layout (each stage a separate LDS object, so that the compiler can tell
// the reads of one stage from the copies into another):
//   A stage: BM rows x BK floats, unpadded; row r holds its 4 quads in the
//     order q ^ swz(r), swz(r) = ((r >> 1) & 3) ^ ((r >> 3) & 1). One copy
//     instruction fills 16 consecutive rows (4 with 4-byte copies: a lane's
//     source address is free, so the swizzle holds either way). The MFMA
//     operand read of lane (i, g) fetches quad 2h + g of row i; over any 8
//     consecutive rows from a multiple of 8, and over 16 from a multiple of
//     16, the swizzle sends these reads to distinct 16-byte bank groups (32 or
//     64 banks).
//   B stage: BK rows x BN floats, row-major; one copy instruction per row (a
//     quarter row with 4-byte copies).
#pragma once

#include "gemm_mfma.hpp"
#include "timestamps.hpp"

namespace fgr {

typedef __attribute__((address_space(3))) void lds_void_t;

// VA / VB: 16-byte copies of A / B (rows 16-byte aligned: N % 4 == 0 and an
// aligned A; K % 4 == 0 and an aligned B), otherwise 4-byte copies, four
// times as many, into the same LDS layout (any 4-byte alignment). VC:
// 128-bit stores of C (K % 4 == 0, aligned C). VEC: all three.
template <int S_, bool VA_ = true, bool VB_ = VA_, bool VC_ = VB_>
struct DmaConfig {
  static constexpr int BM = 256, BN = 256, BK = 16, WM = 2, WN = 2, S = S_;
  static constexpr bool VA = VA_, VB = VB_, VC = VC_, VEC = VA_ && VB_ && VC_;
  static constexpr int kACopyFloats = VA ? 4 : 1;  // floats per lane per copy
  static constexpr int kBCopyFloats = VB ? 4 : 1;
  static constexpr int kABlock = 64 * kACopyFloats;  // LDS floats one copy fills
  static constexpr int kBBlock = 64 * kBCopyFloats;
  static constexpr int kThreads = WM * WN * 64;
  static constexpr int kWaves = WM * WN;
  static constexpr int kWaveM = BM / WM;
  static constexpr int kWaveN = BN / WN;
  static constexpr int kRB = kWaveM / 32;
  static constexpr int kCB = kWaveN / 32;
  static constexpr int kQuads = BK / 4;                      // quads per A row
  static constexpr int kStage = BM * BK;                     // floats, A and B stages alike
  static constexpr int kACopies = kStage / kABlock / kWaves;  // per wave per chunk
  static constexpr int kBCopies = kStage / kBBlock / kWaves;
  static constexpr int kCopies = kACopies + kBCopies;

  static_assert(BN % kBBlock == 0, "a B copy stays inside one row");
  static_assert(BM * BK == BK * BN, "A and B stages have one size");
  static_assert(kQuads == 4, "the A swizzle is written for 4 quads per row");
  static_assert(kCB == 4, "B operands are read as 4 adjacent floats");
  static_assert(kRB * kCB * 16 == 256, "the accumulators fill the 256 AGPRs");
  static_assert(kStage % (kABlock * kWaves) == 0 && kStage % (kBBlock * kWaves) == 0,
                "copies split evenly over waves");
  static_assert(S >= 3 && S <= 5, "a ring of 3 to 5 stages");
  static_assert(kCopies * (S - 2) <= 63, "the wait count fits the vmcnt field");
  static_assert(S * 2 * kStage * 4 <= 160 * 1024, "LDS budget of a gfx950 workgroup");
};

__host__ __device__ __forceinline__ int a_swizzle(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }

// Column (inside the 16-deep chunk) of the A element a copy puts at float
// position pos of an A stage: row pos / 16, stored slot (pos % 16) / 4, which
// holds quad slot ^ a_swizzle(row).
__host__ __device__ __forceinline__ int dma_a_col(int pos) {
  return 4 * (((pos % 16) / 4) ^ a_swizzle(pos / 16)) + pos % 4;
}

// Float offset, in an A stage, of quad q of row row0 + 32 i (row0's swizzle
// serves every i: 32 i leaves bits 1-3 of the row unchanged).
__host__ __device__ __forceinline__ int dma_a_read(int row0, int i, int q) {
  return (row0 + 32 * i) * 16 + 4 * (q ^ a_swizzle(row0));
}

// s_waitcnt immediate (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8) that waits until at most `vm` vector-memory operations are
// outstanding and every LDS operation is done.
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | (7 << 4) | (((vm >> 4) & 3) << 14); }

// Largest N and K whose copy offsets fit the buffers' 32-bit byte range:
// 256 rows of A (BM N floats) and 16 rows of B (BK K floats).
constexpr int kDmaMaxN = (int)(0xffffffffu / (256u * 4u));
constexpr int kDmaMaxK = (int)(0xffffffffu / (16u * 4u));

// BYTES (16 or 4) bytes per lane from the buffer at soff + voff into LDS at
// lds + BYTES * lane (lds and soff are wave-uniform). A plain device
// function: the builtin has no host form.
template <int BYTES>
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, float* lds) {
  static_assert(BYTES == 16 || BYTES == 4, "16- or 4-byte copies");
  if constexpr (BYTES == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds, 16, voff, soff, 0, 0);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds, 4, voff, soff, 0, 0);
}

template <class T>
__global__ __launch_bounds__(T::kThreads) void gemm_mfma_dma_kernel(
    const float* __restrict__ A, const float* __restrict__ B, float* __restrict__ C, int M, int N,
    int K, int tiles_m, int tiles_n, int group) {
  constexpr int S = T::S, BK = T::BK, BN = T::BN, WN = T::WN;
  using I0 = std::integral_constant<int, 0>;
  using ICopies = std::integral_constant<int, T::kCopies>;
  __shared__ __attribute__((aligned(1024))) float As0[T::kStage];
  __shared__ __attribute__((aligned(1024))) float As1[T::kStage];
  __shared__ __attribute__((aligned(1024))) float As2[T::kStage];
  __shared__ __attribute__((aligned(1024))) float As3[T::kStage];
  __shared__ __attribute__((aligned(1024))) float As4[T::kStage];
  __shared__ __attribute__((aligned(1024))) float Bs0[T::kStage];
  __shared__ __attribute__((aligned(1024))) float Bs1[T::kStage];
  __shared__ __attribute__((aligned(1024))) float Bs2[T::kStage];
  __shared__ __attribute__((aligned(1024))) float Bs3[T::kStage];
  __shared__ __attribute__((aligned(1024))) float Bs4[T::kStage];
  // stage by compile-time index (stages beyond S are never referenced)
  auto a_stage = [&](auto sc) __attribute__((always_inline)) -> float* {
    constexpr int s = decltype(sc)::value;
    if constexpr (s == 0) return As0;
    else if constexpr (s == 1) return As1;
    else if constexpr (s == 2) return As2;
    else if constexpr (s == 3) return As3;
    else return As4;
  };
  auto b_stage = [&](auto sc) __attribute__((always_inline)) -> float* {
    constexpr int s = decltype(sc)::value;
    if constexpr (s == 0) return Bs0;
    else if constexpr (s == 1) return Bs1;
    else if constexpr (s == 2) return Bs2;
    else if constexpr (s == 3) return Bs3;
    else return Bs4;
  };

  TsMarks ts;  // measurement build only (timestamps.hpp)
  ts.start();
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
  const int m0 = tm * T::BM;
  const int k0 = tn * BN;

  // Copy sources for this lane. Copy j of this wave fills LDS floats
  // [blk * kABlock, (blk + 1) * kABlock) of an A stage, blk = wave * kACopies
  // + j; lane L fills the kACopyFloats floats at position p = blk * kABlock +
  // L * kACopyFloats (likewise for B). In the A stage position p is row p / 16, stored slot
  // (p % 16) / 4, element p % 4, and the slot holds quad slot ^ swz(row), so
  // the lane reads that quad's element (the whole quad with 16-byte copies).
  // Rows past M read row M - 1 instead (their outputs are not stored).
  // a_src is the lane's source in chunk 0 (loaded through registers); the
  // copies of later chunks read the A buffer (the tile's rows) at a_off plus
  // 4 n0 bytes.
  const int tile_rows = M - m0 < T::BM ? M - m0 : T::BM;
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A + (int64_t)m0 * N, (uint32_t)tile_rows * (uint32_t)N * 4u);
  const float* a_src[T::kACopies];
  uint32_t a_off[T::kACopies];  // byte offset of the lane's source in the A buffer at n0 = 0
  int a_dst[T::kACopies];       // LDS float offset of the copy's block
  int a_col[T::kACopies];       // column of the lane's first element inside the chunk
#pragma unroll
  for (int j = 0; j < T::kACopies; ++j) {
    const int blk = wave * T::kACopies + j;
    const int pos = blk * T::kABlock + lane * T::kACopyFloats;
    const int r = pos / BK;
    const int c = dma_a_col(pos);
    const int row = m0 + r < M ? m0 + r : M - 1;
    a_src[j] = A + (int64_t)row * N + c;
    a_off[j] = (uint32_t)((row - m0) * N + c) * 4u;
    a_dst[j] = blk * T::kABlock;
    a_col[j] = c;
  }
  // In the B stage position p is row p / 256, column p % 256 (columns past K
  // read the last column, or the last quad with 16-byte copies; not stored).
  // The copies of the chunk at n0 read a buffer over rows [n0, n0 + BK) of B
  // at b_off.
  const float* b_src[T::kBCopies];
  uint32_t b_off[T::kBCopies];
  int b_dst[T::kBCopies];
  int b_row[T::kBCopies];
#pragma unroll
  for (int j = 0; j < T::kBCopies; ++j) {
    const int blk = wave * T::kBCopies + j;
    const int pos = blk * T::kBBlock + lane * T::kBCopyFloats;
    const int r = pos / BN;
    const int c = k0 + pos % BN;
    const int col = c < K ? c : K - T::kBCopyFloats;
    b_src[j] = B + (int64_t)r * K + col;
    b_off[j] = (uint32_t)(r * K + col) * 4u;
    b_dst[j] = blk * T::kBBlock;
    b_row[j] = r;
  }

  // copies [P0, P1) of this wave's kCopies (A first, then B) of the chunk at n0
  auto copy_part = [&](auto p0c, auto p1c, int n0, float* As, float* Bs) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(B + (int64_t)n0 * K, (uint32_t)(BK * K) * 4u);
    static_for<decltype(p0c)::value, decltype(p1c)::value>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      if constexpr (p < T::kACopies) {
        copy_to_lds<4 * T::kACopyFloats>(a_rsrc, a_off[p], (uint32_t)n0 * 4u, As + a_dst[p]);
      } else {
        copy_to_lds<4 * T::kBCopyFloats>(b_rsrc, b_off[p - T::kACopies], 0u, Bs + b_dst[p - T::kACopies]);
      }
    });
  };

  struct Frag {
    float4 a[T::kRB];
    float b[T::kCB][4];
  };
  // Row of A block i read by this lane, and its swizzle (the same for every
  // block: blocks start at multiples of 32 and the swizzle reads bits 1-3).
  const int a_row0 = wm * T::kWaveM + li;
  // Output columns inside the wave tile are interleaved across the MFMA
  // column blocks: lane column li of block j is column 4 * li + j, so one
  // lane's B operands for all four blocks are 4 consecutive floats of a row
  // (one 128-bit LDS read). Every output keeps its own column of B, so the
  // product is unchanged; the epilogue writes with the same mapping.
  const int b_frag = 4 * lg * BN + wn * T::kWaveN + 4 * li;
  auto read_frag = [&](Frag& f, const float* As, const float* Bs, int h) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < T::kRB; ++i)
      f.a[i] = *reinterpret_cast<const float4*>(As + dma_a_read(a_row0, i, 2 * h + lg));
    const float* Bh = Bs + b_frag + 8 * h * BN;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float4 v = *reinterpret_cast<const float4*>(Bh + t * BN);
      f.b[0][t] = v.x;
      f.b[1][t] = v.y;
      f.b[2][t] = v.z;
      f.b[3][t] = v.w;
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

  constexpr int kMfmas = T::kRB * T::kCB * 4;  // per step of 8 reduction indices
  constexpr int kReads = T::kRB + 4;
  const int nchunks = (N + BK - 1) / BK;
  const int n_first = N - BK * nchunks;  // in (-BK, 0]
  Frag f[2];

  // Pipeline fill with chunk 0 in stage OFF: chunk 0 through registers (zero
  // outside [0, N)), chunks 1 .. S - 2 copied into the stages after it.
  // With 16-byte copies of A, N % 4 == 0 and n_first % 4 == 0, so a quad is
  // wholly inside or outside.
  auto fill = [&](auto offc) __attribute__((always_inline)) {
    constexpr int OFF = decltype(offc)::value;
    using S0 = std::integral_constant<int, OFF>;
    typedef typename std::conditional<T::VA, float4, float>::type CopyTA;
    typedef typename std::conditional<T::VB, float4, float>::type CopyTB;
    CopyTA va[T::kACopies];
    CopyTB vb[T::kBCopies];
    bool oka[T::kACopies], okb[T::kBCopies];
#pragma unroll
    for (int j = 0; j < T::kACopies; ++j) {
      oka[j] = n_first + a_col[j] >= 0;
      va[j] = *reinterpret_cast<const CopyTA*>(oka[j] ? a_src[j] + n_first : A);
    }
#pragma unroll
    for (int j = 0; j < T::kBCopies; ++j) {
      okb[j] = n_first + b_row[j] >= 0;
      vb[j] = *reinterpret_cast<const CopyTB*>(okb[j] ? b_src[j] + (int64_t)n_first * K : B);
    }
    static_for<1, S - 1>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      using Sj = std::integral_constant<int, (OFF + j) % S>;
      copy_part(I0{}, ICopies{}, n_first + BK * min(j, nchunks - 1), a_stage(Sj{}), b_stage(Sj{}));
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
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frag(f[0], a_stage(S0{}), b_stage(S0{}), 0);
  };

  // Chunk c in stage s (two steps of 8 reduction indices). f[0] holds its
  // first operands on entry and the next chunk's on exit.
  auto chunk = [&](auto sc, int c) __attribute__((always_inline)) {
    constexpr int s = decltype(sc)::value;
    using Ss = std::integral_constant<int, s>;
    using Sn = std::integral_constant<int, (s + 1) % S>;
    using Sp = std::integral_constant<int, (s + S - 1) % S>;
    copy_part(I0{}, ICopies{}, n_first + BK * min(c + S - 1, nchunks - 1), a_stage(Sp{}), b_stage(Sp{}));
    read_frag(f[1], a_stage(Ss{}), b_stage(Ss{}), 1);
    mma(f[0]);
    // an MFMA first: the loop-carried operands are ready, the new reads are not
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    sched_interleave<kMfmas - 1, T::kCopies, 0, kReads>();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(T::kCopies * (S - 2)));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frag(f[0], a_stage(Sn{}), b_stage(Sn{}), 0);
    mma(f[1]);
    sched_interleave<kMfmas, 0, 0, kReads>();
    __builtin_amdgcn_sched_barrier(0);
  };

  // The nchunks mod S leading chunks run in stages S - r .. S - 1, so the loop
  // always starts at stage 0 with whole groups of S chunks. (A loop followed
  // by a partial group instead makes the register allocator shuttle
  // accumulators between AGPRs at every iteration.)
  const int r = nchunks % S;
  static_for<0, S>([&](auto rc) {
    constexpr int R = decltype(rc)::value;
    if (r == R) {
      fill(std::integral_constant<int, (S - R) % S>{});
      static_for<0, R>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        chunk(std::integral_constant<int, S - R + k>{}, k);
      });
    }
  });
  for (int c = r; c < nchunks; c += S)
    static_for<0, S>([&](auto sc) { chunk(sc, c + decltype(sc)::value); });
  // no copy may still be writing LDS when the workgroup ends
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
  ts.loop_done();

  // Epilogue. Offsets from the tile's corner (a wave-uniform base) are
  // row * K + col, 64-bit: 256 rows of a K beyond 2^24 already pass 2^32.
  // With 16-byte rows (K % 4 == 0) a lane's 4 adjacent columns start at a
  // multiple of 4, so they are wholly inside or outside; otherwise each column
  // is guarded and stored alone.
  // The 32-bit-store forms take the lane's index afresh from mbcnt, so that
  // nothing derived from it has to stay live across the loop (their loops
  // leave no register for it).
  int eli = li, elg = lg;
  if constexpr (!T::VC) {
    const int elane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    eli = elane & 31;
    elg = elane >> 5;
  }
  float* const Ct = C + (int64_t)m0 * K + k0;
  const int col = wn * T::kWaveN + 4 * eli;
  const bool col_ok = k0 + col < K;
#pragma unroll
  for (int i = 0; i < T::kRB; ++i)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int row = wm * T::kWaveM + i * 32 + 8 * (rr / 4) + 4 * elg + (rr % 4);
      if (col_ok && m0 + row < M) {
        float* dst = Ct + (uint64_t)row * (uint32_t)K + (uint32_t)col;
        if constexpr (T::VC) {
          *reinterpret_cast<float4*>(dst) = make_float4(acc[i][0][rr], acc[i][1][rr], acc[i][2][rr], acc[i][3][rr]);
        } else {
#pragma unroll
          for (int j = 0; j < T::kCB; ++j)
            if (k0 + col + j < K) dst[j] = acc[i][j][rr];
        }
      }
    }
  ts.finish();
}

}  // namespace fgr
