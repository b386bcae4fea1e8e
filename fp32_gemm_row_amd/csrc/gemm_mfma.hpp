// FP32 matrix-core (MFMA) GEMM for gfx950: C[M,K] = A[M,N] x B[N,K], row-major.
//
// The tiling follows the shared-memory / register-tiling line of "LeetGPU |
// 02_Matrix_Multiplication" (sections "V1: Original 16 x 16 Shared-Memory
// Tiling", "V1: Two-Dimensional Thread Tiling", "V2: Vectorized float4
// Transfers", "V3: Register Prefetch and Double-Buffered Shared Memory") and
// the T x T tile argument of "分块计算与矩阵乘法" (section 2), re-designed for CDNA4:
//
//  * one workgroup owns a BM x BN tile of C and the whole reduction over N
//    (outputs are independent; no cross-workgroup reduction);
//  * the reduction advances in chunks of BK: each chunk of A (BM x BK) and of
//    B (BK x BN) is fetched with 128-bit loads (32-bit loads when rows are not
//    16-byte aligned) into registers, written to one of two LDS buffers, and
//    consumed by v_mfma_f32_32x32x2_f32 from the other buffer - one barrier
//    per chunk (the register-prefetch double buffer of the V3 section);
//  * each wave owns a (BM/WM) x (BN/WN) sub-tile held in FP32 accumulators,
//    32 x 32 per MFMA block; an MFMA step contracts two reduction indices,
//    one per half-wave;
//  * out-of-range rows, columns and reduction indices are zero-filled in LDS
//    and never loaded (the zero-padding rule of the study notes, section 4,
//    and of the tutorial, section 2); stores are guarded by row < M, col < K.
//
// Operand layouts of v_mfma_f32_32x32x2_f32 (wave64, checked on the device):
//   A operand: lane l holds A[i = l % 32][kk = l / 32]
//   B operand: lane l holds B[kk = l / 32][j = l % 32]
//   D (16 floats per lane): element r of lane l is D[8*(r/4) + 4*(l/32) + r%4][l % 32]
//
// Reduction order: any permutation of the reduction index applied to both
// operands leaves the product unchanged. Lane half g of an MFMA step (t, h)
// takes reduction index n = 8h + 4g + t inside the chunk, so that a lane reads
// its four A values n = 8h+4g .. 8h+4g+3 with one 128-bit LDS read and feeds
// them to four consecutive MFMAs, while B is read as one 32-bit value per lane
// per step (32 consecutive columns per half-wave, conflict-free).
//
// LDS layout: A chunk row-major with a row pitch of BK+4 floats (80 bytes for
// BK = 16): eight consecutive rows read at the same column land in eight
// disjoint groups of four banks, so the 128-bit fragment reads are
// conflict-free. B chunk row-major with pitch BN.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fgr {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each

// Workgroups are dispatched round-robin over the XCDs (id % 8). Renumber them
// so that consecutive logical ids run on the same XCD and share its L2.
__host__ __device__ __forceinline__ int xcd_remap(int wg, int nwg) {
  const int xcd = wg % kNumXcd;
  const int local = wg / kNumXcd;
  const int per = nwg / kNumXcd;
  const int rem = nwg % kNumXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

// Grouped order (the program-id regrouping of the Triton section of the
// LeetGPU write-up): walk `group` tile-rows at a time, row index fastest, so
// that neighbouring logical ids share rows of A and columns of B.
__host__ __device__ __forceinline__ void grouped_tile(int logical, int tiles_m, int tiles_n, int group,
                                             int& tm, int& tn) {
  const int per_group = group * tiles_n;
  const int g = logical / per_group;
  const int first_m = g * group;
  const int rows_left = tiles_m - first_m;
  const int gsz = rows_left < group ? rows_left : group;
  const int in = logical - g * per_group;
  tm = first_m + in % gsz;
  tn = in / gsz;
}

// Compile-time shape of one kernel instance.
//   BM x BN   output tile of a workgroup;  BK  reduction chunk per LDS stage
//   WM x WN   waves per workgroup (each owns a (BM/WM) x (BN/WN) sub-tile)
//   MINB      workgroups per CU the register budget must allow
//   BUFS      LDS buffers: 2 = double buffer with register prefetch (the
//             pipeline below), 1 = one buffer, loads and MFMAs in turn (the
//             single-buffer control of the controlled comparison)
template <int BM_, int BN_, int BK_, int WM_, int WN_, int MINB_ = 1, int BUFS_ = 2>
struct MfmaConfig {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static constexpr int kMinBlocks = MINB_;
  static constexpr int kBufs = BUFS_;
  static constexpr int kThreads = WM * WN * 64;
  static constexpr int kWaveM = BM / WM;  // rows of C per wave
  static constexpr int kWaveN = BN / WN;  // columns of C per wave
  static constexpr int kRB = kWaveM / 32;  // 32x32 MFMA blocks per wave, down
  static constexpr int kCB = kWaveN / 32;  // and across
  static constexpr int kLdA = BK + 4;      // padded A pitch in LDS (floats)
  static constexpr int kLdB = BN;          // B pitch in LDS (floats)
  static constexpr int kAQuads = BK / 4;   // float4 per A chunk row
  static constexpr int kBQuads = BN / 4;   // float4 per B chunk row
  static constexpr int kAPerThread = BM * BK / 4 / kThreads;
  static constexpr int kBPerThread = BK * BN / 4 / kThreads;
  static constexpr int kLdsFloats = kBufs * (BM * kLdA + BK * kLdB);

  static_assert(kWaveM % 32 == 0 && kWaveN % 32 == 0, "wave tile must be a multiple of 32x32");
  static_assert(BK % 16 == 0, "BK must be a multiple of 16 (an even number of half-steps)");
  static_assert(BM * BK / 4 % kThreads == 0, "A chunk must split evenly over threads");
  static_assert(BK * BN / 4 % kThreads == 0, "B chunk must split evenly over threads");
  static_assert(kThreads % kAQuads == 0 && kThreads % kBQuads == 0,
                "a thread must keep the same column quad in every load slot");
  static_assert(kLdsFloats * 4 <= 160 * 1024, "LDS budget of a gfx950 workgroup");
  static_assert(kBufs == 1 || kBufs == 2, "one or two LDS buffers");
};

// One float4 slot of a chunk, loaded branch-free: an element outside the
// matrix reads a harmless in-bounds address instead (`safe`, the matrix base)
// and its bit in `ok` is cleared; mask_quad() then replaces it by zero when
// the slot is written to LDS, so padding never carries real data. VEC: the
// four elements are all inside or all outside (rows 16-byte aligned, extent a
// multiple of 4) and one 128-bit load is used; otherwise each element is
// checked and loaded on its own.
template <bool VEC>
__device__ __forceinline__ float4 load_quad(const float* __restrict__ p, const float* __restrict__ safe,
                                            bool row_ok, int col, int ncols, unsigned& ok) {
  if (VEC) {
    const bool in = row_ok && col < ncols;
    ok = in ? 0xfu : 0u;
    return *reinterpret_cast<const float4*>(in ? p : safe);
  } else {
    float e[4];
    ok = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool in = row_ok && col + i < ncols;
      ok |= in ? 1u << i : 0u;
      e[i] = *(in ? p + i : safe);
    }
    return make_float4(e[0], e[1], e[2], e[3]);
  }
}

__device__ __forceinline__ float4 mask_quad(float4 v, unsigned ok) {
  return make_float4(ok & 1u ? v.x : 0.f, ok & 2u ? v.y : 0.f, ok & 4u ? v.z : 0.f, ok & 8u ? v.w : 0.f);
}

// V (float2 or float4) consecutive floats at an address that is only 4-byte
// aligned, and the store of such a vector. On gfx9-family GPUs global loads and
// stores of two or more dwords need only dword alignment; the compiler emits
// one global_load_dwordx2 / x4 (store) for these.
// Raw buffer resource over `bytes` bytes from `base` (word 3 as on every
// gfx9-family GPU: raw buffer, 32-bit data). Loads through it take a 32-bit
// per-lane offset and a 32-bit scalar offset, so a kernel that keeps its
// per-lane offsets fixed and moves a scalar one (or the base) per chunk
// issues its loads with no vector address arithmetic. A load at an offset at
// or past `bytes` returns zeros (the hardware's range check); the kernels'
// loads all stay inside.
constexpr int kBufferWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const float* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, (int)bytes, kBufferWord3);
}

// The k-split kernels address a tile's rows_a rows of A and a chunk's 8 rows
// of B with 32-bit byte offsets: both spans must stay within 2^32 bytes.
__host__ __device__ constexpr bool ksplit_offsets_fit(int rows_a, int N, int K) {
  return (uint64_t)rows_a * (uint64_t)N * 4u <= 0xffffffffu && (uint64_t)K * 32u <= 0xffffffffu;
}

template <class V>
__device__ __forceinline__ V load_dwords(const float* p) {
  V v;
  __builtin_memcpy(&v, p, sizeof(V));
  return v;
}

template <class V>
__device__ __forceinline__ void store_dwords(float* p, V v) {
  __builtin_memcpy(p, &v, sizeof(V));
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmemRead = 0x020;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedDsWrite = 0x200;

template <int I, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < E) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, E>(f);
  }
}

template <int MASK, int PER, int N>
__device__ __forceinline__ void sched_pairs() {
  if constexpr (N > 0) {
    __builtin_amdgcn_sched_group_barrier(MASK, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, PER, 0);
    sched_pairs<MASK, PER, N - 1>();
  }
}

// Interleave the memory instructions of a half-step with its MFMAS MFMAs:
// each LDS read (NR), global load (NV) or LDS write (NW) is followed by a few
// MFMAs, so the wave never issues a burst of memory instructions while the
// matrix core idles.
template <int MFMAS, int NV, int NW, int NR>
__device__ __forceinline__ void sched_interleave() {
  constexpr int others = NV + NW + NR;
  constexpr int per = others ? MFMAS / (others + 1) : MFMAS;
  sched_pairs<kSchedDsRead, per, NR>();
  sched_pairs<kSchedVmemRead, per, NV>();
  sched_pairs<kSchedDsWrite, per, NW>();
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, MFMAS - per * others, 0);
}

// Number of load slots s in [0, slots) with s * steps / slots == h.
constexpr int slots_in_step(int h, int steps, int slots) {
  int n = 0;
  for (int s = 0; s < slots; ++s)
    if (s * steps / slots == h) ++n;
  return n;
}

template <class T, bool VEC>
__global__ __launch_bounds__(T::kThreads, T::kMinBlocks) void gemm_mfma_kernel(
    const float* __restrict__ A, const float* __restrict__ B, float* __restrict__ C, int M, int N,
    int K, int tiles_m, int tiles_n, int group) {
  constexpr int BM = T::BM, BN = T::BN, BK = T::BK, WN = T::WN;
  constexpr int H = BK / 8;  // half-steps per chunk
  __shared__ __attribute__((aligned(16))) float lds[T::kLdsFloats];
  float* const As0 = lds;
  float* const Bs0 = lds + T::kBufs * BM * T::kLdA;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int li = lane & 31;  // row (A operand) / column (B operand, D) inside a 32x32 block
  const int lg = lane >> 5;  // half-wave: which of the two reduction indices of a step

  int tm, tn;
  grouped_tile(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, group, tm, tn);
  const int m0 = tm * BM;
  const int k0 = tn * BN;

  // Per-thread load slots. A: slot f covers row f / kAQuads, float4 f % kAQuads
  // of the chunk; B: row f / kBQuads, float4 f % kBQuads.
  const float* a_ptr[T::kAPerThread];
  bool a_row_ok[T::kAPerThread];
  int a_lds[T::kAPerThread];
  int a_col[T::kAPerThread];
#pragma unroll
  for (int i = 0; i < T::kAPerThread; ++i) {
    const int f = tid + i * T::kThreads;
    const int r = f / T::kAQuads;
    const int q = f % T::kAQuads;
    a_row_ok[i] = (m0 + r) < M;
    a_col[i] = 4 * q;
    a_ptr[i] = A + (int64_t)(a_row_ok[i] ? m0 + r : 0) * N + 4 * q;
    a_lds[i] = r * T::kLdA + 4 * q;
  }
  const float* b_ptr[T::kBPerThread];
  int b_row[T::kBPerThread];
  int b_lds[T::kBPerThread];
  const int b_col = k0 + 4 * (tid % T::kBQuads);
#pragma unroll
  for (int i = 0; i < T::kBPerThread; ++i) {
    const int f = tid + i * T::kThreads;
    const int r = f / T::kBQuads;
    b_row[i] = r;
    b_ptr[i] = B + (int64_t)r * K + b_col;
    b_lds[i] = r * T::kLdB + 4 * (f % T::kBQuads);
  }

  // Registers staging the next chunk: slots 0 .. kAPerThread-1 are A's, the
  // rest B's. On the 128-bit path a slot is one float4 (a quad of a row). On
  // the 32-bit path a slot holds four single elements, placed so that
  // consecutive threads take consecutive columns: element (s, e) of a thread
  // is row r0 + (4 s + e) * row_step, column c of the chunk, c = tid % width.
  // Each 32-bit load instruction then reads whole row segments.
  constexpr int kSlots = T::kAPerThread + T::kBPerThread;
  constexpr int kARowStep = T::kThreads / BK;  // element rows between a thread's A elements
  constexpr int kBRowStep = T::kThreads / BN;
  static_assert(T::kThreads % BK == 0 && T::kThreads % BN == 0, "element slots keep one column");
  const int ea_r0 = tid / BK, ea_c = tid % BK;
  const int eb_r0 = tid / BN, eb_c = tid % BN;
  const float* const ea_base = A + (int64_t)(m0 + ea_r0 < M ? m0 + ea_r0 : 0) * N + ea_c;
  const float* const eb_base = B + (int64_t)eb_r0 * K + k0 + eb_c;
  unsigned ea_rows = 0;  // bit 4 s + e: that A element's row is inside M
#pragma unroll
  for (int i = 0; i < 4 * T::kAPerThread; ++i) ea_rows |= (m0 + ea_r0 + i * kARowStep < M) ? 1u << i : 0u;

  float4 stage[kSlots];
  unsigned stage_ok[kSlots];
  auto load_slot = [&](int s, int n0) {
    if constexpr (VEC) {
      if (s < T::kAPerThread)
        stage[s] = load_quad<VEC>(a_ptr[s] + n0, A, a_row_ok[s], n0 + a_col[s], N, stage_ok[s]);
      else {
        const int i = s - T::kAPerThread;
        stage[s] = load_quad<VEC>(b_ptr[i] + (int64_t)n0 * K, B, n0 + b_row[i] < N, b_col, K, stage_ok[s]);
      }
    } else {
      float x[4];
      unsigned ok = 0;
      if (s < T::kAPerThread) {
        const bool col_in = n0 + ea_c < N;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * s + e;
          const bool in = col_in && (ea_rows >> i & 1u);
          ok |= in ? 1u << e : 0u;
          x[e] = *(in ? ea_base + (int64_t)i * kARowStep * N + n0 : A);
        }
      } else {
        const int sb = s - T::kAPerThread;
        const bool col_in = k0 + eb_c < K;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * sb + e;
          const bool in = col_in && n0 + eb_r0 + i * kBRowStep < N;
          ok |= in ? 1u << e : 0u;
          x[e] = *(in ? eb_base + ((int64_t)n0 + i * kBRowStep) * K : B);
        }
      }
      stage[s] = make_float4(x[0], x[1], x[2], x[3]);
      stage_ok[s] = ok;
    }
  };
  auto store_slot = [&](int s, int buf) {
    const float4 v = mask_quad(stage[s], stage_ok[s]);
    if constexpr (VEC) {
      if (s < T::kAPerThread)
        *reinterpret_cast<float4*>(As0 + buf * BM * T::kLdA + a_lds[s]) = v;
      else
        *reinterpret_cast<float4*>(Bs0 + buf * BK * T::kLdB + b_lds[s - T::kAPerThread]) = v;
    } else {
      const float x[4] = {v.x, v.y, v.z, v.w};
      if (s < T::kAPerThread) {
        float* As = As0 + buf * BM * T::kLdA + ea_r0 * T::kLdA + ea_c;
#pragma unroll
        for (int e = 0; e < 4; ++e) As[(4 * s + e) * kARowStep * T::kLdA] = x[e];
      } else {
        const int sb = s - T::kAPerThread;
        float* Bs = Bs0 + buf * BK * T::kLdB + eb_r0 * T::kLdB + eb_c;
#pragma unroll
        for (int e = 0; e < 4; ++e) Bs[(4 * sb + e) * kBRowStep * T::kLdB] = x[e];
      }
    }
  };

  // MFMA operands of one half-step (8 reduction indices): per 32-row block a
  // float4 of A (indices 4*lg .. 4*lg+3), per 32-column block four B values.
  struct Frag {
    float4 a[T::kRB];
    float b[T::kCB][4];
  };
  const int a_frag = (wm * T::kWaveM + li) * T::kLdA + 4 * lg;
  const int b_frag = 4 * lg * T::kLdB + wn * T::kWaveN + li;
  auto read_frag = [&](Frag& f, int buf, int h) {
    const float* As = As0 + buf * BM * T::kLdA + a_frag + 8 * h;
    const float* Bs = Bs0 + buf * BK * T::kLdB + b_frag + 8 * h * T::kLdB;
#pragma unroll
    for (int i = 0; i < T::kRB; ++i) f.a[i] = *reinterpret_cast<const float4*>(As + i * 32 * T::kLdA);
#pragma unroll
    for (int j = 0; j < T::kCB; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) f.b[j][t] = Bs[t * T::kLdB + j * 32];
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

  constexpr int kMfmas = T::kRB * T::kCB * 4;  // per wave and half-step
  constexpr int kReads = T::kRB + 2 * T::kCB;  // b128 A reads, paired 32-bit B reads
  constexpr int kLoadInsts = VEC ? 1 : 4;      // global loads per slot
  constexpr int kStoreInsts = VEC ? 1 : 4;     // LDS writes per slot

  // Software pipeline. Chunk c is consumed from LDS buffer c % 2 in H = BK/8
  // half-steps; the operands of half-step h + 1 are read from LDS while the
  // MFMAs of half-step h run (two register sets, f[0] and f[1]). Chunk c + 1
  // is fetched into registers during the first H - 2 half-steps of chunk c and
  // written to the other LDS buffer during half-step H - 2 (with H = 2: all
  // loads at the top of half-step 0, all writes after it). One barrier before
  // the last half-step then both publishes chunk c + 1 and releases buffer
  // c % 2 (all its reads were issued and completed before it); the first
  // operands of chunk c + 1 are read while the last half-step of chunk c
  // computes. The LDS writes into buffer (c + 1) % 2 are safe because the
  // barrier of chunk c - 1 released it.
  constexpr int kLoadSteps = H >= 3 ? H - 2 : 0;
  const int nchunks = (N + BK - 1) / BK;
  Frag f[2];
  if constexpr (T::kBufs == 1) {
    // One LDS buffer: each chunk is loaded into registers, written to LDS
    // once every wave is done reading the previous chunk, and consumed after
    // a second barrier; loads, LDS writes and MFMAs of a workgroup take turns
    // (other workgroups on the CU are what overlaps them). Operand reads one
    // half-step ahead as above.
    for (int c = 0; c < nchunks; ++c) {
#pragma unroll
      for (int s = 0; s < kSlots; ++s) load_slot(s, c * BK);
      __syncthreads();
#pragma unroll
      for (int s = 0; s < kSlots; ++s) store_slot(s, 0);
      __syncthreads();
      read_frag(f[0], 0, 0);
      static_for<0, H - 1>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        read_frag(f[(h + 1) & 1], 0, h + 1);
        mma(f[h & 1]);
        sched_interleave<kMfmas, 0, 0, kReads>();
        __builtin_amdgcn_sched_barrier(0);
      });
      mma(f[(H - 1) & 1]);
    }
  } else {
#pragma unroll
  for (int s = 0; s < kSlots; ++s) load_slot(s, 0);
#pragma unroll
  for (int s = 0; s < kSlots; ++s) store_slot(s, 0);
  __syncthreads();
  read_frag(f[0], 0, 0);

  // Steady state: every chunk but the last. (The last is peeled off so that the
  // loop body has no data-dependent branch around its barrier.)
  for (int c = 0; c + 1 < nchunks; ++c) {
    const int buf = c & 1;
    const int n1 = (c + 1) * BK;
    if (kLoadSteps == 0) {
#pragma unroll
      for (int s = 0; s < kSlots; ++s) load_slot(s, n1);
    }
    static_for<0, H - 1>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      constexpr int n_slots = kLoadSteps > 0 ? slots_in_step(h, kLoadSteps, kSlots) : 0;
      constexpr bool writes = kLoadSteps > 0 && h == H - 2;
#pragma unroll
      for (int s = 0; s < kSlots; ++s)
        if (kLoadSteps > 0 && s * kLoadSteps / kSlots == h) load_slot(s, n1);
      if (writes) {
#pragma unroll
        for (int s = 0; s < kSlots; ++s) store_slot(s, buf ^ 1);
      }
      read_frag(f[(h + 1) & 1], buf, h + 1);
      mma(f[h & 1]);
      sched_interleave<kMfmas, n_slots * kLoadInsts, writes ? kSlots * kStoreInsts : 0, kReads>();
      __builtin_amdgcn_sched_barrier(0);
    });
    if (kLoadSteps == 0) {
#pragma unroll
      for (int s = 0; s < kSlots; ++s) store_slot(s, buf ^ 1);
    }
    __syncthreads();
    read_frag(f[H & 1], buf ^ 1, 0);
    mma(f[(H - 1) & 1]);
    sched_interleave<kMfmas, 0, 0, kReads>();
    __builtin_amdgcn_sched_barrier(0);
  }
  {
    const int buf = (nchunks - 1) & 1;
    static_for<0, H - 1>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      read_frag(f[(h + 1) & 1], buf, h + 1);
      mma(f[h & 1]);
      sched_interleave<kMfmas, 0, 0, kReads>();
      __builtin_amdgcn_sched_barrier(0);
    });
    mma(f[(H - 1) & 1]);
  }
  }

  // Epilogue: element r of lane l in block (i, j) is row 8*(r/4) + 4*lg + r%4,
  // column li of that block. Each half-wave stores 32 consecutive floats.
  // The 32-bit-copy forms, whose loops leave no register to carry the lane's
  // indices across, take them afresh: the wave from a scalar copy made at the
  // start, the lane from mbcnt.
  int ewm = wm, ewn = wn, eli = li, elg = lg;
  if constexpr (!VEC) {
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int el = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    ewm = w / WN;
    ewn = w % WN;
    eli = el & 31;
    elg = el >> 5;
  }
#pragma unroll
  for (int i = 0; i < T::kRB; ++i)
#pragma unroll
    for (int j = 0; j < T::kCB; ++j) {
      const int col = k0 + ewn * T::kWaveN + j * 32 + eli;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + ewm * T::kWaveM + i * 32 + 8 * (r / 4) + 4 * elg + (r % 4);
        if (row < M && col < K) C[(int64_t)row * K + col] = acc[i][j][r];
      }
    }
}

}  // namespace fgr
