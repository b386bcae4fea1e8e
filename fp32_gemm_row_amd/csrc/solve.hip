// C-ABI entry points of the row-major FP32 GEMM library (declared, with the
// full contract, in include/fp32_gemm_row.h): argument checks, path and tile
// selection, and the launches. Every step of the product runs in the kernels
// (gemm_mfma*.hpp, gemm_valu.hpp, gemv.hpp, reduce_parts.hpp); this file only
// decides, takes the split-reduction workspace, and enqueues.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <atomic>
#include <mutex>

#include "fp32_gemm_row.h"
#ifdef FGR_TIMESTAMPS
#include "fp32_gemm_row_timestamps.h"
#endif
#include "gemm_mfma.hpp"
#include "gemm_mfma_dma.hpp"
#include "gemm_mfma_ksplit.hpp"
#include "gemm_mfma_kreg.hpp"
#include "gemm_mfma_split.hpp"
#include "gemm_valu.hpp"
#include "gemv.hpp"
#include "reduce_parts.hpp"
#include "strip.hpp"
#include "stream_read.hpp"

namespace {

constexpr int kVersion = 200;  // 0.2.0
constexpr int kMaxDevices = 64;
constexpr int kDefaultCus = 256;  // MI355X
constexpr int kTileGroup = 4;     // tile-rows per group in the workgroup order

struct DeviceInfo {
  bool probed = false;
  bool ok = false;
  int cus = 0;
  bool pool_tried = false;
  hipMemPool_t pool = nullptr;  // the split-reduction workspace pool, made on first use
  bool scratch_tried = false;
  char* scratch = nullptr;  // device address of this device's copy of `scratch` (fgr_solve_noalloc)
};

std::mutex g_dev_mu;
DeviceInfo g_dev[kMaxDevices];

// Current device, checked once: it must be a gfx950 (the FP32 MFMA layouts and
// the LDS budget used here are gfx950's).
int current_device(int* cus, int* dev_out = nullptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FGR_ERR_DEVICE;
  if (dev_out) *dev_out = dev;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.probed) {
    hipDeviceProp_t p;
    d.probed = true;
    if (hipGetDeviceProperties(&p, dev) == hipSuccess && std::strncmp(p.gcnArchName, "gfx950", 6) == 0) {
      d.ok = true;
      d.cus = p.multiProcessorCount;
    }
  }
  if (!d.ok) return FGR_ERR_DEVICE;
  *cus = d.cus;
  return FGR_OK;
}

// The current device's CU count, after checking that it is a gfx950 and
// that `stream` (other than the null and per-thread streams, which follow
// the current device) belongs to it: the kernels run on the stream's device,
// while the CU count and the split workspace come from the current one.
int device_for(hipStream_t stream, int* cus, int* dev_out = nullptr) {
  int dev = -1;
  const int rc = current_device(cus, &dev);
  if (dev_out) *dev_out = dev;
  if (rc != FGR_OK) return rc;
  if (stream && stream != hipStreamPerThread) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) {
      (void)hipGetLastError();
      return FGR_ERR_DEVICE;
    }
    if (sdev != dev) return FGR_ERR_DEVICE;
  }
  return FGR_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void* p, int64_t pn, const void* q, int64_t qn) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), a1 = a0 + (uintptr_t)pn * 4;
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(q), b1 = b0 + (uintptr_t)qn * 4;
  return a0 < b1 && b0 < a1;
}

int check_args(const float* A, const float* B, const float* C, int M, int N, int K) {
  if (!A || !B || !C) return FGR_ERR_NULL_POINTER;
  if (M < 1 || N < 1 || K < 1) return FGR_ERR_BAD_DIMS;
  if (!aligned(A, 4) || !aligned(B, 4) || !aligned(C, 4)) return FGR_ERR_MISALIGNED;
  const int64_t mn = (int64_t)M * N, nk = (int64_t)N * K, mk = (int64_t)M * K;
  if (overlaps(C, mk, A, mn) || overlaps(C, mk, B, nk)) return FGR_ERR_ALIAS;
  return FGR_OK;
}

bool mfma_vec_ok(const float* A, const float* B, const float* C, int N, int K) {
  return N % 4 == 0 && K % 4 == 0 && aligned(A, 16) && aligned(B, 16) && aligned(C, 16);
}

bool gemv_vec_ok(const float* B, int K) { return K % 4 == 0 && aligned(B, 16); }

// Row alignment of a product, for the k-split configurations: 16-byte copies
// of A (N % 4 == 0, aligned A) and of B (K % 4 == 0, aligned B) with 128-bit
// stores (aligned C), of A only, of B only, or of neither. (A product with
// aligned A and B but not C takes the A-only form.)
enum class Rows { kAll, kAOnly, kBOnly, kNone };
Rows rows_of(const float* A, const float* B, const float* C, int N, int K) {
  const bool va = N % 4 == 0 && aligned(A, 16);
  const bool vb = K % 4 == 0 && aligned(B, 16);
  const bool vc = K % 4 == 0 && aligned(C, 16);
  if (va && vb && vc) return Rows::kAll;
  if (va) return Rows::kAOnly;
  if (vb) return Rows::kBOnly;
  return Rows::kNone;
}

// 128x128 k-split tiles load their operands straight into registers, four
// columns of B per lane (gemm_mfma_kreg.hpp): they need K >= 4 and no
// alignment beyond 4 bytes.
bool ksplit128_ok(int K) { return K >= 4; }

// The direct-copy kernel's global->LDS copies need at least four 16-deep
// reduction chunks, N >= 64 (the copies that run past the last chunk re-read
// it, and must never reach the zero-padded first chunk), and their byte
// offsets inside 32 bits (256 rows of A, 16 rows of B). They are 16 bytes wide
// for 16-byte aligned rows, 4 bytes otherwise.
bool mfma_dma_ok(int N, int K) { return N >= 64 && N <= fgr::kDmaMaxN && K <= fgr::kDmaMaxK; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Largest last partial wave of 256x256 tiles that is cheaper to spread over
// every CU as small split-reduction tiles than to run as a wave of its own
// (measured on MI355X, 4096 x 4096 x K: the split tail wins up to 160 tiles
// left over, 130.6 vs 121.7 TFLOP/s, and loses at 192, 129.0 vs 131.5).
int64_t tail_tiles(int cus) { return (int64_t)cus * 11 / 16; }

// The same for 128x128 tiles of the k-split kernel (measured: 2560^3, 144 of
// 256 left over, 105.4 TFLOP/s with the split tail, 108.4 without; 3072^3, 64
// left over, 131.1 vs 104.7).
int64_t ksplit_tail_tiles(int cus) { return cus / 2; }

// Matrix-vector plan: column block width (32, or 16 when 32-column blocks
// fill at most half the CUs) and parts of the reduction across workgroups,
// by an estimate of the call's time. GPU side: streaming B (and A and C) at
// 40 GB/s per workgroup of 32 columns and 26 GB/s per workgroup of 16, at
// most 5.5 TB/s for the device, plus 4 us, and for a split 3 us and the P M K
// 8 bytes of partial rows; host side 6 us, 10 us with a split (as for the
// k-split plan below); the call takes the longer of the two. Candidates: 16
// columns unsplit; 32 columns with P = 1, 2, 4, ... while the workgroups fit
// one per CU and parts keep at least 1024 rows of B. Measured on MI355X (us,
// previous rule of at least 8192 rows per part -> this plan): 1 x 16384 x
// 1024 31.3 -> 17.6, 1 x 32768 x 512 30.9 -> 17.8, 4 x 8192 x 1024 27.3 ->
// 16.0, 2 x 65536 x 256 35.4 -> 19.3, 1 x 8192 x 2048 21.4 -> 17.9;
// unchanged where no split pays (1 x 2048 x 2048 7.4, 1 x 4096 x 4096 15.0,
// 1 x 8192 x 8192 45.8, 1 x 65536 x 1024 52.3).
struct GemvPlan {
  int cols;
  int parts;
};

double gemv_time(int cols, int p, int M, int N, int K) {
  const double wgs = (double)cdiv(K, cols) * p;
  const double bytes = 4.0 * ((double)N * K + (double)M * N + (double)M * K);
  const double rate = std::min(5.5e12, wgs * (cols == fgr::kGemvCols ? 40e9 : 26e9));
  double gpu = bytes / rate + 4e-6;
  if (p > 1) gpu += 3e-6 + (double)p * M * K * 8.0 / 5e12;
  const double host = p > 1 ? 10e-6 : 6e-6;
  return std::max(host, gpu) + 1e-3 * gpu;  // the small second term breaks ties
}

constexpr int kGemvMinPart = 1024;
GemvPlan gemv_plan(int M, int N, int K, int cus) {
  const int64_t wide = cdiv(K, fgr::kGemvCols);
  GemvPlan best{fgr::kGemvCols, 1};
  double best_time = gemv_time(fgr::kGemvCols, 1, M, N, K);
  if (wide * 2 <= cus) {
    const double e = gemv_time(fgr::kGemvCols / 2, 1, M, N, K);
    if (e < best_time) {
      best = {fgr::kGemvCols / 2, 1};
      best_time = e;
    }
  }
  for (int p = 2; wide * p <= cus && N / p >= kGemvMinPart && p <= 65535; p *= 2) {
    const double e = gemv_time(fgr::kGemvCols, p, M, N, K);
    if (e < best_time) {
      best = {fgr::kGemvCols, p};
      best_time = e;
    }
  }
  return best;
}

struct SplitPlan {
  int tile;
  int parts;
};

// Estimated time (seconds) of one call with k-split tiles of size t whose
// reduction is split into p parts, on `cus` CUs at 2.4 GHz. GPU side: the
// larger of the MFMA time of the busiest CU (its workgroups, each a t x t tile
// over N / p reduction indices, t^2 N / (128 p) cycles of its four SIMDs, at
// an efficiency of 0.9 for 64x64 and 0.7 for 32x32 tiles, 10% more when two
// or more of them share the CU) and the HBM time (A and B panels of every
// tile, 25% of them from HBM and the rest from L2, at 5 TB/s), plus 3 us and
// 1 us per workgroup of the busiest CU and, for a split, 3 us and the P M K 8
// bytes of partial tiles written and read back. Host side (measured from
// Python): 6 us per call, 10 us with a split (second launch, workspace lookup
// and event); the two overlap, so the call takes the longer. Ties go to the
// smaller GPU time. The constants are fitted to MI355X measurements of 24
// shapes with few output tiles (M, K from 96 to 1024, N from 1024 to 262144;
// 64x64 and 32x32 tiles, P = 1 .. 256): the chosen plan is within 5% of the
// best measured one on each of them and within 7% on 18 others, where the
// first estimate, which added the host cost to the GPU time, lost up to 35%
// (1024 x 32768 x 512: 387 us against 286).
double splitk_time(int t, int p, int M, int N, int K, int cus) {
  const double tiles = (double)cdiv(M, t) * (double)cdiv(K, t);
  const double per_cu = std::ceil(tiles * p / cus);  // workgroups on the busiest CU
  const int resident = t >= 128 ? 1 : t >= 64 ? 2 : 4;  // workgroups per CU (LDS)
  const double eff = (t >= 64 ? 0.9 : 0.7) * (std::min<double>(per_cu, resident) >= 2 ? 1.1 : 1.0);
  const double t_mfma = per_cu * ((double)t * t * ((double)N / p) / 128.0) / (2.4e9 * eff);
  const double t_hbm = 4.0 * N * tiles * 2.0 * t * 0.25 / 5e12;
  double gpu = std::max(t_mfma, t_hbm) + 3e-6 + per_cu * 1e-6;
  if (p > 1) gpu += 3e-6 + (double)p * M * K * 8.0 / 5e12;
  const double host = p > 1 ? 10e-6 : 6e-6;
  return std::max(host, gpu) + 1e-3 * gpu;  // the small second term breaks ties
}

// Parts to try: powers of two and, with `rounds`, the counts that fill whole
// rounds of the CUs (k CUs / tiles, k = 1 .. 4: with few tiles a power of two
// either leaves CUs idle or starts a second round, e.g. nine 128x128 tiles:
// 16 parts on 144 CUs or 32 in two rounds, against 28); each part at least
// 256 reduction indices long (32 chunks, 8 per wave), at most four
// workgroups per CU.
constexpr int kSplitkMinPart = 256;
template <class F>
void for_each_parts(int t, int M, int N, int K, int cus, bool rounds, F&& f) {
  const int64_t tiles = cdiv(M, t) * cdiv(K, t);
  auto ok = [&](int64_t p) { return p >= 2 && N / p >= kSplitkMinPart && tiles * p <= 4 * (int64_t)cus; };
  for (int p = 2; ok(p); p *= 2) f(p);
  for (int k = 1; rounds && k <= 4; ++k) {
    const int64_t p = k * (int64_t)cus / tiles;
    if (ok(p) && (p & (p - 1)) != 0) f((int)p);  // powers of two came above
  }
}

// Split plans with 128x128 tiles: taken over the estimate's 64x64 or 32x32
// choice when they pad the output no more than 64x64 tiles do and their parts
// are at least this long. Each operand element is then read by fewer tiles,
// and the long parts amortise the 128x128 tile's start and its 64 KiB
// partial write; the estimate does not model either. MI355X, us per call,
// 64x64 plan vs 128x128 plan (128x128 parts): 128 x 2097152 x 128 980 vs 788
// (8192), 512 x 131072 x 512 572 vs 513 (8192), 128 x 1048576 x 128 503 vs
// 418 (4096), 256 x 262144 x 256 364 vs 307 (4096), 512 x 65536 x 512 273 vs
// 258 (4096), 128 x 524288 x 128 253 vs 222 (2048), 128 x 262144 x 256 170
// vs 148 (2048), 256 x 131072 x 256 146 vs 140 (2048). With parts of 1024 or
// less it lost (128 x 262144 x 128 83 vs 86, 384 x 32768 x 384 114 vs 126),
// and so it did where it pads more (192 x 262144 x 192 230 vs 260, 320 x
// 200000 x 320 412 vs 572).
constexpr int kSplitk128MinPart = 2048;

// Best parts (>= 2) for k-split tiles of size t, by the estimate above, over
// power-of-two parts or (rounds) also the whole-round counts. With rounds,
// 128x128 tiles whose power-of-two plan has parts of at least
// kSplitk128MinPart (the plans choose() takes them for) keep parts that long:
// shorter ones lost there (896 x 16384 x 1024 247 vs 264 us). A forced
// 128x128 split elsewhere takes the estimate's count (one 128x128 tile of
// 128 x 262144 x 128: 128 parts of 2048 on half the CUs ran 60.6 TFLOP/s,
// 256 of 1024 ran 82.9).
SplitPlan splitk_plan_tile(int t, int M, int N, int K, int cus, bool rounds) {
  SplitPlan best{t, 2};
  double best_time = 0;
  const int min_part = rounds && t == FGR_TILE_128 &&
                               N / splitk_plan_tile(t, M, N, K, cus, false).parts >= kSplitk128MinPart
                           ? kSplitk128MinPart
                           : kSplitkMinPart;
  for_each_parts(t, M, N, K, cus, rounds, [&](int p) {
    if (N / p < min_part) return;
    const double e = splitk_time(t, p, M, N, K, cus);
    if (best_time == 0 || e < best_time) {
      best = {t, p};
      best_time = e;
    }
  });
  return best;
}

// For a shape with fewer 64x64 tiles than CUs: the k-split tile size (64 or
// 32) and parts (1: no split) with the smallest estimated time, over
// power-of-two parts. The launch then takes the tile's best parts among the
// whole-round counts too (splitk_plan_tile with rounds). Choosing the tile
// over those counts as well was measured on 62 few-tile shapes (MI355X, us
// per call against power-of-two plans): keeping the tile, worst +1.4% and
// mean -4.1% (384 x 131072 x 384 385 vs 290, 640 x 65536 x 640 483 vs 392,
// 384 x 32768 x 384 108 vs 87); re-choosing it gained more on short
// reductions (mean -10.7%) but lost up to 34% where the estimate misjudges
// 32x32 tiles (96 x 262144 x 384 226 vs 302), and offering those counts
// against no split turned short reductions into splits that lost up to 34%
// (320 x 1024 x 1000 13.2 vs 17.7).
SplitPlan splitk_plan(int M, int N, int K, int cus) {
  SplitPlan best{FGR_TILE_32, 1};
  double best_time = splitk_time(FGR_TILE_32, 1, M, N, K, cus);
  for (int t : {FGR_TILE_64, FGR_TILE_32}) {
    auto consider = [&](int p) {
      const double e = splitk_time(t, p, M, N, K, cus);
      if (e < best_time) {
        best = {t, p};
        best_time = e;
      }
    };
    consider(1);
    for_each_parts(t, M, N, K, cus, false, consider);
  }
  return best;
}

// Skinny outputs (kSkinnyMinM <= M <= 64, K >= 128, B as in skinny_b below):
// 32x128 k-split tiles, each reduction split into the largest number of
// parts that keeps tiles x parts within the CU count and parts at least 512
// long. The work is streaming B once; wide column blocks and one workgroup
// per CU measured best (MI355X, TB/s of algorithmic bytes, 32x128 tiles vs
// the previous choice: 16 x 8192 x 28672 5.61 vs 3.43, 32 x 11008 x 4096 4.21
// vs 2.56, 32 x 8192 x 8192 4.90 vs 3.25, 16 x 4096 x 4096 2.70 vs 1.99; and
// at M = 5..8 against the matrix-vector kernel: 8 x 8192 x 28672 5.68 vs 3.61,
// 8 x 65536 x 256 2.50 vs 1.10). With K < 128 half of a 128-column tile would
// be padding (16 x 1048576 x 64: 3.57 vs 4.01 with 32x32 tiles). Up to M = 64
// two rows of these tiles still beat the square ones (48 x 8192 x 8192 3.01
// vs 2.18, 64 x 8192 x 28672 3.15 vs 2.87, 64 x 11008 x 4096 2.87 vs 1.72).
constexpr int kSkinnyMinM = 5;  // fewer rows: the matrix-vector kernel
constexpr int kSkinnyMaxM = 64;  // two rows of 32x128 tiles at most
// B large enough for the 32x128 tiles: at least 32 Mi elements, or 16 Mi when
// 32x32 tiles alone would leave CUs idle. Below that the split plan's 32x32
// tiles measured faster (MI355X, us, 32x128 vs the plan: 16 x 4096 x 2048
// 18.5 vs 14.8, 32 x 2048 x 4096 19.4 vs 14.9, 16 x 2048 x 8192 20.2 vs 15.7
// with 256 tiles of 32x32; but 16 x 8192 x 8192 55.3 vs 63.9, 32 x 4096 x
// 4096 21.7 vs 22.8).
constexpr int64_t kSkinnyMinB = int64_t(16) << 20;
constexpr int64_t kSkinnyWideB = int64_t(32) << 20;
bool skinny_b(int M, int N, int K, int cus) {
  const int64_t b = (int64_t)N * K;
  return b >= kSkinnyWideB || (b >= kSkinnyMinB && cdiv(M, 32) * cdiv(K, 32) < cus);
}
int skinny_parts(int M, int N, int K, int cus) {
  const int64_t tiles = cdiv(M, 32) * cdiv(K, 128);
  return (int)std::max<int64_t>(1, std::min<int64_t>(cus / tiles, N / 512));
}

struct Choice {
  int path;
  int tile;
};

// The strip plan (launch_strip) applies when K = 64 q + w, 1 <= w <=
// kStripMax, N >= 64, and the q whole column blocks of 64x64 tiles fit one
// tile per CU while the w columns would add a partial second wave.
bool strip_shape(int M, int N, int K) { return N >= 64 && K > 64 && K % 64 >= 1 && K % 64 <= fgr::kStripMax; }
bool strip_plan_ok(int M, int N, int K, int cus) {
  return strip_shape(M, N, K) && cdiv(M, 64) * (K / 64) <= cus && cdiv(M, 64) * cdiv(K, 64) > cus;
}

// Reductions shorter than this (with at least one 64x64 tile per CU) take
// register-staged 64x64 tiles (128x128 for unaligned rows with many tiles).
constexpr int kShortReduction = 104;
// With every row aligned and whole waves of 256x256 tiles the direct-copy
// kernel wins from this length on (measured on MI355X, us per call,
// register-staged 64x64 vs direct copies: 8192 x N x 8192, N = 64 110.0 vs
// 109.9, 72 122.8 vs 117.5, 80 124.9 vs 118.1, 96 145.3 vs 133.2; 4096 x 80 x
// 4096 32.5 vs 31.6); with a partial last wave the short tiles keep the
// lead (6144 x 80 x 6144 72.3 vs 76.3 with the split tail, 65792 x 96 x 256
// 40.0 vs 41.3).
constexpr int kShortReductionWholeWaves = 72;
// With whole-device shapes whose B rows are not 16-byte aligned (the
// direct-copy kernel would copy B 4 bytes at a time) the register-staged
// tiles win up to this reduction length.
constexpr int kShortReductionNarrowB = 384;
// With neither operand's rows aligned, whole-device shapes from this
// reduction length on take 128x128 k-split tiles instead of direct copies
// (8191 x N x 8191, us: N = 511 613 vs 596, 767 842 vs 849, 1023 1069 vs 1092).
constexpr int kKsplitUnalignedMinN = 768;

// Kernel choice by the number of output tiles the shape makes at each tile
// size, relative to the CU count (measured on MI355X; see the design notes):
// whole-device 256x256 tiles take the direct-copy kernel; shapes with few
// tiles split each tile's reduction across a workgroup's waves.
Choice choose(const float* A, const float* B, const float* C, int M, int N, int K, int cus) {
  if (cus <= 0) cus = kDefaultCus;
  const bool skinny_shape =
      M >= kSkinnyMinM && M <= kSkinnyMaxM && N >= 64 && K >= 128 && fgr::ksplit_offsets_fit(32, N, K);
  const bool skinny = skinny_shape && skinny_b(M, N, K, cus);
  // M <= 8: the matrix-vector kernel, except that from 5 rows on the split
  // plan below wins where the skinny tiles do not apply (measured on MI355X,
  // us: 5 x 4096 x 1024 16.5 vs 12.4, 8 x 4096 x 256 15.6 vs 10.8, 8 x 2048
  // x 2048 14.8 vs 12.1; at M <= 4 the two are within 15% either way)
  if (M <= fgr::kGemvMaxRows && !skinny && !skinny_shape)
    return {gemv_vec_ok(B, K) ? FGR_PATH_GEMV_VEC : FGR_PATH_GEMV_SCALAR, FGR_TILE_AUTO};
  if (skinny) {
    // skinny: stream B once in 32x128 tiles (see skinny_parts)
    return {skinny_parts(M, N, K, cus) >= 2 ? FGR_PATH_MFMA_SPLITK : FGR_PATH_MFMA_KSPLIT, FGR_TILE_32X128};
  }
  const int64_t t256 = cdiv(M, 256) * cdiv(K, 256);
  const int64_t t128 = cdiv(M, 128) * cdiv(K, 128);
  const int64_t t64 = cdiv(M, 64) * cdiv(K, 64);
  const bool vec = mfma_vec_ok(A, B, C, N, K);
  const Rows rows = rows_of(A, B, C, N, K);
  const bool narrow_b = rows == Rows::kAOnly || rows == Rows::kNone;
  const bool whole_waves = rows == Rows::kAll && t256 >= cus && t256 % cus == 0 && mfma_dma_ok(N, K);
  const int short_n = whole_waves ? kShortReductionWholeWaves : kShortReduction;
  if (t64 >= cus && (N < short_n || (narrow_b && t256 >= cus && N < kShortReductionNarrowB))) {
    // A short reduction over many tiles: the time goes to writing C. Small
    // register-staged tiles keep several workgroups per CU, so that one's
    // stores overlap another's loads and MFMAs (measured, 8192 x N x 8192:
    // 64x64 tiles 46 us at N = 16 vs 77 us with 256x256; 100 vs 112 us with
    // the direct-copy kernel at N = 64; equal at N = 96; 4% slower at N =
    // 112). Unaligned rows take 32-bit loads; against direct copies that move
    // B 4 bytes at a time they win up to N = 384 (us: 8191 x 65 x 8191 121 vs
    // 177, 8191 x 255 x 8191 317 vs 346, 8191 x 383 x 8191 463 vs 475, 8191 x
    // 128 x 8191 170 vs 216; but 8191 x 511 x 8191 611 vs 596; with B's rows
    // aligned 8192 x 129 x 8192 188 vs 180).
    if (vec) return {FGR_PATH_MFMA_VEC, FGR_TILE_64};
    return {FGR_PATH_MFMA_SCALAR, t128 >= 4 * cus ? FGR_TILE_128 : FGR_TILE_64};
  }
  // Whole-device shapes take the direct-copy kernel, unless neither operand's
  // rows are 16-byte aligned, the reduction is long and the 256x256 tiles
  // leave a partial last wave: the k-split kernel's 128x128 tiles, which load
  // at any alignment, then even that wave out better than the direct-copy
  // kernel's 4-byte copies and split tail (measured on MI355X, us per call,
  // direct copies vs 128x128: partial waves 4095 x 4097 x 4099 1043 vs 1003,
  // 6143 x 4095 x 6143 2287 vs 2126, 5119 x 3001 x 5119 1401 vs 1141; whole
  // waves 8191 x 1023 x 8191 1000 vs 1052, 8191 x 2047 x 8191 1901 vs 1963,
  // 8191 x 4095 x 8191 3692 vs 3773, 8191 x 6143 x 4095 2765 vs 2803; below
  // N = 768 8191 x 511 x 8191 557 vs 605; with one operand aligned the direct
  // copies are faster or within 1%: 4096 x 4096 x 4095 927 vs 952).
  if (t256 >= cus && mfma_dma_ok(N, K) &&
      (rows != Rows::kNone || N < kKsplitUnalignedMinN || !ksplit128_ok(K) || t256 % cus == 0)) {
    // a last, partial wave of at most tail_tiles(cus) tiles goes to the split kernel
    const int64_t rem = t256 % cus;
    if (rem != 0 && rem <= tail_tiles(cus)) return {FGR_PATH_MFMA_DMA_TAIL, FGR_TILE_256};
    return {FGR_PATH_MFMA_DMA, FGR_TILE_256};
  }
  if (N >= 64) {
    // Fewer 256x256 tiles than CUs (or, above, unaligned rows): tiles whose
    // reduction is split over the four waves of a workgroup (k-split), the
    // largest that still gives every CU a tile; a last partial wave of up to
    // half the CUs is spread over every CU (launch_ksplit_tail). 128x128
    // tiles where they make whole waves, three waves or more, or a last wave
    // more than three quarters full; else 64x64, whose two workgroups per CU
    // even out a partial wave better (measured on MI355X, us per call, 128x128
    // vs 64x64 tiles: 2047^3 128 vs 135, 1024 x 6144 x 4095 358 vs 395, 2048 x
    // 8192 x 2048 464 vs 470, aligned 2048 x 4096 x 4096 474 vs 478, 3584^3
    // 669 vs 694; but 2304^3 237 vs 184, 2560^3 302 vs 248, 2303 x 2305 x 2307
    // 269 vs 206, aligned 3072^3 (2.25 waves) 424 vs 409; 2816^3 334 vs 329).
    const int64_t rem128 = t128 % cus;
    if (ksplit128_ok(K) && t128 >= cus && (rem128 == 0 || t128 >= 3 * cus || 4 * rem128 > 3 * cus)) {
      if (rem128 != 0 && rem128 <= ksplit_tail_tiles(cus)) return {FGR_PATH_MFMA_KSPLIT_TAIL, FGR_TILE_128};
      return {FGR_PATH_MFMA_KSPLIT, FGR_TILE_128};
    }
    if (t64 >= cus) {
      // a few columns past whole 64-column blocks that give every CU at most
      // one tile: those columns on the vector ALUs, not a wave of tiles
      if (strip_plan_ok(M, N, K, cus)) return {FGR_PATH_MFMA_STRIP, FGR_TILE_64};
      const int64_t rem = t64 % cus;
      if (rem != 0 && rem <= ksplit_tail_tiles(cus)) return {FGR_PATH_MFMA_KSPLIT_TAIL, FGR_TILE_64};
      return {FGR_PATH_MFMA_KSPLIT, FGR_TILE_64};
    }
    // fewer 64x64 tiles than CUs: 64x64 or 32x32 k-split tiles, with the
    // reduction also split across workgroups where that is estimated faster
    // (the k-split 32x32 tiles measured faster than the split kernel's on
    // unaligned rows even when they still took 4-byte copies through LDS:
    // 400 x 1000 x 401 10.0 vs 14.8 us, 512 x 4095 x 512 30.8 vs 50.9)
    const SplitPlan sp = splitk_plan(M, N, K, cus);
    if (sp.parts >= 2) {
      if (ksplit128_ok(K) && 4 * cdiv(M, 128) * cdiv(K, 128) == t64 &&
          N / splitk_plan_tile(FGR_TILE_128, M, N, K, cus, false).parts >= kSplitk128MinPart)
        return {FGR_PATH_MFMA_SPLITK, FGR_TILE_128};
      return {FGR_PATH_MFMA_SPLITK, sp.tile};
    }
    return {FGR_PATH_MFMA_KSPLIT, sp.tile};
  }
  // N < 64 with fewer 64x64 tiles than CUs: the split kernel's 32x32 tiles
  return {FGR_PATH_MFMA_SPLIT, FGR_TILE_32};
}

// Tile for a forced path when the caller left it open.
int default_tile(int path, const Choice& auto_choice, int M, int N, int K, int cus, bool vec_rows) {
  if (path == auto_choice.path) return auto_choice.tile;
  switch (path) {
    case FGR_PATH_MFMA_DMA:
    case FGR_PATH_MFMA_DMA_TAIL: return FGR_TILE_256;
    case FGR_PATH_MFMA_KSPLIT:
    case FGR_PATH_MFMA_KSPLIT_TAIL:
      if (vec_rows && cdiv(M, 128) * cdiv(K, 128) >= cus) return FGR_TILE_128;
      if (path == FGR_PATH_MFMA_KSPLIT_TAIL || cdiv(M, 64) * cdiv(K, 64) >= cus) return FGR_TILE_64;
      return FGR_TILE_32;
    case FGR_PATH_MFMA_SPLITK:
      if (cdiv(M, 64) * cdiv(K, 64) < cus) return splitk_plan(M, N, K, cus).tile;
      return vec_rows && cdiv(M, 128) * cdiv(K, 128) < cus ? FGR_TILE_128 : FGR_TILE_64;
    case FGR_PATH_MFMA_SPLIT: return cdiv(M, 64) * cdiv(K, 64) < cus ? FGR_TILE_32 : FGR_TILE_64;
    case FGR_PATH_VALU: return FGR_TILE_128;
    case FGR_PATH_MFMA_STRIP: return FGR_TILE_64;
    case FGR_PATH_MFMA_VEC:
    case FGR_PATH_MFMA_SCALAR:
      if (cdiv(M, 256) * cdiv(K, 256) >= cus) return FGR_TILE_256;
      if (cdiv(M, 128) * cdiv(K, 128) >= cus) return FGR_TILE_128;
      return FGR_TILE_64;
    default: return FGR_TILE_AUTO;
  }
}

// Scratch of fgr_solve_noalloc, for callers that cannot allocate: every
// workspace of such a call is carved from this array instead (256-byte aligned
// pieces). Each device holds its own copy, at its own address, until the
// process ends. In host code the name is a host-side stand-in, never a device
// address: the device address comes from hipGetSymbolAddress, once per device
// with that device current (scratch_of), and only that address is passed to
// kernels. Nothing in it needs to start at zero: every piece is written in full
// by one kernel of the call before another reads it.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of the current device's `scratch` (dev is current).
int scratch_of(int dev, char** out) {
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.scratch_tried) {
    d.scratch_tried = true;
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess && p) d.scratch = static_cast<char*>(p);
    else (void)hipGetLastError();
  }
  if (!d.scratch) return FGR_ERR_DEVICE;
  *out = d.scratch;
  return FGR_OK;
}

// One fgr_solve_noalloc call, on the calling thread (t_scratch points at it
// for the call's duration). Its launch sequence runs twice: a dry pass that
// launches nothing and makes no HIP call, only adding up the workspace the
// plan takes, then, if that fits the array, the real pass over the same plan.
struct ScratchCall {
  bool dry = true;
  char* base = nullptr;  // the device's array (real pass)
  size_t used = 0;       // bytes handed out so far
};
thread_local ScratchCall* t_scratch = nullptr;
// Stand-in base of the dry pass's pieces: never dereferenced (nothing is
// launched), 256-byte aligned like the array so that alignment tests agree.
constexpr uintptr_t kDryBase = uintptr_t(1) << 32;

int launch(const void* kernel, int64_t blocks, int threads, void** args, hipStream_t stream, int rows = 1) {
  if (blocks < 1 || blocks > INT_MAX || rows < 1 || rows > 65535) return FGR_ERR_BAD_DIMS;
  if (t_scratch && t_scratch->dry) return FGR_OK;  // counting a scratch call's workspace
  const hipError_t e =
      hipLaunchKernel(kernel, dim3((unsigned)blocks, (unsigned)rows), dim3(threads), args, 0, stream);
  return e == hipSuccess ? FGR_OK : FGR_ERR_LAUNCH;
}

// Workspace: device memory a call needs beyond A, B and C: the partial tiles
// (or rows) of a reduction split across workgroups (parts x M x K floats, or
// parts x tiles x tile^2 in compact slots). A workspace is either the caller's
// stream's cached one (below), borrowed with the cache lock held until the
// call's last kernel is enqueued, or a stream-ordered allocation from a
// per-device pool on the caller's stream, given back with hipFreeAsync on it
// behind the call's last kernel. Either way calls on different streams never
// share one. A call that cannot get its workspace runs its plan's form
// without one (same result up to rounding order).
struct CachedWorkspace;

struct Workspace {
  float* w = nullptr;
  hipStream_t s = nullptr;
  bool owned = false;                 // allocated for this call
  CachedWorkspace* cached = nullptr;  // or borrowed from the stream's cache entry
  std::unique_lock<std::mutex> cache_lock;
  ~Workspace();
};

// Largest workspace one request may take, in bytes (fgr_set_workspace_limit;
// negative: no limit). A larger request fails as a failed allocation does.
std::atomic<long long> g_ws_limit{-1};

// Freed workspace a device's pool keeps for reuse instead of returning it at
// each synchronisation (measured on MI355X, 128 x 262144 x 128 with a
// synchronisation after every call: 158 us per call from the device's default
// pool, 118 from this one; 16 MiB workspace).
constexpr uint64_t kPoolKeepBytes = 64ull << 20;

// The current device's workspace pool (created on first use; null if that
// failed, and then the device's default pool serves).
hipMemPool_t workspace_pool() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.pool_tried) {
    d.pool_tried = true;
    hipMemPoolProps props;
    std::memset(&props, 0, sizeof(props));
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    if (hipMemPoolCreate(&pool, &props) == hipSuccess) {
      uint64_t keep = kPoolKeepBytes;
      (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
      d.pool = pool;
    } else {
      (void)hipGetLastError();  // clear the failed call's error
    }
  }
  return d.pool;
}

hipError_t pool_alloc(float** w, size_t bytes, hipStream_t s) {
  hipMemPool_t pool = workspace_pool();
  return pool ? hipMallocFromPoolAsync(reinterpret_cast<void**>(w), bytes, pool, s)
              : hipMallocAsync(reinterpret_cast<void**>(w), bytes, s);
}

// Workspace kept between calls, one per stream handle (up to kCachedStreams
// per process, each up to kCachedMaxBytes): a stream-ordered allocation and
// free cost about 9 us of host time per call (measured on MI355X; a split
// call took 30 us of host time against 9 us unsplit). Each entry has an
// event recorded behind the last kernel that used its buffer, and every call
// that borrows the buffer first makes its stream wait for that event: on the
// same stream the wait is already satisfied by stream order, and a new stream
// that happens to reuse a destroyed one's handle still waits for the old
// stream's work. The lock, held from the lookup until the call's last kernel
// and the event are enqueued, keeps two threads' calls on one stream from
// interleaving their kernels. A buffer too small for a call is freed with
// hipFreeAsync on the stream, behind that wait, and replaced. Buffers are
// never returned otherwise (the process holds at most kCachedStreams x
// kCachedMaxBytes); a full table, hipStreamPerThread (one handle for many
// streams), stream capture (the workspace then becomes a graph allocation)
// and larger workspaces take the per-call allocation.
constexpr int kCachedStreams = 16;
constexpr size_t kCachedMaxBytes = size_t(64) << 20;
constexpr size_t kCachedGrain = size_t(1) << 20;

struct CachedWorkspace {
  hipStream_t stream = nullptr;
  int dev = -1;
  hipEvent_t done = nullptr;  // recorded behind the buffer's last use
  bool recorded = false;
  float* w = nullptr;
  size_t bytes = 0;
};

std::mutex g_ws_mu;
CachedWorkspace g_ws[kCachedStreams];
int g_ws_used = 0;

Workspace::~Workspace() {
  if (cached) {
    cached->recorded = hipEventRecord(cached->done, s) == hipSuccess;
    if (!cached->recorded) (void)hipGetLastError();
  } else if (w && owned) {
    (void)hipFreeAsync(w, s);
  }
}  // cache_lock, if held, is released after the event is enqueued

bool cached_workspace(Workspace& ws, size_t bytes, hipStream_t s) {
  if (bytes > kCachedMaxBytes || s == hipStreamPerThread) return false;
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  int dev = -1;
  if (hipStreamIsCapturing(s, &capture) != hipSuccess || capture != hipStreamCaptureStatusNone ||
      hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  std::unique_lock<std::mutex> lock(g_ws_mu);
  CachedWorkspace* e = nullptr;
  for (int i = 0; i < g_ws_used && !e; ++i)
    if (g_ws[i].stream == s && g_ws[i].dev == dev) e = &g_ws[i];
  if (!e) {
    if (g_ws_used == kCachedStreams) return false;
    hipEvent_t ev = nullptr;
    if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) {
      (void)hipGetLastError();
      return false;
    }
    e = &g_ws[g_ws_used++];
    *e = CachedWorkspace{s, dev, ev, false, nullptr, 0};
  }
  if (e->recorded && hipStreamWaitEvent(s, e->done, 0) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (e->bytes < bytes) {
    const size_t grown = (bytes + kCachedGrain - 1) / kCachedGrain * kCachedGrain;
    float* w = nullptr;
    if (pool_alloc(&w, grown, s) != hipSuccess) {
      (void)hipGetLastError();
      return false;
    }
    if (e->w) (void)hipFreeAsync(e->w, s);
    e->w = w;
    e->bytes = grown;
  }
  ws.w = e->w;
  ws.s = s;
  ws.cached = e;
  ws.cache_lock = std::move(lock);
  return true;
}

// A workspace of `floats` floats for this call on `s`: the stream's cached one
// (one per call at a time: the cache lock is held while it is borrowed), else
// a stream-ordered allocation freed after the call's last kernel.
int alloc_floats(Workspace& ws, size_t floats, hipStream_t s) {
  const size_t bytes = floats * sizeof(float);
  if (t_scratch) {  // fgr_solve_noalloc: a piece of the scratch array
    ScratchCall& sc = *t_scratch;
    const size_t off = (sc.used + 255) & ~size_t(255);
    if (!sc.dry && off + bytes > kScratchBytes) return FGR_ERR_SCRATCH;  // the dry pass rules this out
    sc.used = off + bytes;
    ws.w = reinterpret_cast<float*>(sc.dry ? kDryBase + off : reinterpret_cast<uintptr_t>(sc.base) + off);
    ws.s = s;
    return FGR_OK;
  }
  const long long limit = g_ws_limit.load(std::memory_order_relaxed);
  if (limit >= 0 && bytes > (unsigned long long)limit) return FGR_ERR_LAUNCH;  // as a failed allocation
  if (cached_workspace(ws, bytes, s)) return FGR_OK;
  ws.s = s;
  if (pool_alloc(&ws.w, bytes, s) != hipSuccess) {
    ws.w = nullptr;
    (void)hipGetLastError();  // the caller runs the unsplit kernel instead
    return FGR_ERR_LAUNCH;
  }
  ws.owned = true;
  return FGR_OK;
}

// The parts' sum into C: `slices` (a power of two <= min(parts, 16)) threads
// per output, each adding a contiguous run of parts, so that few outputs
// still give many loads in flight.
int launch_reduce_parts(const float* W, float* C, int M, int K, int parts, bool vec, hipStream_t s) {
  int64_t n = (int64_t)M * K;
  const int64_t items = vec ? n / 4 : n;
  int slices = 1;
  while (slices * 2 <= std::min(parts, fgr::kReduceMaxSlices)) slices *= 2;
  const int64_t blocks = cdiv(items, fgr::kReduceThreads / slices);
  void* args[] = {&W, &C, &n, &parts, &slices};
  return launch(vec ? reinterpret_cast<const void*>(&fgr::reduce_parts_kernel<4>)
                    : reinterpret_cast<const void*>(&fgr::reduce_parts_kernel<1>),
                blocks, fgr::kReduceThreads, args, s);
}

template <class Cfg, bool VEC>
int launch_mfma(const float* A, const float* B, float* C, int M, int N, int K, hipStream_t s) {
  int tiles_m = (int)cdiv(M, Cfg::BM);
  int tiles_n = (int)cdiv(K, Cfg::BN);
  int group = kTileGroup;
  void* args[] = {&A, &B, &C, &M, &N, &K, &tiles_m, &tiles_n, &group};
  return launch(reinterpret_cast<const void*>(&fgr::gemm_mfma_kernel<Cfg, VEC>),
                (int64_t)tiles_m * tiles_n, Cfg::kThreads, args, s);
}

using Tile256 = fgr::MfmaConfig<256, 256, 32, 2, 4>;  // 8 waves, 128x64 each
// 32-bit loads stage four times as many registers per chunk: 16-deep chunks
// keep them within the register budget (32-deep ones spilled)
using Tile256Scalar = fgr::MfmaConfig<256, 256, 16, 2, 4>;
using TileDma = fgr::DmaConfig<4>;  // 256x256, 4 waves of 128x128 (accumulators in AGPRs), 4 LDS stages
// 4-byte copies for rows that are not 16-byte aligned: four times as many, so
// 3 stages (the copies in flight must fit the wave's vmcnt counter)
using TileDmaScalar = fgr::DmaConfig<3, false>;

template <class Cfg>
const void* dma_kernel() {
  return reinterpret_cast<const void*>(&fgr::gemm_mfma_dma_kernel<Cfg>);
}

// The direct-copy kernel over the first `count` tiles of the grouped order
// (count < 0: all of them). Each operand takes 16-byte copies when its rows
// are 16-byte aligned; with one operand so, 4 + 16 copies per wave and chunk
// still fit 4 stages (measured on MI355X, TFLOP/s, 4-byte copies of both vs
// of the unaligned one only: 8192 x 6143 x 4096 and 8192 x 6144 x 4095, see
// the design notes).
int launch_mfma_dma(const float* A, const float* B, float* C, int M, int N, int K, int64_t count,
                    hipStream_t s) {
  int tiles_m = (int)cdiv(M, TileDma::BM);
  int tiles_n = (int)cdiv(K, TileDma::BN);
  int group = kTileGroup;
  void* args[] = {&A, &B, &C, &M, &N, &K, &tiles_m, &tiles_n, &group};
  const bool va = N % 4 == 0 && aligned(A, 16);
  const bool vb = K % 4 == 0 && aligned(B, 16);
  const bool vc = K % 4 == 0 && aligned(C, 16);
  const void* kernel;
  if (va && vb) kernel = vc ? dma_kernel<TileDma>() : dma_kernel<fgr::DmaConfig<4, true, true, false>>();
  else if (va) kernel = vc ? dma_kernel<fgr::DmaConfig<4, true, false, true>>()
                           : dma_kernel<fgr::DmaConfig<4, true, false, false>>();
  else if (vb) kernel = vc ? dma_kernel<fgr::DmaConfig<4, false, true, true>>()
                           : dma_kernel<fgr::DmaConfig<4, false, true, false>>();
  else kernel = dma_kernel<TileDmaScalar>();
  return launch(kernel, count < 0 ? (int64_t)tiles_m * tiles_n : count, TileDma::kThreads, args, s);
}
using Tile128 = fgr::MfmaConfig<128, 128, 16, 2, 2>;
using Tile64 = fgr::MfmaConfig<64, 64, 16, 2, 2>;

template <bool VEC>
int launch_mfma_tile(int tile, const float* A, const float* B, float* C, int M, int N, int K,
                     hipStream_t s) {
  switch (tile) {
    case FGR_TILE_256:
      if constexpr (VEC) return launch_mfma<Tile256, true>(A, B, C, M, N, K, s);
      else return launch_mfma<Tile256Scalar, false>(A, B, C, M, N, K, s);
    case FGR_TILE_128: return launch_mfma<Tile128, VEC>(A, B, C, M, N, K, s);
    case FGR_TILE_64: return launch_mfma<Tile64, VEC>(A, B, C, M, N, K, s);
    default: return FGR_ERR_BAD_PATH;
  }
}

template <class Cfg, bool VEC>
int launch_split(const float* A, const float* B, float* C, int M, int N, int K, hipStream_t s) {
  int tiles_m = (int)cdiv(M, Cfg::BM);
  int tiles_n = (int)cdiv(K, Cfg::BN);
  int group = kTileGroup;
  int first = 0, sub = 0;
  void* args[] = {&A, &B, &C, &M, &N, &K, &tiles_m, &tiles_n, &group, &first, &sub};
  return launch(reinterpret_cast<const void*>(&fgr::gemm_mfma_split_kernel<Cfg, VEC>),
                (int64_t)tiles_m * tiles_n, Cfg::kThreads, args, s);
}

// The split kernel over big tiles [first, first + count) of a BIG x BIG grid
// (same grouped order as the kernel that ran the others), each cut into
// (BIG / BM)^2 tiles.
template <class Cfg, int BIG, bool VEC>
int launch_split_big(const float* A, const float* B, float* C, int M, int N, int K, int first, int count,
                     hipStream_t s) {
  int tiles_m = (int)cdiv(M, BIG);
  int tiles_n = (int)cdiv(K, BIG);
  int group = kTileGroup;
  int sub = BIG / Cfg::BM;
  void* args[] = {&A, &B, &C, &M, &N, &K, &tiles_m, &tiles_n, &group, &first, &sub};
  return launch(reinterpret_cast<const void*>(&fgr::gemm_mfma_split_kernel<Cfg, VEC>),
                (int64_t)count * sub * sub, Cfg::kThreads, args, s);
}

using Split32 = fgr::SplitConfig<32, 32, 16, 4>;
using Split64x4 = fgr::SplitConfig<64, 64, 16, 4>;
using Split64x8 = fgr::SplitConfig<64, 64, 16, 8>;
// 16 waves per 32x32 tile, each a sixteenth of the reduction: for tails of a
// few tiles, where a wave's chain of dependent chunk loads sets the time
using Split32x16 = fgr::SplitConfig<32, 32, 16, 16>;

// The split kernel over the BIG x BIG tiles [full, full + rem): 64x64 pieces
// (eight waves each while there are fewer than two per CU), or 32x32 pieces
// while 64x64 ones would leave CUs idle (sixteen waves each while even those
// leave CUs idle).
template <int BIG, bool VEC>
int launch_split_tail(const float* A, const float* B, float* C, int M, int N, int K, int64_t full, int64_t rem,
                      int cus, hipStream_t s) {
  constexpr int64_t per64 = (BIG / 64) * (BIG / 64), per32 = (BIG / 32) * (BIG / 32);
  if (rem * per64 >= 2 * cus) return launch_split_big<Split64x4, BIG, VEC>(A, B, C, M, N, K, (int)full, (int)rem, s);
  if (rem * per64 >= cus) return launch_split_big<Split64x8, BIG, VEC>(A, B, C, M, N, K, (int)full, (int)rem, s);
  if (rem * per32 >= cus) return launch_split_big<Split32, BIG, VEC>(A, B, C, M, N, K, (int)full, (int)rem, s);
  return launch_split_big<Split32x16, BIG, VEC>(A, B, C, M, N, K, (int)full, (int)rem, s);
}

// Whole waves of 256x256 tiles (one tile per CU) on the direct-copy kernel;
// the tiles of the last, partial wave on the split kernel, cut into 64x64
// tiles (32x32 while 64x64 would leave CUs idle), so that the tail occupies
// every CU instead of a few.
int launch_dma_tail(const float* A, const float* B, float* C, int M, int N, int K, int cus, hipStream_t s) {
  const int64_t tiles = cdiv(M, TileDma::BM) * cdiv(K, TileDma::BN);
  const int64_t full = tiles / cus * cus;
  const int64_t rem = tiles - full;
  if (full > 0) {
    const int rc = launch_mfma_dma(A, B, C, M, N, K, full, s);
    if (rc != FGR_OK || rem == 0) return rc;
  }
  if (full > INT_MAX || rem > INT_MAX / 64) return FGR_ERR_BAD_DIMS;
  if (mfma_vec_ok(A, B, C, N, K)) return launch_split_tail<256, true>(A, B, C, M, N, K, full, rem, cus, s);
  return launch_split_tail<256, false>(A, B, C, M, N, K, full, rem, cus, s);
}

// Configurations with kStrip cover columns [0, 64 q) with tiles and add the
// strip's workgroups (four rows of A each) after them.
template <class Cfg>
int launch_ksplit_cfg(const float* A, const float* B, float* C, int M, int N, int K, int64_t count, hipStream_t s,
                      int parts, float* W, int first, int compact, int nfull) {
  int tiles_m = (int)cdiv(M, Cfg::BM);
  int tiles_n = (int)cdiv(Cfg::kStrip ? K / Cfg::BN * Cfg::BN : K, Cfg::BN);
  int group = kTileGroup;
  void* args[] = {&A,     &B,    &C,     &M,       &N,     &K,     &tiles_m, &tiles_n, &group,
                  &parts, &W,    &first, &compact, &nfull};
  const int64_t strip_blocks = Cfg::kStrip ? cdiv(M, fgr::kStripRows) : 0;
  const void* kernel;
  if constexpr (Cfg::kReg) kernel = reinterpret_cast<const void*>(&fgr::gemm_mfma_kreg_kernel<Cfg>);
  else kernel = reinterpret_cast<const void*>(&fgr::gemm_mfma_ksplit_kernel<Cfg>);
  return launch(kernel,
                nfull + (count < 0 ? (int64_t)tiles_m * tiles_n : count) * parts + strip_blocks, Cfg::kThreads,
                args, s);
}

// k-split configurations by tile and by the row alignment of the product.
// 64x64 and 32x32 tiles with 16-byte rows of A, B and C, and the skinny
// 32x128 tiles: direct copies through LDS (KsplitConfig; 32x128 with 4-byte
// copies of an operand whose rows are not 16-byte aligned). All other tiles
// (128x128; 64x64 and 32x32 with unaligned rows): operands loaded straight
// into registers at any 4-byte alignment (KregConfig; 128x128 needs K >= 4
// and 64x64 K >= 2, run() maps K = 1 to 32x32). Measured on MI355X (us per
// call), aligned rows, LDS vs registers: 64x64 96 x 8192 x 4096 67 vs 84,
// 2048^3 134 vs 139; 32x32 96 x 8192 x 4096 (split) 81 vs 97; unaligned rows,
// 4-byte copies vs registers: 64x64 1023 x 1025 x 1023 27.6 vs 21.4, 2047 x
// 2049 x 2051 227 vs 173; 32x32 250 x 1001 x 250 11.4 vs 7.2.
constexpr int kKregDepth = 2;  // chunks of operands in registers: deeper rings measured slower

template <int BM, int BN = BM>
int launch_ksplit_rows(Rows rows, const float* A, const float* B, float* C, int M, int N, int K, int64_t count,
                       hipStream_t s, int parts, float* W, int first, int compact, int nfull) {
  if constexpr (BM == BN) {
    if constexpr (BM <= 64) {
      if (rows == Rows::kAll && fgr::ksplit_offsets_fit(BM, N, K))
        return launch_ksplit_cfg<fgr::KsplitConfig<BM, 4, true>>(A, B, C, M, N, K, count, s, parts, W, first,
                                                                 compact, nfull);
    }
    if (K < BM / 32) return FGR_ERR_BAD_PATH;
    // buffer loads at 128x128 where their offsets fit (see KregConfig)
    if constexpr (BM == 128) {
      if (fgr::ksplit_offsets_fit(BM, N, K))
        return launch_ksplit_cfg<fgr::KregConfig<BM, kKregDepth, false, true>>(A, B, C, M, N, K, count, s, parts, W,
                                                                             first, compact, nfull);
    }
    return launch_ksplit_cfg<fgr::KregConfig<BM, kKregDepth, false, false>>(A, B, C, M, N, K, count, s, parts, W,
                                                                          first, compact, nfull);
  } else {
    if (!fgr::ksplit_offsets_fit(BM, N, K)) return FGR_ERR_BAD_PATH;
    switch (rows) {
      case Rows::kAll:
        return launch_ksplit_cfg<fgr::KsplitConfig<BM, 4, true, BN>>(A, B, C, M, N, K, count, s, parts, W, first,
                                                                      compact, nfull);
      case Rows::kAOnly:
        return launch_ksplit_cfg<fgr::KsplitConfig<BM, 4, true, BN, false>>(A, B, C, M, N, K, count, s, parts, W,
                                                                             first, compact, nfull);
      case Rows::kBOnly:
        return launch_ksplit_cfg<fgr::KsplitConfig<BM, 4, false, BN, true>>(A, B, C, M, N, K, count, s, parts, W,
                                                                             first, compact, nfull);
      default:
        return launch_ksplit_cfg<fgr::KsplitConfig<BM, 4, false, BN>>(A, B, C, M, N, K, count, s, parts, W, first,
                                                                       compact, nfull);
    }
  }
}

// The k-split kernels with tile x tile tiles over tiles [first, first + count)
// of the grouped order (count < 0: all of them). parts > 1: each tile's
// reduction also split over `parts` workgroups writing partial tiles to W (at
// their place in copies of C, or in compact per-tile slots). nfull > 0: the
// same grid first runs whole tiles [first, first + nfull) into C, and the
// count split tiles follow them.
int launch_ksplit(int tile, const float* A, const float* B, float* C, int M, int N, int K, int64_t count,
                  hipStream_t s, int parts = 1, float* W = nullptr, int first = 0, int compact = 0,
                  int nfull = 0) {
  const Rows rows = rows_of(A, B, C, N, K);
  switch (tile) {
    case FGR_TILE_128:
      return launch_ksplit_rows<128>(rows, A, B, C, M, N, K, count, s, parts, W, first, compact, nfull);
    case FGR_TILE_64:
      return launch_ksplit_rows<64>(rows, A, B, C, M, N, K, count, s, parts, W, first, compact, nfull);
    case FGR_TILE_32:
      return launch_ksplit_rows<32>(rows, A, B, C, M, N, K, count, s, parts, W, first, compact, nfull);
    case FGR_TILE_32X128:
      return launch_ksplit_rows<32, 128>(rows, A, B, C, M, N, K, count, s, parts, W, first, compact, nfull);
    default: return FGR_ERR_BAD_PATH;
  }
}

// The strip plan: K = 64 q + w with 1 <= w <= kStripMax. One launch of a
// k-split kernel: its 64x64 tiles cover columns [0, 64 q) and, after them,
// workgroups of four rows of A each compute C's last w columns on the vector
// ALUs (strip.hpp). No workspace. Direct 16-byte copies when the rows of A, B
// and C allow them, else operands straight into registers.
int launch_strip(const float* A, const float* B, float* C, int M, int N, int K, hipStream_t s) {
  if (rows_of(A, B, C, N, K) == Rows::kAll && fgr::ksplit_offsets_fit(64, N, K))
    return launch_ksplit_cfg<fgr::KsplitConfig<64, 4, true, 64, true, true>>(A, B, C, M, N, K, -1, s, 1, nullptr,
                                                                            0, 0, 0);
  return launch_ksplit_cfg<fgr::KregConfig<64, kKregDepth, true, false>>(A, B, C, M, N, K, -1, s, 1, nullptr, 0, 0,
                                                                        0);
}

// Sum of compact partial tiles (tiles [first, first + count) of the grouped
// order, tile x tile each) into C.
int launch_reduce_tiles(const float* W, float* C, int M, int K, int tile, int parts, int first, int count,
                        hipStream_t s) {
  int tiles_m = (int)cdiv(M, tile);
  int tiles_n = (int)cdiv(K, tile);
  int group = kTileGroup;
  void* args[] = {&W, &C, &M, &K, &parts, &tiles_m, &tiles_n, &group, &first, &count};
  const int64_t blocks = (int64_t)tile * tile / fgr::kReduceThreads;
  switch (tile) {
    case FGR_TILE_128:
      return launch(reinterpret_cast<const void*>(&fgr::reduce_tiles_kernel<128>), blocks, fgr::kReduceThreads,
                    args, s, count);
    case FGR_TILE_64:
      return launch(reinterpret_cast<const void*>(&fgr::reduce_tiles_kernel<64>), blocks, fgr::kReduceThreads,
                    args, s, count);
    default: return FGR_ERR_BAD_PATH;
  }
}

bool vec4_rows(const float* C, int M, int K) { return ((int64_t)M * K) % 4 == 0 && aligned(C, 16); }

// k-split tiles with the reduction also split across workgroups: the partial
// tiles into a stream-ordered workspace, then added in part order (two parts
// where no longer parts fit the estimate's limits). Without a
// workspace (allocation failed) the tiles keep their whole reduction.
int split_parts(int tile, int M, int N, int K, int cus) {
  const int parts =
      tile == FGR_TILE_32X128 ? skinny_parts(M, N, K, cus) : splitk_plan_tile(tile, M, N, K, cus, true).parts;
  return parts < 2 ? 2 : parts;  // N >= 128 gives 8 chunks per part
}

int launch_ksplit_parts(int tile, const float* A, const float* B, float* C, int M, int N, int K, int cus,
                        hipStream_t s) {
  const int parts = split_parts(tile, M, N, K, cus);
  Workspace ws;
  if (alloc_floats(ws, (size_t)parts * (size_t)M * (size_t)K, s) != FGR_OK)
    return launch_ksplit(tile, A, B, C, M, N, K, -1, s);
  const int rc = launch_ksplit(tile, A, B, C, M, N, K, -1, s, parts, ws.w);
  if (rc != FGR_OK) return rc;
  return launch_reduce_parts(ws.w, C, M, K, parts, vec4_rows(C, M, K), s);
}

constexpr int kTailSplitMinN = 4096;
constexpr int kMixedTailMinN = 1024;

// Whole waves of tile x tile tiles on the k-split kernel, the last partial
// wave's tiles cut into smaller split-reduction tiles (as launch_dma_tail) or,
// for long reductions, their reduction split across workgroups.
int launch_ksplit_tail(int tile, const float* A, const float* B, float* C, int M, int N, int K,
                       int cus, hipStream_t s) {
  const int64_t tiles = cdiv(M, tile) * cdiv(K, tile);
  const int64_t full = tiles / cus * cus;
  const int64_t rem = tiles - full;
  if (full > INT_MAX || rem > INT_MAX / 16) return FGR_ERR_BAD_DIMS;
  // 64x64 tiles (two workgroups fit a CU) and N >= kMixedTailMinN: the tail
  // tiles' reduction split over CUs / rem parts in the same grid as the whole
  // tiles, so that they run next to the full wave on every CU, then their
  // parts added. Measured on MI355X (us per call, separate tail launch vs one
  // grid): 1023 x 1025 x 1027 41.0 vs 37.9, 2047 x 2049 x 2051 211 vs 203,
  // 1536^3 75.0 vs 71.8, 1023 x 4097 x 1027 114.6 vs 109.1, 1040 x 2048 x
  // 1040 53.9 vs 51.5; with short reductions the adding launch costs more
  // than the overlap gives (1030 x 128 x 1030 13.9 vs 15.6, 1088 x 512 x 1024
  // 19.4 vs 21.7).
  const int mixed_parts = (int)std::min<int64_t>(cus / std::max<int64_t>(rem, 1), cdiv(N, 8) / 8);
  if (tile == FGR_TILE_64 && N >= kMixedTailMinN && full > 0 && rem > 0 && mixed_parts >= 2) {
    Workspace ws;
    if (alloc_floats(ws, (size_t)mixed_parts * (size_t)rem * tile * tile, s) == FGR_OK) {
      const int rc = launch_ksplit(tile, A, B, C, M, N, K, rem, s, mixed_parts, ws.w, 0, 1, (int)full);
      if (rc != FGR_OK) return rc;
      return launch_reduce_tiles(ws.w, C, M, K, tile, mixed_parts, (int)full, (int)rem, s);
    }
  }
  if (full > 0) {
    const int rc = launch_ksplit(tile, A, B, C, M, N, K, full, s);
    if (rc != FGR_OK || rem == 0) return rc;
  }
  // With a long reduction the tail tiles' reduction is split over up to
  // CUs / rem parts (so every CU gets a workgroup), through compact per-tile
  // slots; otherwise, or without a workspace, the tail is cut into smaller
  // tiles of the split kernel. Measured on MI355X (us per call, split kernel
  // tail vs split reduction): 1023 x 4097 x 1027 132 vs 114, 1536 x 16384 x
  // 1536 680 vs 630; but 2047^3 equal, 3072^3 446 vs 456, 1023 x 1025 x 1027
  // 45 vs 48 (three launches and the workspace cost more than they save).
  const int parts = N >= kTailSplitMinN ? (int)std::min<int64_t>(cus / rem, cdiv(N, 8) / 8) : 1;
  if (parts >= 2 && rem <= 65535) {
    Workspace ws;
    if (alloc_floats(ws, (size_t)parts * (size_t)rem * tile * tile, s) == FGR_OK) {
      const int rc = launch_ksplit(tile, A, B, C, M, N, K, rem, s, parts, ws.w, (int)full, 1);
      if (rc != FGR_OK) return rc;
      return launch_reduce_tiles(ws.w, C, M, K, tile, parts, (int)full, (int)rem, s);
    }
  }
  const bool vec = mfma_vec_ok(A, B, C, N, K);
  if (tile == FGR_TILE_128)
    return vec ? launch_split_tail<128, true>(A, B, C, M, N, K, full, rem, cus, s)
               : launch_split_tail<128, false>(A, B, C, M, N, K, full, rem, cus, s);
  if (tile == FGR_TILE_64)
    return vec ? launch_split_tail<64, true>(A, B, C, M, N, K, full, rem, cus, s)
               : launch_split_tail<64, false>(A, B, C, M, N, K, full, rem, cus, s);
  return FGR_ERR_BAD_PATH;
}

template <bool VEC>
int launch_split_tile(int tile, const float* A, const float* B, float* C, int M, int N, int K, int cus,
                      hipStream_t s) {
  if (tile == FGR_TILE_32) return launch_split<Split32, VEC>(A, B, C, M, N, K, s);
  // 64x64 tiles: eight waves per tile while the tiles alone would fill fewer
  // than two waves of workgroups, four otherwise
  if (cdiv(M, 64) * cdiv(K, 64) < 2 * cus) return launch_split<Split64x8, VEC>(A, B, C, M, N, K, s);
  return launch_split<Split64x4, VEC>(A, B, C, M, N, K, s);
}

// The vector-ALU kernel (128x128 tiles, 8-deep reduction chunks: 16-deep
// ones made the compiler hold the whole chunk's operands and exceed 256 VGPRs).
template <bool VEC>
int launch_valu(const float* A, const float* B, float* C, int M, int N, int K, hipStream_t s) {
  using Cfg = fgr::ValuConfig<8, VEC>;
  int tiles_m = (int)cdiv(M, Cfg::BM);
  int tiles_n = (int)cdiv(K, Cfg::BN);
  int group = kTileGroup;
  void* args[] = {&A, &B, &C, &M, &N, &K, &tiles_m, &tiles_n, &group};
  return launch(reinterpret_cast<const void*>(&fgr::gemm_valu_kernel<Cfg>), (int64_t)tiles_m * tiles_n,
                fgr::kValuThreads, args, s);
}

// Rows of A per matrix-vector workgroup: the smallest of 1, 2, 4, 8 that holds
// all M rows (B is streamed once). Each lane keeps one row of B in
// flight (two at 8 rows): with 16 waves per CU that saturates HBM, and more
// loads in flight measured slower (M = 1: 5.79 TB/s with one, 4.82 with four).
template <int VW, int COLS>
int launch_gemv_parts(const float* A, const float* B, float* C, int M, int N, int K, int parts, float* W,
                      hipStream_t s) {
  void* args[] = {&A, &B, &C, &M, &N, &K, &parts, &W};
  const int64_t blocks = cdiv(K, COLS);
  const void* kernel;
  if (M <= 1) kernel = reinterpret_cast<const void*>(&fgr::gemv_kernel<VW, 1024, 1, 1, fgr::kGemvAFloats, COLS>);
  else if (M <= 2) kernel = reinterpret_cast<const void*>(&fgr::gemv_kernel<VW, 1024, 1, 2, fgr::kGemvAFloats, COLS>);
  else if (M <= 4) kernel = reinterpret_cast<const void*>(&fgr::gemv_kernel<VW, 1024, 1, 4, fgr::kGemvAFloats, COLS>);
  else kernel = reinterpret_cast<const void*>(&fgr::gemv_kernel<VW, 1024, 2, 8, fgr::kGemvAFloats, COLS>);
  return launch(kernel, blocks, 1024, args, s, parts);
}

// The matrix-vector kernel with the plan above: the partial rows of a split
// into a workspace, then added in part order (without a workspace the
// unsplit kernel runs).
template <int VW>
int launch_gemv(const float* A, const float* B, float* C, int M, int N, int K, int cus, hipStream_t s) {
  const GemvPlan plan = gemv_plan(M, N, K, cus);
  Workspace ws;
  float* W = nullptr;
  if (plan.parts >= 2 && alloc_floats(ws, (size_t)plan.parts * (size_t)M * (size_t)K, s) == FGR_OK) W = ws.w;
  const int p = W ? plan.parts : 1;
  const int rc = plan.cols == fgr::kGemvCols
                     ? launch_gemv_parts<VW, fgr::kGemvCols>(A, B, C, M, N, K, p, W, s)
                     : launch_gemv_parts<VW, fgr::kGemvCols / 2>(A, B, C, M, N, K, p, W, s);
  if (rc != FGR_OK || !W) return rc;
  return launch_reduce_parts(W, C, M, K, p, vec4_rows(C, M, K), s);
}

int dispatch(const float* A, const float* B, float* C, int M, int N, int K, hipStream_t s, int cus, int path,
             int tile);

int run(const float* A, const float* B, float* C, int M, int N, int K, void* stream, int path,
        int tile, bool noalloc = false) {
  int rc = check_args(A, B, C, M, N, K);
  if (rc != FGR_OK) return rc;
  switch (path) {
    case FGR_PATH_AUTO: break;
    case FGR_PATH_MFMA_VEC:
      if (!mfma_vec_ok(A, B, C, N, K)) return FGR_ERR_BAD_PATH;
      break;
    case FGR_PATH_MFMA_DMA:
    case FGR_PATH_MFMA_DMA_TAIL:
      if (!mfma_dma_ok(N, K) || (tile != FGR_TILE_AUTO && tile != FGR_TILE_256)) return FGR_ERR_BAD_PATH;
      break;
    case FGR_PATH_MFMA_KSPLIT:
    case FGR_PATH_MFMA_KSPLIT_TAIL:
      // N >= 64; tiles of 128 (K >= 4) or 64, and 32 or 32x128 without the tail form
      if (N < 64 || (tile == FGR_TILE_128 && !ksplit128_ok(K)) || tile == FGR_TILE_256 ||
          ((tile == FGR_TILE_32 || tile == FGR_TILE_32X128) && path == FGR_PATH_MFMA_KSPLIT_TAIL))
        return FGR_ERR_BAD_PATH;
      break;
    case FGR_PATH_MFMA_SPLITK:
      // N >= 128 (two parts of at least 8 chunks); tiles of 128 (K >= 4), 64 or 32
      if (N < 128 || (tile == FGR_TILE_128 && !ksplit128_ok(K)) || tile == FGR_TILE_256)
        return FGR_ERR_BAD_PATH;
      break;
    case FGR_PATH_VALU:
      if (tile != FGR_TILE_AUTO && tile != FGR_TILE_128) return FGR_ERR_BAD_PATH;
      break;
    case FGR_PATH_MFMA_STRIP:
      if (!strip_shape(M, N, K) || (tile != FGR_TILE_AUTO && tile != FGR_TILE_64)) return FGR_ERR_BAD_PATH;
      break;
    case FGR_PATH_MFMA_SCALAR: break;
    case FGR_PATH_MFMA_SPLIT:
      if (tile != FGR_TILE_AUTO && tile != FGR_TILE_32 && tile != FGR_TILE_64) return FGR_ERR_BAD_PATH;
      break;
    case FGR_PATH_GEMV_VEC:
      if (M > fgr::kGemvMaxRows || !gemv_vec_ok(B, K)) return FGR_ERR_BAD_PATH;
      break;
    case FGR_PATH_GEMV_SCALAR:
      if (M > fgr::kGemvMaxRows) return FGR_ERR_BAD_PATH;
      break;
    default: return FGR_ERR_BAD_PATH;
  }
  if (tile != FGR_TILE_AUTO && tile != FGR_TILE_256 && tile != FGR_TILE_128 && tile != FGR_TILE_64 &&
      tile != FGR_TILE_32 && tile != FGR_TILE_32X128)
    return FGR_ERR_BAD_PATH;
  if (tile == FGR_TILE_32X128 &&
      (N < 64 || !fgr::ksplit_offsets_fit(32, N, K) ||
       (path != FGR_PATH_MFMA_KSPLIT && path != FGR_PATH_MFMA_SPLITK && path != FGR_PATH_AUTO)))
    return FGR_ERR_BAD_PATH;  // direct copies need N >= 64 and 32-bit copy offsets
  if (tile == FGR_TILE_32 && path != FGR_PATH_MFMA_SPLIT && path != FGR_PATH_MFMA_KSPLIT &&
      path != FGR_PATH_MFMA_SPLITK && path != FGR_PATH_AUTO)
    return FGR_ERR_BAD_PATH;

  int cus = 0, dev = -1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  rc = device_for(s, &cus, &dev);
  if (rc != FGR_OK) return rc;
  const Choice best = choose(A, B, C, M, N, K, cus);
  if (path == FGR_PATH_AUTO) {
    if (tile == FGR_TILE_AUTO) {
      path = best.path;
      tile = best.tile;
    } else if (best.path == FGR_PATH_GEMV_VEC || best.path == FGR_PATH_GEMV_SCALAR) {
      path = best.path;  // the matrix-vector kernel has no tiles
    } else if (tile == best.tile && (best.path == FGR_PATH_MFMA_DMA || best.path == FGR_PATH_MFMA_DMA_TAIL ||
                                     best.path == FGR_PATH_MFMA_KSPLIT || best.path == FGR_PATH_MFMA_KSPLIT_TAIL ||
                                     best.path == FGR_PATH_MFMA_SPLITK || best.path == FGR_PATH_MFMA_SPLIT ||
                                     best.path == FGR_PATH_MFMA_STRIP)) {
      path = best.path;  // the kernel the table picked for this tile
    } else if (tile == FGR_TILE_32) {
      path = FGR_PATH_MFMA_SPLIT;  // 32x32 tiles for any shape
    } else if (tile == FGR_TILE_32X128) {
      path = FGR_PATH_MFMA_KSPLIT;  // the only kernel with 32x128 tiles (N >= 64 checked above)
    } else {
      path = mfma_vec_ok(A, B, C, N, K) ? FGR_PATH_MFMA_VEC : FGR_PATH_MFMA_SCALAR;
    }
  }
  if (tile == FGR_TILE_AUTO) tile = default_tile(path, best, M, N, K, cus, mfma_vec_ok(A, B, C, N, K));
  if (tile == FGR_TILE_64 && K < 2 &&
      (path == FGR_PATH_MFMA_KSPLIT || path == FGR_PATH_MFMA_KSPLIT_TAIL || path == FGR_PATH_MFMA_SPLITK)) {
    // the register-fed 64x64 tiles load B two columns at a time: one column
    // takes 32x32 tiles (which have no tail form)
    tile = FGR_TILE_32;
    if (path == FGR_PATH_MFMA_KSPLIT_TAIL) path = FGR_PATH_MFMA_KSPLIT;
  }
  if (!noalloc) return dispatch(A, B, C, M, N, K, s, cus, path, tile);

  // fgr_solve_noalloc: the same plan, its workspace from the scratch array
  char* base = nullptr;
  rc = scratch_of(dev, &base);
  if (rc != FGR_OK) return rc;
  ScratchCall call;
  struct Reset {
    ~Reset() { t_scratch = nullptr; }
  } reset;
  t_scratch = &call;
  rc = dispatch(A, B, C, M, N, K, s, cus, path, tile);  // dry: count the bytes
  if (rc != FGR_OK) return rc;
  const long long limit = g_ws_limit.load(std::memory_order_relaxed);
  if (call.used > kScratchBytes || (limit >= 0 && call.used > (unsigned long long)limit))
    return FGR_ERR_SCRATCH;  // nothing enqueued
  call = ScratchCall{false, base, 0};
  return dispatch(A, B, C, M, N, K, s, cus, path, tile);
}

// The launches of one call's plan (path and tile resolved).
int dispatch(const float* A, const float* B, float* C, int M, int N, int K, hipStream_t s, int cus, int path,
             int tile) {
  switch (path) {
    case FGR_PATH_MFMA_DMA: return launch_mfma_dma(A, B, C, M, N, K, -1, s);
    case FGR_PATH_MFMA_DMA_TAIL: return launch_dma_tail(A, B, C, M, N, K, cus, s);
    case FGR_PATH_MFMA_KSPLIT:
    case FGR_PATH_MFMA_KSPLIT_TAIL:
    case FGR_PATH_MFMA_SPLITK:
      if (path == FGR_PATH_MFMA_KSPLIT) return launch_ksplit(tile, A, B, C, M, N, K, -1, s);
      if (path == FGR_PATH_MFMA_KSPLIT_TAIL) return launch_ksplit_tail(tile, A, B, C, M, N, K, cus, s);
      return launch_ksplit_parts(tile, A, B, C, M, N, K, cus, s);
    case FGR_PATH_MFMA_VEC: return launch_mfma_tile<true>(tile, A, B, C, M, N, K, s);
    case FGR_PATH_MFMA_SCALAR: return launch_mfma_tile<false>(tile, A, B, C, M, N, K, s);
    case FGR_PATH_MFMA_SPLIT:
      return mfma_vec_ok(A, B, C, N, K) ? launch_split_tile<true>(tile, A, B, C, M, N, K, cus, s)
                                        : launch_split_tile<false>(tile, A, B, C, M, N, K, cus, s);
    case FGR_PATH_MFMA_STRIP: return launch_strip(A, B, C, M, N, K, s);
    case FGR_PATH_GEMV_VEC: return launch_gemv<4>(A, B, C, M, N, K, cus, s);
    case FGR_PATH_GEMV_SCALAR: return launch_gemv<1>(A, B, C, M, N, K, cus, s);
    case FGR_PATH_VALU:
      return mfma_vec_ok(A, B, C, N, K) ? launch_valu<true>(A, B, C, M, N, K, s)
                                        : launch_valu<false>(A, B, C, M, N, K, s);
  }
  return FGR_ERR_BAD_PATH;
}

// The controlled comparison (buffering x output tile x reduction chunk, each
// variant a kernel of its own, timed alike): the register-staged kernel with
// one LDS buffer or two (with register prefetch), 256x256 / 256x128 / 128x128
// tiles and 16- or 32-deep chunks, and the direct-copy kernel with LDS rings
// of 3, 4 and 5 stages (256x256 tiles, 16-deep chunks). 16-byte rows only.
struct Variant {
  const char* name;
  int (*run)(const float*, const float*, float*, int, int, int, hipStream_t);
  bool dma;
};

template <int BM, int BN, int BK, int WN, int BUFS>
int run_regs_variant(const float* A, const float* B, float* C, int M, int N, int K, hipStream_t s) {
  return launch_mfma<fgr::MfmaConfig<BM, BN, BK, 2, WN, 1, BUFS>, true>(A, B, C, M, N, K, s);
}

template <int S>
int run_dma_variant(const float* A, const float* B, float* C, int M, int N, int K, hipStream_t s) {
  int tiles_m = (int)cdiv(M, 256);
  int tiles_n = (int)cdiv(K, 256);
  int group = kTileGroup;
  void* args[] = {&A, &B, &C, &M, &N, &K, &tiles_m, &tiles_n, &group};
  return launch(dma_kernel<fgr::DmaConfig<S>>(), (int64_t)tiles_m * tiles_n, fgr::DmaConfig<S>::kThreads, args, s);
}

constexpr Variant kVariants[] = {
    {"regs single 256x256 bk16", &run_regs_variant<256, 256, 16, 4, 1>, false},
    {"regs single 256x256 bk32", &run_regs_variant<256, 256, 32, 4, 1>, false},
    {"regs single 256x128 bk16", &run_regs_variant<256, 128, 16, 2, 1>, false},
    {"regs single 256x128 bk32", &run_regs_variant<256, 128, 32, 2, 1>, false},
    {"regs single 128x128 bk16", &run_regs_variant<128, 128, 16, 2, 1>, false},
    {"regs single 128x128 bk32", &run_regs_variant<128, 128, 32, 2, 1>, false},
    {"regs double 256x256 bk16", &run_regs_variant<256, 256, 16, 4, 2>, false},
    {"regs double 256x256 bk32", &run_regs_variant<256, 256, 32, 4, 2>, false},
    {"regs double 256x128 bk16", &run_regs_variant<256, 128, 16, 2, 2>, false},
    {"regs double 256x128 bk32", &run_regs_variant<256, 128, 32, 2, 2>, false},
    {"regs double 128x128 bk16", &run_regs_variant<128, 128, 16, 2, 2>, false},
    {"regs double 128x128 bk32", &run_regs_variant<128, 128, 32, 2, 2>, false},
    {"direct ring3 256x256 bk16", &run_dma_variant<3>, true},
    {"direct ring4 256x256 bk16", &run_dma_variant<4>, true},
    {"direct ring5 256x256 bk16", &run_dma_variant<5>, true},
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

int run_variant(const float* A, const float* B, float* C, int M, int N, int K, void* stream, int variant) {
  int rc = check_args(A, B, C, M, N, K);
  if (rc != FGR_OK) return rc;
  if (variant < 0 || variant >= kNumVariants || !mfma_vec_ok(A, B, C, N, K) ||
      (kVariants[variant].dma && !mfma_dma_ok(N, K)))
    return FGR_ERR_BAD_PATH;
  int cus = 0;
  rc = device_for(reinterpret_cast<hipStream_t>(stream), &cus);
  if (rc != FGR_OK) return rc;
  return kVariants[variant].run(A, B, C, M, N, K, reinterpret_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

int solve(const float* A, const float* B, float* C, int M, int N, int K, void* stream) {
  return run(A, B, C, M, N, K, stream, FGR_PATH_AUTO, FGR_TILE_AUTO);
}

int fgr_solve_noalloc(const float* A, const float* B, float* C, int M, int N, int K, void* stream) {
  return run(A, B, C, M, N, K, stream, FGR_PATH_AUTO, FGR_TILE_AUTO, /*noalloc=*/true);
}

int fgr_solve_default(const float* A, const float* B, float* C, int M, int N, int K) {
  return run(A, B, C, M, N, K, nullptr, FGR_PATH_AUTO, FGR_TILE_AUTO);
}

int fgr_solve_path(const float* A, const float* B, float* C, int M, int N, int K, void* stream,
                   int path, int tile) {
  return run(A, B, C, M, N, K, stream, path, tile);
}

int fgr_select_path(const float* A, const float* B, const float* C, int M, int N, int K) {
  const int rc = check_args(A, B, C, M, N, K);
  if (rc != FGR_OK) return rc;
  return choose(A, B, C, M, N, K, kDefaultCus).path;
}

int fgr_select_tile(const float* A, const float* B, const float* C, int M, int N, int K) {
  const int rc = check_args(A, B, C, M, N, K);
  if (rc != FGR_OK) return rc;
  return choose(A, B, C, M, N, K, kDefaultCus).tile;
}

int fgr_select_parts(const float* A, const float* B, const float* C, int M, int N, int K) {
  const int rc = check_args(A, B, C, M, N, K);
  if (rc != FGR_OK) return rc;
  const Choice c = choose(A, B, C, M, N, K, kDefaultCus);
  return c.path == FGR_PATH_MFMA_SPLITK ? split_parts(c.tile, M, N, K, kDefaultCus) : 1;
}

const char* fgr_status_string(int status) {
  switch (status) {
    case FGR_OK: return "ok";
    case FGR_ERR_NULL_POINTER: return "null pointer argument";
    case FGR_ERR_BAD_DIMS: return "M, N and K must be >= 1";
    case FGR_ERR_MISALIGNED: return "pointer not 4-byte aligned";
    case FGR_ERR_ALIAS: return "C overlaps A or B";
    case FGR_ERR_BAD_PATH: return "forced path or tile cannot run these arguments";
    case FGR_ERR_DEVICE: return "no gfx950 HIP device is current";
    case FGR_ERR_LAUNCH: return "HIP kernel launch failed";
    case FGR_ERR_SCRATCH:
      return "the plan needs more workspace than fgr_solve_noalloc's 64 MiB scratch or the workspace limit allows";
    default: return "unknown status";
  }
}

int fgr_version(void) { return kVersion; }

int fgr_stream_read(const float* X, long long n, float* out, int blocks, void* stream) {
  if (!X || !out) return FGR_ERR_NULL_POINTER;
  if (n < 4 || n % 4 != 0 || blocks < 1) return FGR_ERR_BAD_DIMS;
  if (!aligned(X, 16) || !aligned(out, 4)) return FGR_ERR_MISALIGNED;
  if (overlaps(out, blocks, X, n)) return FGR_ERR_ALIAS;
  int cus = 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int rc = device_for(s, &cus);
  if (rc != FGR_OK) return rc;
  const float4* X4 = reinterpret_cast<const float4*>(X);
  int64_t n4 = n / 4;
  void* args[] = {&X4, &n4, &out};
  return launch(reinterpret_cast<const void*>(&fgr::stream_read_kernel), blocks, fgr::kStreamThreads, args, s);
}

#ifdef FGR_TIMESTAMPS
// The measurement build's per-workgroup records of the last launch (see
// timestamps.hpp and fp32_gemm_row_timestamps.h).
int fgr_timestamps_read(void* host, int records) {
  if (!host) return FGR_ERR_NULL_POINTER;
  if (records < 1 || records > fgr::kTsRecords) return FGR_ERR_BAD_DIMS;
  const hipError_t e = hipMemcpyFromSymbol(host, HIP_SYMBOL(fgr::fgr_ts_records),
                                           (size_t)records * sizeof(fgr::TsRecord));
  return e == hipSuccess ? FGR_OK : FGR_ERR_LAUNCH;
}
#endif

long long fgr_set_workspace_limit(long long bytes) {
  return g_ws_limit.exchange(bytes < 0 ? -1 : bytes, std::memory_order_relaxed);
}

int fgr_variant_count(void) { return kNumVariants; }

const char* fgr_variant_name(int variant) {
  return variant >= 0 && variant < kNumVariants ? kVariants[variant].name : nullptr;
}

int fgr_solve_variant(const float* A, const float* B, float* C, int M, int N, int K, void* stream, int variant) {
  return run_variant(A, B, C, M, N, K, stream, variant);
}

}  // extern "C"
