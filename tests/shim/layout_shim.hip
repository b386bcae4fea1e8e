// Test infrastructure only (never linked into the product library): host entry
// points onto the library's own index and layout helpers, so that CPU tests
// can check them, and a probe kernel for the FP32 MFMA lane layout the kernels
// are written against (checked on the GPU against the CPU oracle).
#include <hip/hip_runtime.h>

#include "gemm_mfma.hpp"
#include "gemm_mfma_dma.hpp"
#include "gemm_mfma_kreg.hpp"
#include "gemm_mfma_ksplit.hpp"

namespace {

// One v_mfma_f32_32x32x2_f32 of one wave with the operand and result layouts
// the kernels assume: lane l holds A[l % 32][l / 32] and B[l / 32][l % 32];
// result element r of lane l is D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
// A is 32 x 2, B 2 x 32, D 32 x 32, all row-major.
__global__ __launch_bounds__(64) void mfma_layout_probe(const float* A, const float* B, float* D) {
  const int l = threadIdx.x;
  const float a = A[(l % 32) * 2 + l / 32];
  const float b = B[(l / 32) * 32 + l % 32];
  fgr::f32x16 acc = fgr::f32x16{};
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r) D[(8 * (r / 4) + 4 * (l / 32) + r % 4) * 32 + l % 32] = acc[r];
}

}  // namespace

extern "C" {

int shim_xcd_remap(int wg, int nwg) { return fgr::xcd_remap(wg, nwg); }

void shim_grouped_tile(int logical, int tiles_m, int tiles_n, int group, int* tm, int* tn) {
  fgr::grouped_tile(logical, tiles_m, tiles_n, group, *tm, *tn);
}

int shim_a_swizzle(int r) { return fgr::a_swizzle(r); }
int shim_a_swizzle2(int r) { return fgr::a_swizzle2(r); }
int shim_dma_a_col(int pos) { return fgr::dma_a_col(pos); }
int shim_dma_a_read(int row0, int i, int q) { return fgr::dma_a_read(row0, i, q); }
int shim_ksplit_a_col(int pos) { return fgr::ksplit_a_col(pos); }
int shim_ksplit_a_read(int li, int g) { return fgr::ksplit_a_read(li, g); }

void shim_kreg_cols(int k0, int li, int K, int kcb, int* first, int* skip) {
  const fgr::KregCols c = fgr::kreg_cols(k0, li, K, kcb);
  *first = c.first;
  *skip = c.skip;
}

// D = A x B through one MFMA (device pointers; one wave). 0 or a HIP error.
int shim_mfma_probe(const float* A, const float* B, float* D, void* stream) {
  hipLaunchKernelGGL(mfma_layout_probe, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), A, B, D);
  return (int)hipGetLastError();
}

}  // extern "C"
