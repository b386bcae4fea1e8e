// Per-workgroup timestamps, for measurement only.
//
// Compiled in only when FGR_TIMESTAMPS is defined (the separate measurement
// build libfp32_gemm_row_ts.so; the library that solve() ships in has none
// of it). A kernel that takes part marks three moments - its start, the end
// of its main loop and its end after its stores have completed - on the
// constant 100 MHz clock (s_memrealtime), and the first two also on the
// shader clock (s_memtime), so that a loop's cycles and the clock it ran at
// both follow. Thread 0 of each workgroup writes one record, indexed by
// workgroup, with the XCD and CU it ran on (hardware registers XCC_ID and
// HW_ID). The records stay in a static device array until the next launch
// overwrites them; fgr_timestamps_read copies them to the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgr {

constexpr int kTsRecords = 4096;  // workgroups recorded per launch (those past it are not)
constexpr int kTsWords = 8;       // 64-bit words per record

struct TsRecord {
  uint64_t t_start, t_loop, t_end;  // 100 MHz clock
  uint64_t c_start, c_loop;         // shader clock
  uint64_t hw_id;                   // XCC_ID << 32 | HW_ID
  uint64_t kind;                    // 0: a tile's workgroup; 1: another role (e.g. a strip)
  uint64_t pad;
};
static_assert(sizeof(TsRecord) == kTsWords * 8, "record size");

#ifdef FGR_TIMESTAMPS
__device__ TsRecord fgr_ts_records[kTsRecords];

struct TsMarks {
  uint64_t t0, c0, t1, c1;
  __device__ __forceinline__ void start() {
    t0 = __builtin_amdgcn_s_memrealtime();
    c0 = __builtin_amdgcn_s_memtime();
  }
  __device__ __forceinline__ void loop_done() {
    t1 = __builtin_amdgcn_s_memrealtime();
    c1 = __builtin_amdgcn_s_memtime();
  }
  // After the workgroup's stores: waits for them, then thread 0 writes the record.
  __device__ __forceinline__ void finish(int kind = 0) {
    __builtin_amdgcn_s_waitcnt(0);
    const uint64_t t2 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0 && blockIdx.x < (unsigned)kTsRecords) {
      // HW_ID (register 4) and XCC_ID (register 20), whole registers
      const uint32_t hw = __builtin_amdgcn_s_getreg(4 | (31 << 11));
      const uint32_t xcc = __builtin_amdgcn_s_getreg(20 | (15 << 11));
      TsRecord r;
      r.t_start = t0;
      r.t_loop = t1;
      r.t_end = t2;
      r.c_start = c0;
      r.c_loop = c1;
      r.hw_id = ((uint64_t)xcc << 32) | hw;
      r.kind = (uint64_t)kind;
      r.pad = 0;
      fgr_ts_records[blockIdx.x] = r;
    }
  }
};
#else
struct TsMarks {
  __device__ __forceinline__ void start() {}
  __device__ __forceinline__ void loop_done() {}
  __device__ __forceinline__ void finish(int = 0) {}
};
#endif

}  // namespace fgr
