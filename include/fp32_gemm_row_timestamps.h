/*
 * fp32_gemm_row_timestamps.h - the measurement build's extra entry point.
 *
 * libfp32_gemm_row_ts.so is the library built with FGR_TIMESTAMPS: the same
 * entry points and kernels as libfp32_gemm_row.so (fp32_gemm_row.h), except
 * that the direct-copy, k-split, register-fed k-split and matrix-vector
 * kernels each record one timestamp record per workgroup of their last
 * launch. It is for
 * measurement only (bench.py --timestamps); solve() callers use the plain
 * library, which has none of this.
 *
 * Record i (workgroup i of the last launch of a recording kernel; workgroups
 * from 4096 on are not recorded), eight 64-bit words:
 *   t_start, t_loop, t_end  constant 100 MHz clock (s_memrealtime) at the
 *                           workgroup's start, the end of its main loop, and
 *                           the end of wave 0's stores (after they completed)
 *   c_start, c_loop         the shader clock (s_memtime) at the first two
 *   hw_id                   XCC_ID << 32 | HW_ID (hardware registers: the
 *                           XCD, and the shader engine, CU and SIMD)
 *   kind                    0: a tile's workgroup; 1: another role (the
 *                           column strip of the strip plan)
 *   pad                     0
 * Records of workgroups that a later launch did not reach keep their old
 * contents; launches of other kernels leave them alone.
 */
#ifndef FP32_GEMM_ROW_TIMESTAMPS_H
#define FP32_GEMM_ROW_TIMESTAMPS_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fgr_timestamps_read - copy the first `records` records (1..4096, 64 bytes
 * each) to the host buffer `host`. Synchronous copy on the null stream: call
 * it after synchronising the stream the measured launch ran on. Returns
 * FGR_OK, FGR_ERR_NULL_POINTER (host NULL), FGR_ERR_BAD_DIMS (records out of
 * range) or FGR_ERR_LAUNCH (the copy failed).
 */
int fgr_timestamps_read(void *host, int records);

#ifdef __cplusplus
}
#endif

#endif /* FP32_GEMM_ROW_TIMESTAMPS_H */
