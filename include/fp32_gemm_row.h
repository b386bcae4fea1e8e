/*
 * fp32_gemm_row.h - C ABI of the MI355X (gfx950) row-major FP32 GEMM library.
 *
 * Operation (the LeetGPU problem of "LeetGPU | 02_Matrix_Multiplication",
 * sections "Problem Description" and "Implementation Requirements", and the
 * CUDA "Approach" there; restated in section 1 of "CUDA 学习笔记 Matrix
 * Multiplication：LeetGPU FP32 矩阵乘法，从逐元素到分块复用"):
 *
 *     C[m,k] = sum over n = 0 .. N-1 of A[m,n] * B[n,k]
 *
 * A is M x N, B is N x K, C is M x K, all dense row-major FP32 with leading
 * dimensions exactly N, K and K: A[m,n] = A[m*N+n], B[n,k] = B[n*K+k],
 * C[m,k] = C[m*K+k]. N is the reduction length. (The tutorial
 * "分块计算与矩阵乘法" swaps the letters for the same product.)
 *
 * Arithmetic is IEEE FP32 throughout (FP32 matrix-core or vector FMA, FP32
 * accumulation, no reduced-precision inputs). The summation order over n is
 * unspecified, so results may differ from a sequential sum in the last bits;
 * where every partial sum is exactly representable (e.g. small integers) the
 * result is exact. The result is |C - exact| <= 1e-5 * sum_n |A[m,n]||B[n,k]|
 * + 1e-6 per element on the tested workloads.
 *
 * Memory and ownership
 *   A, B and C are DEVICE pointers owned by the caller. The library never
 *   synchronises. It keeps a per-device cache of device properties, and some
 *   plans need device memory beyond A, B and C, called workspace here (see
 *   solve() below for sizes and where it comes from): the partial results of
 *   a reduction split across workgroups (paths MFMA_SPLITK, MFMA_KSPLIT_TAIL
 *   and the matrix-vector paths). Nothing else is allocated. C is
 *   overwritten (every one of its M*K
 *   elements is written once; its prior contents, even NaN, are ignored: the
 *   output goes to C, as the LeetGPU problem's "Implementation Requirements"
 *   and the write-back rule of the CUDA study notes, section 3, have it). A
 *   and B are only read and may alias each other; C must not overlap A or B.
 *
 * Streams
 *   `stream` is a hipStream_t passed as void* (NULL = the null stream). Work
 *   is enqueued on it and the call returns without waiting for it. It must
 *   belong to the current device (FGR_ERR_DEVICE otherwise), where A, B and C
 *   must live too. The LeetGPU form below uses the null stream. The library
 *   holds device memory and events (the split workspace, below) for the life
 *   of the process; it must not be called after hipDeviceReset.
 *
 * Alignment and paths
 *   Any 4-byte-aligned pointers are accepted. An operand's rows are "aligned"
 *   below when its row length is a multiple of 4 floats and its pointer is
 *   16-byte aligned; aligned rows move in 16-byte pieces, others in 4-byte or
 *   8-byte ones (the role of the scalar fallback of the LeetGPU write-up,
 *   section "V2: Vectorized float4 Transfers"). With T256, T128 and T64 the
 *   numbers of 256 x 256, 128 x 128 and 64 x 64 output tiles and CUs the
 *   device's compute units, solve() takes the first of these that applies:
 *   1. M <= 4, or M <= 8 without rule 2's shape: the bandwidth-bound
 *      matrix-vector path, which streams B once for all rows of A
 *      (FGR_PATH_GEMV_VEC when B's rows are aligned, else GEMV_SCALAR).
 *   2. 5 <= M <= 64, N >= 64 and K >= 128 (within the 32 x 128 tiles'
 *      offset limits), with B of at least 32 Mi floats, or 16 Mi when 32 x 32
 *      tiles would not fill the CUs: 32 x 128 k-split tiles, their reduction
 *      also split across workgroups where that fills the device
 *      (MFMA_KSPLIT or MFMA_SPLITK, tile 32X128). The same shape with a
 *      smaller B goes on to the rules below, also at M <= 8.
 *   3. T64 >= CUs and a short reduction: N < 104 (N < 72 when every row is
 *      aligned and the 256 x 256 tiles make whole waves), or N < 384 when
 *      T256 >= CUs and B's rows (or, with A's aligned, C's) are not
 *      aligned: register-staged 64 x 64 tiles (MFMA_VEC when all rows are
 *      aligned; else MFMA_SCALAR, tile 128 when T128 >= 4 CUs).
 *   4. T256 >= CUs within FGR_PATH_MFMA_DMA's limits, unless neither A's nor
 *      B's rows are aligned, N >= 768 and the tiles leave a partial last
 *      wave: 256 x 256 tiles whose operands are copied straight from global
 *      memory into LDS (the role of the cp.async pipeline of the write-up's
 *      section "V4"), MFMA_DMA; a partial last wave of at most 11/16 of the
 *      CUs is cut into split-kernel tiles (MFMA_DMA_TAIL).
 *   5. N >= 64: tiles whose reduction is split over the four waves of a
 *      workgroup (k-split). 128 x 128 when K >= 4, T128 >= CUs and they
 *      make whole waves, three waves or more, or a last wave over three
 *      quarters full;
 *      else the strip plan where it applies (MFMA_STRIP); else 64 x 64 when
 *      T64 >= CUs. A partial last wave of at most half the CUs takes
 *      MFMA_KSPLIT_TAIL, else MFMA_KSPLIT. With T64 < CUs: 64 x 64 or
 *      32 x 32 tiles, their reduction also split across workgroups where a
 *      time estimate prefers it (MFMA_SPLITK; 128 x 128 tiles when they pad
 *      no more and their parts are at least 2048 long).
 *   6. Otherwise (N < 64, T64 < CUs): the split kernel's 32 x 32 tiles
 *      (MFMA_SPLIT).
 *   fgr_select_path() and fgr_select_tile() report the choice for a 256-CU
 *   device.
 *
 * Errors
 *   Every entry point returns 0 (FGR_OK) on success or a negative FGR_ERR_*
 *   code. Argument errors are detected on the host before any HIP call, and
 *   nothing is enqueued then. FGR_ERR_LAUNCH reports an error returned by the
 *   kernel launch itself (hipLaunchKernel); errors raised later, while the
 *   kernel runs, surface at the caller's next synchronisation.
 *
 * Limits
 *   The problem statement guarantees 1 <= M, N, K <= 8192 (LeetGPU
 *   "Constraints"); that is the tested range. Larger values are accepted:
 *   index and size arithmetic is 64-bit. Values < 1 are rejected. Some
 *   kernels address their operands with 32-bit byte offsets from a tile's
 *   first row (see FGR_PATH_MFMA_DMA and FGR_PATH_MFMA_KSPLIT); shapes past
 *   those offsets take kernels with 64-bit addresses (solve() chooses them
 *   itself; a forced path that cannot take the shape returns
 *   FGR_ERR_BAD_PATH).
 */
#ifndef FP32_GEMM_ROW_H
#define FP32_GEMM_ROW_H

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define FGR_OK 0
#define FGR_ERR_NULL_POINTER (-1) /* A, B or C is NULL */
#define FGR_ERR_BAD_DIMS (-2)     /* M, N or K < 1 */
#define FGR_ERR_MISALIGNED (-3)   /* a pointer is not 4-byte aligned */
#define FGR_ERR_ALIAS (-4)        /* C overlaps A or B */
#define FGR_ERR_BAD_PATH (-5)     /* forced path/tile cannot run this shape */
#define FGR_ERR_DEVICE (-6)       /* no HIP device, the current one is not gfx950, or the
                                     stream belongs to another device */
#define FGR_ERR_LAUNCH (-7)       /* HIP reported an error at launch */
#define FGR_ERR_SCRATCH (-8)      /* fgr_solve_noalloc: the plan needs more workspace than its
                                     scratch array holds or the workspace limit allows;
                                     nothing was enqueued */

/* Paths (fgr_select_path / fgr_solve_path). */
#define FGR_PATH_AUTO 0
#define FGR_PATH_MFMA_VEC 1    /* FP32 MFMA, 128-bit loads; needs N%4 == K%4 == 0 and 16-B aligned pointers */
#define FGR_PATH_MFMA_SCALAR 2 /* FP32 MFMA, 32-bit loads; any shape and 4-B alignment */
#define FGR_PATH_GEMV_VEC 3    /* matrix-vector and skinny (M <= 8), 128-bit loads of B; needs K%4 == 0
                                  and a 16-B aligned B */
#define FGR_PATH_GEMV_SCALAR 4 /* matrix-vector and skinny (M <= 8), 32-bit loads */
#define FGR_PATH_MFMA_DMA 5    /* FP32 MFMA, 256x256 tiles fed by direct global->LDS copies
                                  (16-byte copies of an operand whose rows are 16-byte aligned,
                                  else 4-byte); needs 64 <= N <= 4194303 and K <= 67108863 (the
                                  copies use 32-bit byte offsets over 256 rows of A and 16 rows
                                  of B); tile 256 only */
#define FGR_PATH_MFMA_SPLIT 6  /* FP32 MFMA, small tiles (32 or 64) whose reduction is split over
                                  the waves of a workgroup; any shape (128-bit loads when the
                                  MFMA_VEC conditions hold, else 32-bit) */
#define FGR_PATH_MFMA_DMA_TAIL 7 /* MFMA_DMA on the whole waves of 256x256 tiles (one per CU), the
                                    split kernel on the tiles of the last, partial wave, cut into
                                    64x64 or 32x32 tiles; same conditions as MFMA_DMA. Two
                                    launches on `stream`. */
#define FGR_PATH_MFMA_KSPLIT 8 /* FP32 MFMA, 128x128, 64x64, 32x32 or 32x128 tiles, each of a
                                  workgroup's four waves reducing a quarter of N into the whole
                                  tile. Operands: 64x64 and 32x32 tiles with 16-byte aligned rows
                                  of A, B and C, and all 32x128 tiles, through direct
                                  global->LDS copies (32x128: 4-byte copies of an operand whose
                                  rows are not 16-byte aligned). The copies use 32-bit byte
                                  offsets over a tile's rows of A and 8 rows of B: 64x64 needs
                                  N <= 16777215, 32x32 and 32x128 N <= 33554431, all K <=
                                  134217727 (past that 64x64 and 32x32 tiles load into
                                  registers; 32x128 is refused). 128x128 tiles and the other
                                  64x64 and 32x32 tiles load operands straight into registers
                                  (16- and 8-byte loads at any 4-byte alignment; 128x128 needs
                                  K >= 4; 64x64 with K = 1 runs as 32x32). N >= 64 */
#define FGR_PATH_MFMA_KSPLIT_TAIL 9 /* MFMA_KSPLIT (tile 128 or 64) on the whole waves of tiles; the
                                       tiles of the last, partial wave either with their reduction
                                       split over workgroups through a workspace (N >= 4096, or
                                       N >= 1024 at tile 64, which then runs in the same grid as
                                       the whole tiles) and a second kernel adding the parts, or
                                       cut into tiles of the split kernel (also when the workspace
                                       cannot be had); two or three launches */
#define FGR_PATH_MFMA_SPLITK 10 /* MFMA_KSPLIT (tile 128, 64 or 32) with each tile's reduction also
                                   split into P parts over P workgroups, which write partial tiles
                                   to a workspace of P*M*K floats; a second kernel adds the parts
                                   in part order into C. For few output tiles and a long N
                                   (N >= 128). P is chosen from the shape; two launches. */
#define FGR_PATH_VALU 11 /* FP32 FMAs on the vector ALUs, no matrix cores: 128x128 tiles, an 8x8
                            register micro-tile per thread, two LDS buffers (128-bit loads when the
                            MFMA_VEC conditions hold, else 32-bit); any shape. A reference for the
                            register-tiled CUDA-core line of the LeetGPU write-up (sections "V1:
                            Two-Dimensional Thread Tiling" to "V3"); never chosen by solve(). Tile
                            AUTO or 128 only. */

#define FGR_PATH_MFMA_STRIP 12 /* K = 64 q + w with 1 <= w <= 8, N >= 64, K > 64: one launch of the
                                  MFMA_KSPLIT kernel whose 64x64 tiles cover columns [0, 64 q),
                                  with workgroups after them that compute C's last w columns
                                  on the vector ALUs (operands as for MFMA_KSPLIT's 64x64
                                  tiles; no workspace). Chosen when those tiles fit one per CU
                                  and the w columns would add a partial second wave of tiles.
                                  Tile AUTO or 64. */

/* Output tile of the MFMA paths (rows x columns of C per workgroup). */
#define FGR_TILE_AUTO 0
#define FGR_TILE_256 256
#define FGR_TILE_128 128
#define FGR_TILE_64 64
#define FGR_TILE_32 32 /* split and k-split paths only */
#define FGR_TILE_32X128 32128 /* 32 rows x 128 columns: k-split paths only (MFMA_KSPLIT, MFMA_SPLITK);
                                 the tile for skinny outputs (M <= 64); N <= 33554431 and
                                 K <= 134217727 (see MFMA_KSPLIT) */

/*
 * solve - C = A x B on `stream`.
 *   A      device pointer, M*N floats, row-major (read only)
 *   B      device pointer, N*K floats, row-major (read only)
 *   C      device pointer, M*K floats, row-major (overwritten)
 *   M,N,K  dimensions, each >= 1; N is the reduction length
 *   stream hipStream_t as void*, NULL for the null stream
 * Returns FGR_OK or an FGR_ERR_* code (see above). Asynchronous.
 * Workspace (device memory beyond A, B and C), by plan:
 *   - a reduction split into P parts across workgroups (MFMA_SPLITK: P*M*K
 *     floats; the matrix-vector paths when their plan splits: P*M*K floats;
 *     the last partial wave of MFMA_KSPLIT_TAIL: P*tiles*tile^2 floats). When
 *     solve() picks the split, P * tiles <= 4 * CUs: on a 256-CU device at most
 *     16 MiB with 64 x 64 or smaller tiles, 64 MiB with 128 x 128 tiles. A
 *     forced MFMA_SPLITK on a large output takes P = 2, i.e. 2*M*K floats.
 *   No other plan takes a workspace.
 * Each stream (up to 16 per process, identified by its handle and device)
 * keeps one split workspace between calls, up to 64 MiB: it is allocated
 * stream-ordered on `stream` at the stream's first split call, replaced (the
 * old one freed with hipFreeAsync on `stream`) when a call needs more, and
 * otherwise held until the process ends; a stream created after another was
 * destroyed may inherit its handle and so its entry, whose buffer it uses only
 * after the old stream's last use of it. Calls from several host threads on one
 * stream are serialised while they enqueue. Every other workspace (more
 * streams, larger workspaces, hipStreamPerThread, or `stream` under capture)
 * is allocated stream-ordered on `stream` for the call and freed
 * with hipFreeAsync after its last kernel. Allocations come from a memory
 * pool the library creates per device on first use (hipMemPoolCreate; it
 * keeps up to 64 MiB of freed memory for reuse and lives until the process
 * ends), or from the device's default pool if that creation failed. If an
 * allocation fails, or would exceed fgr_set_workspace_limit(), the plan runs
 * without that workspace: the unsplit kernel instead of a split, the split
 * kernel for a last partial wave (same result up to rounding order); no error
 * is returned for it. Results are deterministic: the parts are added in a fixed order.
 * solve() can be captured into a HIP graph (stream capture on `stream`); the
 * workspace then becomes a graph allocation.
 * The LeetGPU signature (section "Problem Description", and every "Solution"
 * of the write-up) is solve(A, B, C, M, N, K) returning void; this form adds
 * the stream and a status.
 */
int solve(const float *A, const float *B, float *C, int M, int N, int K, void *stream);

/*
 * fgr_solve_noalloc - solve() for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, plan, kernels, result (bit for bit), layout and
 * asynchrony as solve(); the caller still owns A, B and C. Where solve()'s plan
 * takes a workspace (see solve() above), this call takes it instead from a
 * static device array of 64 MiB (67108864 bytes) that the library holds on
 * each GPU it runs on until the process ends, and it calls no allocating
 * routine (no hipMalloc, hipMallocAsync, hipFree or pool call). If the plan
 * needs more workspace than the array holds, or than fgr_set_workspace_limit()
 * allows, it returns FGR_ERR_SCRATCH and enqueues nothing (on a 256-CU device
 * no plan of solve() needs more than 64 MiB: see the split workspaces above;
 * one with more CUs can). The array keeps what the last call
 * left in it; nothing in it needs to start at zero. All such calls on one GPU
 * share its array: calls that overlap on one GPU (other streams or threads,
 * before the previous one's kernels have finished) race, so the caller must
 * order them (for instance on one stream). Other errors as solve().
 */
int fgr_solve_noalloc(const float *A, const float *B, float *C, int M, int N, int K, void *stream);

/*
 * fgr_solve_default - the six-argument LeetGPU form: solve(A, B, C, M, N, K, NULL).
 */
int fgr_solve_default(const float *A, const float *B, float *C, int M, int N, int K);

/*
 * fgr_solve_path - solve() with the path and output tile forced (for tests and
 * benchmarks; the controlled comparisons of the LeetGPU write-up, section
 * "Controlled Comparison", build each variant separately). path is an
 * FGR_PATH_* value, tile an FGR_TILE_* value (ignored by the GEMV paths).
 * Returns FGR_ERR_BAD_PATH if that path or tile cannot handle these arguments
 * (e.g. a VEC path with N % 4 != 0, a GEMV path with M > 8, the DMA path
 * with a tile other than 256 or N < 64, an unknown value).
 */
int fgr_solve_path(const float *A, const float *B, float *C, int M, int N, int K, void *stream,
                   int path, int tile);

/*
 * fgr_select_path - the FGR_PATH_* value solve() would take for these
 * arguments on a 256-CU device, or a negative FGR_ERR_* code for invalid
 * arguments. Host only: makes no HIP call.
 */
int fgr_select_path(const float *A, const float *B, const float *C, int M, int N, int K);

/*
 * fgr_select_tile - the FGR_TILE_* output tile solve() would use with the path
 * fgr_select_path() reports, on a 256-CU device (FGR_TILE_AUTO for the
 * matrix-vector paths), or a negative FGR_ERR_* code. Host only.
 */
int fgr_select_tile(const float *A, const float *B, const float *C, int M, int N, int K);

/*
 * fgr_select_parts - the number of workgroups each output tile's reduction is
 * split over when fgr_select_path() reports FGR_PATH_MFMA_SPLITK (1 for every
 * other path), on a 256-CU device, or a negative FGR_ERR_* code. Powers of
 * two, or the counts that fill whole rounds of the CUs (k CUs / tiles, k = 1
 * .. 4), whichever the time estimate prefers. Host only.
 */
int fgr_select_parts(const float *A, const float *B, const float *C, int M, int N, int K);

/* fgr_status_string - a static, human-readable name for a status code. */
const char *fgr_status_string(int status);

/* fgr_version - library version as MAJOR*10000 + MINOR*100 + PATCH. */
int fgr_version(void);

/*
 * fgr_set_workspace_limit - the largest workspace, in bytes, that one request
 * of a call may take from now on (process-wide; negative: no limit, the
 * default). A plan of solve() whose workspace would exceed it runs without
 * that workspace, as when an allocation fails (see solve()); fgr_solve_noalloc
 * refuses such a plan with FGR_ERR_SCRATCH. For callers short of device
 * memory, and for tests of those forms (a limit of 0 takes every one of
 * them). Returns the previous limit. Host only; calls already enqueued are not
 * affected.
 */
long long fgr_set_workspace_limit(long long bytes);

/*
 * fgr_stream_read - a measurement hook, not part of the product: reads every
 * float of X (n floats, device memory, 16-byte aligned, n a multiple of 4,
 * n >= 4) once with 128-bit loads on `blocks` workgroups of 256 threads
 * (grid-stride), and writes each workgroup's sum to out[0 .. blocks-1]
 * (device memory, caller-owned, overwritten; must not overlap X). Timed over a
 * buffer several times the last-level cache, it gives the device's practical
 * streaming-read rate, the ceiling the matrix-vector path is judged against
 * beside the datasheet's HBM peak (the byte bound of the study notes "CUDA 学习笔记
 * Matrix Multiplication", section 2). Errors as solve(): FGR_ERR_NULL_POINTER,
 * FGR_ERR_BAD_DIMS (n or blocks out of range), FGR_ERR_MISALIGNED,
 * FGR_ERR_ALIAS, FGR_ERR_DEVICE, FGR_ERR_LAUNCH. Asynchronous; allocates
 * nothing.
 */
int fgr_stream_read(const float *X, long long n, float *out, int blocks, void *stream);

/*
 * The controlled comparison (the LeetGPU write-up, section "Controlled
 * Comparison": one variable changed at a time, every variant built and timed
 * alike, with the compiler's resource report beside it). The library holds a
 * fixed list of kernel variants along three axes: LDS buffering (the
 * register-staged MFMA kernel with one buffer, or two with register
 * prefetch; the direct-copy kernel with rings of 3, 4 or 5 stages), output
 * tile (256x256, 256x128, 128x128) and reduction chunk (16 or 32 deep).
 * None of them is a product path: solve() uses the tuned kernels.
 *
 * fgr_variant_count - the number of variants, V.
 * fgr_variant_name  - a static name for variant 0 <= v < V ("regs double
 *                     256x256 bk32", "direct ring4 256x256 bk16", ...), or
 *                     NULL outside that range.
 * fgr_solve_variant - C = A x B on `stream` with variant v alone, same
 *                     arguments, layout, ownership and asynchrony as solve().
 *                     Returns FGR_ERR_BAD_PATH for v outside [0, V), rows that
 *                     are not 16-byte aligned (N % 4, K % 4 or a pointer), or
 *                     a direct-copy variant with N < 64; the other FGR_ERR_*
 *                     codes as solve(). Host only until the launch; allocates
 *                     nothing.
 */
int fgr_variant_count(void);
const char *fgr_variant_name(int variant);
int fgr_solve_variant(const float *A, const float *B, float *C, int M, int N, int K, void *stream,
                      int variant);

#ifdef __cplusplus
}
#endif

#endif /* FP32_GEMM_ROW_H */
