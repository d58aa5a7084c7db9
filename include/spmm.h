/*
 * spmm.h -- C ABI of the MI355X (gfx950) CSR sparse x dense product library.
 *
 * Operation (page "Performance Optimization of Deep Learning Sparse Matrix
 * Kernels on Intel Max Series GPU", the SpMM operation, Fig. 5 and
 * Algorithm 2): given a sparse M x K matrix A in CSR form and a dense K x N
 * matrix B, compute the dense M x N matrix
 *
 *     C[i, :] = sum over stored entries p of row i of  vals[p] * B[colind[p], :]
 *
 * i.e. every stored value scales one gathered row of B and is accumulated
 * into its output row.  C is overwritten (it is computed, not updated):
 * rows of A with no stored entries produce rows of +0.0.  Stored entries
 * with the same column are all visited, so they add up.
 *
 * Layout
 *   rowptr  int32[M+1]   absolute offsets into colind/vals; row i owns
 *                        positions rowptr[i] .. rowptr[i+1]-1.  rowptr[0]
 *                        may be non-zero, so a caller can pass a view of a
 *                        block of rows (rowptr + r0, C + r0*N) without copies.
 *   colind  int32[nnz]   column indices, 0 <= colind[p] < K; any order and
 *                        repeats are allowed.
 *   vals    [nnz]        float32, or bf16 bit patterns (uint16).
 *   B       K x N        row-major, leading dimension exactly N.
 *   C       M x N        float32, row-major, leading dimension exactly N.
 *
 * Ownership and memory: every pointer is device memory owned by the caller;
 * the library never frees or retains it.  The library allocates its own
 * scratch space (the row plan) from a stream-ordered pool per device, so
 * calls on different streams do not share scratch.  It keeps one scratch
 * block (and, for FusedMM's two-launch route and the element-balanced
 * kernel, one work buffer) per (device, stream handle) it has been called
 * on, grown when a call needs more, until spmm_stream_release is called on
 * that stream or the process ends.  The blocks are keyed by the handle's
 * value: a stream that is destroyed while the library still holds blocks
 * for it leaves them to whatever stream later receives the same handle,
 * possibly while the destroyed stream's last calls are still running.  Call
 * spmm_stream_release(stream) before hipStreamDestroy(stream).
 *
 * Asynchrony: a call only enqueues work on `stream` (a hipStream_t; NULL is
 * the null stream) and returns; it never waits for the device.  Inputs must
 * stay alive, and C must not be read, until the stream has passed the call.
 *
 * Threads: calls may come from several host threads at once, on one stream
 * or on several.  A call holds a per-(device, stream) lock from the moment
 * it takes its share of the stream's scratch until its launches are
 * enqueued, so calls on one stream reach the device one after another in
 * the order they took the lock (the order of calls made from different
 * threads at once is not otherwise defined).  Calls on different streams
 * may run on the device at the same time: each stream has its own scratch.
 *
 * Errors: every call returns a status; nothing throws across the ABI.
 * Argument errors are found on the host before any HIP call.  The contents
 * of the CSR arrays are preconditions that the fast path does not check:
 * rowptr must be non-decreasing, 0 <= colind < K, and
 * rowptr[M] - rowptr[0] < 2^31.  spmm_last_error() gives a text for the most
 * recent failure on the calling thread.
 *
 * Numerics: products and sums are carried in fp32 with fused multiply-adds,
 * in an order that differs from the sequential one.  bf16 inputs: the
 * products of two bf16 values are exact in fp32; rows taken by a whole
 * wavefront (medium rows, chunks of long rows) add two entries' products
 * per column with one bf16 dot-product instruction into the fp32
 * accumulator (its rounding error stays within that of two fp32
 * multiply-adds plus a quarter), other rows widen each element exactly and
 * use fused multiply-adds.  Infinities and NaN in B or vals reach exactly
 * the elements of C that IEEE arithmetic sends them to.  Rows handled by
 * one wavefront are bitwise repeatable from run to run; rows long enough
 * to be split across wavefronts are reduced with fp32 atomic adds, whose
 * order (and so the last bits) can differ between runs.
 */
#ifndef SDL_SPMM_H
#define SDL_SPMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t spmm_status_t;

#define SPMM_SUCCESS             0  /* work enqueued (or nothing to do)            */
#define SPMM_ERROR_INVALID_VALUE 1  /* bad size, null pointer, bad option          */
#define SPMM_ERROR_HIP           2  /* a HIP runtime call or a launch failed       */
#define SPMM_ERROR_OUT_OF_MEMORY 3  /* the scratch space could not be allocated   */
#define SPMM_ERROR_UNSUPPORTED   4  /* valid request this build does not serve    */

#define SPMM_DTYPE_F32  0           /* vals and B are float32                    */
#define SPMM_DTYPE_BF16 1           /* vals and B are bf16 bits, fp32 accumulate */

/*
 * Row-binning thresholds (the plan).  A row with len = rowptr[i+1]-rowptr[i]
 * entries is
 *   short   if len <= short_max          one sub-wavefront lane group per row
 *   medium  if short_max < len <= medium_max   one wavefront per row
 *   long    if medium_max < len <= H     cut into ceil(len / chunk_nnz)
 *                                        near-equal chunks, one wavefront each
 *   hub     if len > H                   cut at column-slab boundaries: chunk
 *                                        s holds the entries with columns in
 *                                        [s*slab_rows, (s+1)*slab_rows) (for
 *                                        ascending columns), one wavefront each
 * with H = max(hub_min, medium_max).  Hub chunks of neighbouring slabs run on
 * the same XCD, slab after slab, so the slab's rows of B are gathered from
 * that XCD's L2 by every hub row that has entries in it ([Multilevel] "Sparse
 * Matrix-Matrix Multiplication on Multilevel Memory Architectures", the
 * access-pattern analysis: row j of B is read once per non-zero in column j).
 * Fields < 0 (short_max, medium_max, hub_min) or <= 0 (chunk_nnz, slab_rows)
 * ask for the library's default for the given element type, K and N: hub
 * rows only when B holds at least 256 MiB (more than the Infinity Cache),
 * slabs of 2 MiB of B's rows, and H at least 32 entries per slab.
 * hub_min = INT32_MAX turns hub rows off.
 * The thresholds never change C beyond rounding; they only route work.
 */
typedef struct spmm_tuning {
    int32_t short_max;
    int32_t medium_max;
    int32_t chunk_nnz;
    int32_t hub_min;
    int32_t slab_rows;
    int32_t reserved;   /* must be 0 */
} spmm_tuning_t;

/*
 * C = A * B with fp32 values and fp32 B, fp32 accumulation, fp32 C.
 * M, K, N >= 0; M, K < 2^31.  M == 0 or N == 0: success, nothing launched.
 * K == 0 requires an A with no stored entries (C becomes zero).
 * Null pointers are rejected when the array they stand for is non-empty.
 */
spmm_status_t spmm_csr_f32(const int32_t *rowptr, const int32_t *colind,
                           const float *vals, const float *B, float *C,
                           int64_t M, int64_t K, int64_t N, void *stream);

/*
 * C = A * B with bf16 values and bf16 B (given as raw 16-bit patterns),
 * widened exactly to fp32, fp32 accumulation, fp32 C.  Same rules as
 * spmm_csr_f32.
 */
spmm_status_t spmm_csr_bf16in_f32acc(const int32_t *rowptr,
                                     const int32_t *colind,
                                     const uint16_t *vals, const uint16_t *B,
                                     float *C, int64_t M, int64_t K,
                                     int64_t N, void *stream);

/*
 * Either element type (dtype = SPMM_DTYPE_*) with explicit thresholds;
 * tuning == NULL means all defaults.  Same rules as spmm_csr_f32, and a
 * tuning with short_max > medium_max (after defaults) or reserved != 0 is
 * SPMM_ERROR_INVALID_VALUE.
 */
spmm_status_t spmm_csr_tuned(int32_t dtype, const int32_t *rowptr,
                             const int32_t *colind, const void *vals,
                             const void *B, float *C, int64_t M, int64_t K,
                             int64_t N, const spmm_tuning_t *tuning,
                             void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * product of spmm_csr_tuned -- same arguments, checks, thresholds, kernel
 * and results -- with its plan scratch in a fixed array that the library
 * holds on each GPU it runs on, instead of a per-stream block from a pool.
 * This entry point calls no hipMalloc, hipFree or other allocating routine
 * (and allocates nothing on the host).
 *
 * Limit: the fixed array holds 12 MiB, enough for the plan of M up to
 * 311,000 rows (about 40 bytes per row); a larger M returns
 * SPMM_ERROR_UNSUPPORTED, found on the host before any HIP call, with the
 * exact limit in spmm_last_error().
 *
 * Every call of this entry point on one GPU uses that GPU's single array,
 * which keeps the last call's contents (plan words tagged with a per-GPU
 * call counter, so nothing needs clearing).  Calls are enqueued one at a
 * time (a per-GPU lock), but calls that overlap on the device -- e.g. made
 * on two streams of one GPU without ordering between them -- race on the
 * array and give wrong results: order them on one stream or with events.
 * The fault count of these calls is kept in the array and reported by
 * spmm_stream_faults (on the stream the calls used).
 */
spmm_status_t spmm_csr_tuned_noalloc(int32_t dtype, const int32_t *rowptr,
                                     const int32_t *colind, const void *vals,
                                     const void *B, float *C, int64_t M,
                                     int64_t K, int64_t N,
                                     const spmm_tuning_t *tuning, void *stream);

/*
 * Host only, no HIP call: the thresholds a call with this dtype, K, N and
 * requested tuning (NULL = all defaults) would use, written to *resolved.
 */
spmm_status_t spmm_resolve_tuning(int32_t dtype, int64_t K, int64_t N,
                                  const spmm_tuning_t *requested,
                                  spmm_tuning_t *resolved);

/*
 * Introspection for tests: run only the planning pass on device rowptr
 * (M rows; colind of K columns for the hub chunks) with the given resolved
 * thresholds, wait for it, and copy the plan to host arrays:
 *   counts[6]          n_short, n_medium, n_long, n_chunks, n_hub,
 *                      n_hub_chunks (= n_hub * ceil(K / slab_rows))
 *   medium_rows[cap]   ascending rows with short_max < len <= medium_max
 *   long_rows[3*cap]   per long row, ascending: row, first chunk, chunks
 *   chunks[4*cap]      per chunk, ordered by row then position:
 *                      row, first position, end position, long-row index
 *   hub_rows[cap]      ascending hub rows
 *   hub_chunks[4*cap]  per hub chunk, slab-major (slab s of hub h at
 *                      s * n_hub + h): row, first position, end position,
 *                      hub index; the bounds come from the product's own
 *                      search over colind
 * Each output array receives at most `cap` records (counts are always
 * complete).  Synchronises `stream`.  The chunk table the worker reads
 * holds M + 4096 records; chunks beyond it are recomputed from long_rows,
 * and this call reports the recomputed values for them as well.  colind
 * may be NULL only when hub_min is INT32_MAX (no hub rows).
 */
spmm_status_t spmm_plan_export(const int32_t *rowptr, const int32_t *colind,
                               int64_t M, int64_t K,
                               const spmm_tuning_t *resolved, void *stream,
                               int64_t cap, int64_t *counts,
                               int32_t *medium_rows, int32_t *long_rows,
                               int32_t *chunks, int32_t *hub_rows,
                               int32_t *hub_chunks);

/* Static text naming a status code. */
const char *spmm_status_string(spmm_status_t status);

/* Text describing the most recent failure on the calling thread ("" if
 * none).  Valid until the next library call on this thread. */
const char *spmm_last_error(void);

/*
 * Kernel timing for benchmarks.  spmm_timing_enable(1) makes every later
 * call attach HIP events to the start and the end of its launch (a call is
 * one launch: the plan runs in its first workgroups), so timing adds no
 * packets to the stream.  spmm_timing_read waits for the recorded events
 * and returns, in *worker_ms, the summed milliseconds of the timed calls
 * and, in *calls, their number, then clears the record; *plan_ms is always
 * 0 (the plan is inside the launch).  Disabled by default.
 */
spmm_status_t spmm_timing_enable(int32_t on);
spmm_status_t spmm_timing_read(double *plan_ms, double *worker_ms,
                               int64_t *calls);

/*
 * The same product C = A * B (either element type), computed by the
 * element-balanced kernel instead of the row plan: [Sgap] "Sgap: Towards
 * Efficient Sparse Tensor Algebra Compilation for GPU", the element-balanced
 * points of atomic parallelism and the grouped segmented reduction.  One
 * launch.  The stored entries are split into equal spans, one per
 * wavefront; partial sums of entries that share a row are combined across
 * lane groups in entry order.  A row cut by a span end is finished inside
 * the same launch: each wavefront that holds part of it writes its partial
 * row to a carry slot and then arrives on the row's counter (a
 * compare-and-swap on a word tagged with the call's epoch); the arrival that
 * completes the count adds the row's slots in span order and stores the
 * row.  No atomic adds touch C and the summation order is fixed, so results
 * repeat bit for bit.  Arguments, layout, ownership and errors as for
 * spmm_csr_tuned (dtype is SPMM_DTYPE_F32 or SPMM_DTYPE_BF16).  The carry
 * slots (2 rows of N floats per wavefront of the GPU) live in the stream's
 * work buffer, the arrival counters in the stream's plan scratch; the call
 * takes one epoch of that scratch like a product call.
 */
spmm_status_t spmm_csr_eb(int32_t dtype, const int32_t *rowptr,
                          const int32_t *colind, const void *vals,
                          const void *B, float *C, int64_t M, int64_t K,
                          int64_t N, void *stream);

/*
 * Sampled dense-dense product (SDDMM) on the pattern of a CSR matrix.
 * [IntelMax] "Performance Optimization of Deep Learning Sparse Matrix
 * Kernels on Intel Max Series GPU", the SDDMM operation (Fig. 3, Algorithm
 * 1): the stored entry p of row i, at column j = colind[p], gets the dot
 * product of row i of C with column j of B^T (row j of B):
 *
 *     A[p - rowptr[0]] = sum over n < N of C[i*N + n] * B[j*N + n]
 *
 *   rowptr  int32[M+1]  as for the product (absolute offsets; a view works)
 *   colind  int32[nnz]  0 <= colind[p] < K
 *   C       M x N       row-major, float32 (or bf16 bits for the bf16 entry)
 *   B       K x N       row-major, same element type as C
 *   A       float32[nnz] output, one value per stored entry in CSR order;
 *                       it is overwritten (not scaled by earlier values)
 *   nnz     rowptr[M] - rowptr[0], the length of A (a precondition, as are
 *           the other CSR invariants)
 *
 * Ownership, asynchrony and errors as for the product.  nnz == 0 returns
 * at once; N == 0 with stored entries is UNSUPPORTED.  Numerics: products
 * and sums in fp32, in an order that differs from the sequential one: fp32
 * operands with fused multiply-adds; bf16 operands (N a multiple of 8) by
 * bf16 dot-product instructions over pairs of neighbouring columns (exact
 * products, fp32 sums), other bf16 widths widened exactly.  Every value is
 * computed by one wavefront, so results repeat bit for bit.
 */
spmm_status_t sddmm_csr_f32(const int32_t *rowptr, const int32_t *colind,
                            const float *C, const float *B, float *A,
                            int64_t M, int64_t K, int64_t N, int64_t nnz,
                            void *stream);
spmm_status_t sddmm_csr_bf16in_f32acc(const int32_t *rowptr,
                                      const int32_t *colind, const uint16_t *C,
                                      const uint16_t *B, float *A, int64_t M,
                                      int64_t K, int64_t N, int64_t nnz,
                                      void *stream);

/*
 * FusedMM on the pattern of a CSR matrix.  [IntelMax], the FusedMM
 * operation (Fig. 6, Algorithm 3): the SDDMM value of each stored entry
 * (row C_i times row B_j, as for sddmm_csr_f32) weights row D_j of a third
 * dense matrix, summed per row:
 *
 *     E[i*N + n] = sum over p in row i of <C_i, B_colind[p]> * D[colind[p]*N + n]
 *
 *   C  M x N, B and D  K x N, E  M x N; all float32, row-major, leading
 *   dimension exactly N (D has the N columns of C and B).
 *   nnz = rowptr[M] - rowptr[0] (a precondition; on the two-launch route
 *   below, a smaller nnz makes the product refuse to run, on the device,
 *   and count a fault for spmm_stream_faults instead of reading past the
 *   value array).
 * E is overwritten; rows with no stored entries become zero rows.
 *
 * One launch on `stream` when N is a multiple of 4 and at most 1024, C, B,
 * D and E are 16-byte aligned, and either N <= 64 or nnz >= 32 * M (rows
 * of 32 entries or more on average): the product's kernel (same plan, same
 * per-stream scratch) forms each entry's value from C_i and B_j where the
 * value is used, and no value array is written.  Otherwise two launches:
 * the SDDMM values are written to a scratch array of nnz floats (kept per
 * stream by the library, from its stream-ordered pool, grown when a call
 * needs more), and the product reads them as the values of A with D as its
 * dense operand.  Errors and ownership as for the product;
 * SPMM_ERROR_OUT_OF_MEMORY if the scratch array cannot be had.
 * Numerics: each value is rounded to fp32 before it weights D_j; both
 * routes form it in the same order when they use the same lane-group width.
 */
spmm_status_t fusedmm_csr_f32(const int32_t *rowptr, const int32_t *colind,
                              const float *C, const float *B, const float *D,
                              float *E, int64_t M, int64_t K, int64_t N,
                              int64_t nnz, void *stream);

/*
 * FusedMM as fusedmm_csr_f32 with C, B and D given as bf16 bit patterns
 * (uint16), widened exactly to fp32; each value <C_i, B_j> is formed and
 * used in fp32, the sums are fp32, and E is fp32.  One launch when N is a
 * multiple of 8 and at most 1024 and C, B, D and E are 16-byte aligned.
 * Otherwise C, B and D are first widened into an fp32 copy of (M + 2K) * N
 * floats, taken from the library's stream-ordered pool and given back on
 * `stream` once the call's launches are enqueued, and fusedmm_csr_f32 runs
 * on the copy (same values: bf16 products are exact in fp32);
 * SPMM_ERROR_OUT_OF_MEMORY if the copy cannot be had or would pass 2^56
 * bytes (found before any HIP call).  C, B and D need
 * 2-byte alignment, E 4-byte.  nnz == 0: E becomes zero.  Other errors and
 * ownership as for the product.
 */
spmm_status_t fusedmm_csr_bf16in_f32acc(const int32_t *rowptr,
                                        const int32_t *colind, const uint16_t *C,
                                        const uint16_t *B, const uint16_t *D,
                                        float *E, int64_t M, int64_t K,
                                        int64_t N, int64_t nnz, void *stream);

/*
 * Health check.  Inside a call, product wavefronts poll for the plan
 * entries they need while the plan workgroups of the same launch write
 * them; each poll is bounded (about a second), and an item whose entry
 * never became visible is left undone and counted.  spmm_stream_faults
 * waits for `stream` and returns in *faults the number of such items in the
 * calls on `stream` since the last query, plus those of the no-allocation
 * calls on the current device since the last query (read in the order of
 * `stream`).  The device only adds to the counts (they carry over when the
 * stream's scratch grows; spmm_stream_release starts a new one), so an item
 * counted while a query runs is reported by the next query, not lost.  A
 * non-zero count means that the outputs of the calls since the last query
 * are not valid.  The
 * count is 0 unless the plan workgroups were kept from running for that
 * long, which can only happen when other kernels running at the same time
 * (calls on other streams, or other libraries) hold the GPU's slots;
 * callers that run concurrent kernels and need a guarantee should check it
 * (the smoke check and the tests do after every call).
 */
spmm_status_t spmm_stream_faults(void *stream, int64_t *faults);

/*
 * Test hook for the path above: the calls enqueued after it poll at most
 * `polls` times for each plan entry (0: they give up at once, so every
 * item that needs the plan is left undone and counted, while every kernel
 * still runs to its end).  polls < 0 restores the default bound (about a
 * second); polls above the default is SPMM_ERROR_INVALID_VALUE.  Process-
 * wide; not for production use.
 */
spmm_status_t spmm_debug_set_wait_polls(int64_t polls);

/*
 * Give back the scratch block and the work buffer the library keeps for
 * `stream` on the current device: both are freed in stream order after
 * the calls already enqueued on it, and the stream is then synchronised,
 * so the caller may destroy the stream afterwards.  A later call on the
 * same handle allocates fresh blocks.  No other call on this stream may be
 * in progress in another thread.  Success (and nothing done) if the
 * library holds nothing for the stream.
 */
spmm_status_t spmm_stream_release(void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SDL_SPMM_H */
