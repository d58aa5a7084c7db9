// internal.h -- shared between the host dispatcher and the HIP kernels of
// the CSR sparse x dense product library.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdl {

constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kWavesPerBlock = 4;    // worker block = 256 threads
constexpr int kBlock = kWave * kWavesPerBlock;
constexpr int kPlanBlock = 256;      // planning kernels: threads per block
constexpr int kPlanMaxTiles = 2048;  // planning tiles per call (upper bound)
constexpr int64_t kChunkTableSlack = 4096;  // chunk table holds M + this
// Entries of one short tile staged per wavefront; short_max is capped at
// kShortCap / R (R = row groups per wavefront) so that a tile of at least R
// rows always fits.
constexpr int kShortCap = 512;

// Routing thresholds, already resolved (see spmm_tuning_t).
struct Thresholds {
    int32_t short_max;
    int32_t medium_max;
    int32_t chunk_nnz;
};

// Per long row: the row, the index of its first chunk, its chunk count.
struct LongRow {
    int32_t row;
    int32_t first_chunk;
    int32_t n_chunks;
};

// One nnz chunk of a long row: positions [p0, p1) of row `row`, which is
// entry `long_idx` of the long-row list.
struct Chunk {
    int32_t row;
    int32_t p0;
    int32_t p1;
    int32_t long_idx;
};

// Totals the planning pass leaves on the device for the worker.
struct PlanCounts {
    int32_t n_medium;
    int32_t n_long;
    int32_t n_chunks;
    int32_t n_short;
};

// Device pointers into one call's scratch space.
struct PlanBuffers {
    int32_t *tile_counts;   // [n_tiles * 4]: medium, long, chunks, short
    PlanCounts *counts;     // [1]
    int32_t *medium_rows;   // [M]
    LongRow *long_rows;     // [M]
    Chunk *chunks;          // [chunk_cap]
    int64_t chunk_cap;
};

// Shape of the planning pass over M rows: n_tiles blocks of tile_rows rows.
struct PlanShape {
    int64_t tile_rows;
    int64_t n_tiles;
};

PlanShape plan_shape(int64_t M);

// Enqueue the two planning kernels.  When zero_long_rows is set, the C rows
// of long rows (leading dimension N) are cleared for atomic accumulation.
// start/stop (may be null) are attached to the first and last kernel.
hipError_t launch_plan(const int32_t *rowptr, int64_t M, Thresholds th,
                       const PlanBuffers &buf, float *C, int64_t N,
                       hipStream_t stream, hipEvent_t start, hipEvent_t stop);

// Enqueue a kernel that writes chunk descriptors 0..count-1 (table entry or
// recomputed) to out; used only by the plan export.
hipError_t launch_chunk_expand(const int32_t *rowptr, Thresholds th,
                               const PlanBuffers &buf, int64_t count,
                               Chunk *out, hipStream_t stream);

// Worker configuration picked by the host for one call.
struct WorkerConfig {
    int dtype;     // SPMM_DTYPE_*
    int vec;       // elements of B per lane load
    int group;     // lanes per row group (G); R = 64 / G groups per wave
    int nv;        // vectors per lane per B row (columns per pass = G*vec*nv)
};

WorkerConfig choose_worker(int dtype, int64_t N, const void *B, const float *C);

struct WorkerArgs {
    const int32_t *rowptr;
    const int32_t *colind;
    const void *vals;
    const void *B;
    float *C;
    int64_t M;
    int64_t K;
    int64_t N;
    Thresholds th;
    PlanBuffers plan;
};

// start/stop (may be null) time the worker kernel.
hipError_t launch_worker(const WorkerConfig &cfg, const WorkerArgs &args,
                         hipStream_t stream, hipEvent_t start, hipEvent_t stop);

}  // namespace sdl

namespace sdl {

// Bounds of chunk k of a long row that starts at `start`, holds `len`
// entries and is cut into n chunks: positions
// [start + floor(k*len/n), start + floor((k+1)*len/n)).  The chunks tile the
// row in order and differ in size by at most one entry.
__host__ __device__ inline void chunk_bounds(int64_t start, int64_t len,
                                             int64_t n, int64_t k,
                                             int32_t *p0, int32_t *p1)
{
    *p0 = (int32_t)(start + (k * len) / n);
    *p1 = (int32_t)(start + ((k + 1) * len) / n);
}

// Descriptor of chunk c: the table entry when c is inside the table,
// otherwise recomputed from the long-row list (binary search for the last
// long row whose first chunk is <= c) and rowptr.
__device__ inline Chunk resolve_chunk(int64_t c, const PlanBuffers &pb,
                                      int32_t n_long, const int32_t *rowptr)
{
    if (c < pb.chunk_cap)
        return pb.chunks[c];
    int32_t lo = 0, hi = n_long - 1;
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (pb.long_rows[mid].first_chunk <= c)
            lo = mid;
        else
            hi = mid - 1;
    }
    const LongRow lr = pb.long_rows[lo];
    const int64_t start = rowptr[lr.row];
    const int64_t len = (int64_t)rowptr[lr.row + 1] - start;
    Chunk ch;
    ch.row = lr.row;
    ch.long_idx = lo;
    chunk_bounds(start, len, lr.n_chunks, c - lr.first_chunk, &ch.p0, &ch.p1);
    return ch;
}

}  // namespace sdl
