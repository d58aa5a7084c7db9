// internal.h -- shared between the host dispatcher and the HIP kernels of
// the CSR sparse x dense product library.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdl {

// Exclusive prefix sum over the 64 lanes of a wavefront (lane l gets the sum
// of lanes 0 .. l-1), by DPP moves, which need no lane-address registers:
// shifts right by 1, 2, 4, 8 within each row of 16 lanes (lanes with no
// source add 0), then lane 15 of rows 0 and 2 into rows 1 and 3, then lane
// 31 into rows 2 and 3.  Called by all 64 lanes.
__device__ inline int wave_exclusive_sum(int v)
{
    int x = v;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x - v;
}

constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kWavesPerBlock = 4;    // worker block = 256 threads
constexpr int kBlock = kWave * kWavesPerBlock;
constexpr int kPlanLaneRows = 4;     // plan rows per lane per round
constexpr int kPlanRoundRows = kWave * kPlanLaneRows;  // rows per plan round
constexpr int kPlanMaxTiles = 1024;  // plan tiles per call (upper bound)
constexpr int kPlanBlockWaves = kWavesPerBlock;  // plan tiles per plan workgroup
constexpr int kPlanMaxBlocks = kPlanMaxTiles / kPlanBlockWaves;
constexpr int kPlanPrefixLoads = kPlanMaxBlocks / kWave;  // earlier blocks per lane
static_assert(kPlanMaxBlocks % kWave == 0, "plan blocks are read a wavefront at a time");
constexpr int64_t kChunkTableSlack = 4096;
// Polls of a product wavefront for a plan entry before it gives up on the
// item (about a second); spmm_debug_set_wait_polls lowers it for tests.
constexpr int32_t kWaitPolls = 1 << 19;  // chunk table holds M + this
// Work queues of the product: kQueues grab counters per call, kQueueStride
// 32-bit words apart (256 bytes, so they sit in different memory channels).
constexpr int kQueues = 64;
// B is read through a buffer resource (32-bit byte offsets, record count =
// B's size in bytes) when it holds at most this many bytes; a gather slot
// with no entry then loads from kNoRowOffset, past the record count, and
// reads zeros.
constexpr uint32_t kNoRowOffset = 0xFFFFFFF0u;
constexpr uint64_t kBufMaxBytes = kNoRowOffset;
constexpr int kQueueStride = 64;
// Entries of one short tile staged per wavefront; short_max is capped at
// kShortCap / R (R = row groups per wavefront) so that a tile of at least R
// rows always fits.
constexpr int kShortCap = 512;

// Routing thresholds, already resolved (see spmm_tuning_t).  Rows with
// more than hub_top entries are hub rows (hub_top >= medium_max; INT32_MAX:
// none), cut into n_slabs chunks at multiples of slab_rows columns.
struct Thresholds {
    int32_t short_max;
    int32_t medium_max;
    int32_t chunk_nnz;
    int32_t hub_top;     // max(hub_min, medium_max)
    int32_t slab_rows;   // rows of B per column slab (>= 1)
    int32_t n_slabs;     // ceil(K / slab_rows) (0 when K == 0)
};

// Shape of the plan over M rows: n_tiles wavefront tiles of tile_rows rows
// (a multiple of kPlanRoundRows).
struct PlanShape {
    int64_t tile_rows;
    int64_t n_tiles;
};

PlanShape plan_shape(int64_t M);

// The plan lives in scratch memory that is kept per stream and reused by
// every call on it.  Each word the plan publishes is tagged with the call's
// epoch (upper 32 bits; the value in the lower 32), written and read with
// device-coherent relaxed atomics; a reader polls until the tag equals the
// current epoch.  Epochs start at 1 and grow by one per call, and the
// scratch is zeroed when it is created, so no word needs clearing between
// calls.
struct PlanBuffers {
    uint64_t *counts;        // [5] n_medium, n_long, n_chunks, n_short, n_hub
    uint64_t *agg;           // [4][kPlanMaxBlocks] per plan block: medium, long,
                             // chunks, hubs
    uint64_t *medium_rows;   // [M] rows with short_max < len <= medium_max
    uint64_t *long_row;      // [M] long rows, ascending, from the front; hub
                             // row l (ascending) at long_row[M - 1 - l] (the
                             // two lists together hold at most M rows)
    uint64_t *long_first;    // [M] index of each long row's first chunk
    uint64_t *chunk_row;     // [chunk_cap] row of each chunk
    uint64_t *chunk_k;       // [chunk_cap] position of the chunk in its row
    uint32_t *faults;        // items the product gave up waiting for (not tagged)
    uint32_t *queues;        // [2][kQueues * kQueueStride] grab counters: a
                             // product call uses set epoch & 1; every call that
                             // takes an epoch (product or element-balanced)
                             // clears set (epoch + 1) & 1 (not tagged)
    int64_t chunk_cap;       // M + kChunkTableSlack
    int64_t rows;            // M: hub row l is long_row[rows - 1 - l]
};

constexpr int kPlanCounts = 4;   // per plan block: medium, long, chunks, hubs

// Bounds of chunk k of a long row that starts at `start`, holds `len`
// entries and is cut into n chunks: positions
// [start + floor(k*len/n), start + floor((k+1)*len/n)).  The chunks tile the
// row in order and differ in size by at most one entry.
__host__ __device__ inline void chunk_bounds(int64_t start, int64_t len,
                                             int64_t n, int64_t k,
                                             int64_t *p0, int64_t *p1)
{
    *p0 = start + (k * len) / n;
    *p1 = start + ((k + 1) * len) / n;
}

// Worker configuration picked by the host for one call.
struct WorkerConfig {
    int dtype;     // SPMM_DTYPE_*
    int vec;       // elements of B per lane load
    int group;     // lanes per row group (G); R = 64 / G groups per wavefront
    int nv;        // vectors per lane per B row (columns per pass = G*vec*nv)
};

WorkerConfig choose_worker(int dtype, int64_t N, const void *B, const float *C);

// Whether the FusedMM form of the worker covers cfg and N: 16-byte vectors
// (4 fp32 or 8 bf16 elements) and a whole row of N <= 1024 columns in one
// column pass.
bool fused_fits(const WorkerConfig &cfg, int64_t N);

struct WorkerArgs {
    const int32_t *rowptr;
    const int32_t *colind;
    const void *vals;      // value of entry p at vals[p] (or vals[p - rowptr[0]])
    int32_t vals_relative; // 1: vals is indexed from rowptr[0], not from 0
    int64_t vals_count;    // vals_relative: entries in vals
    const void *B;         // FusedMM: D, the rows that the values weight
    float *C;              // null: plan only (no product)
    // FusedMM only (null otherwise): the value of an entry of row i at
    // column j is <dot_rows_i, dot_cols_j>, both of B's element type with N
    // columns (dot_rows M x N, dot_cols K x N), and vals is not read.
    const void *dot_rows;
    const void *dot_cols;
    int64_t M;
    int64_t K;
    int64_t N;
    Thresholds th;
    PlanBuffers plan;
    PlanShape shape;
    uint32_t epoch;
    int32_t wait_polls;    // bound of every wait for a plan entry
};

// The bound the next calls put in WorkerArgs::wait_polls.
int32_t current_wait_polls();

// Enqueue a call: one launch that plans and computes the product (the plan
// alone when a.C is null).  start/stop (each may be null) are attached to
// the start and the end of that dispatch.
hipError_t launch_worker(const WorkerConfig &cfg, const WorkerArgs &args,
                         hipStream_t stream, hipEvent_t start, hipEvent_t stop);

// The launchers of the product kernel's variants, one per source file
// (worker_<kind>_<buf|flat>.hip): fp32, bf16 and FusedMM forms, with B
// behind a buffer resource (below 4 GiB) or flat 64-bit addresses.
#define SDL_DECLARE_LAUNCH(name)                                                \
    hipError_t name(const WorkerConfig &cfg, const WorkerArgs &a, hipStream_t s, \
                    hipEvent_t e0, hipEvent_t e1);
SDL_DECLARE_LAUNCH(launch_f32_buf)
SDL_DECLARE_LAUNCH(launch_f32_flat)
SDL_DECLARE_LAUNCH(launch_bf16_buf)
SDL_DECLARE_LAUNCH(launch_bf16_flat)
SDL_DECLARE_LAUNCH(launch_fused_buf)
SDL_DECLARE_LAUNCH(launch_fused_flat)
SDL_DECLARE_LAUNCH(launch_f32_pair)
SDL_DECLARE_LAUNCH(launch_bf16_pair)
#undef SDL_DECLARE_LAUNCH

// One SDDMM call (sddmm.hip): A[p - rowptr[0]] = <C_i, B_colind[p]>.
struct SddmmArgs {
    int dtype;               // SPMM_DTYPE_*: both dense operands
    const int32_t *rowptr;
    const int32_t *colind;
    const void *C;           // M x N
    const void *B;           // K x N
    float *A;                // nnz values, CSR order
    int64_t M;
    int64_t K;
    int64_t N;
    int64_t nnz;             // rowptr[M] - rowptr[0]
};

// Enqueue one SDDMM launch; start/stop (may be null) are attached to it.
hipError_t launch_sddmm(const SddmmArgs &a, hipStream_t stream,
                        hipEvent_t start, hipEvent_t stop);

// Enqueue the exact widening of n bf16 values (bit patterns, 2-byte
// aligned) to fp32: out[i] = in[i] << 16 as a float.
hipError_t launch_widen_bf16(const uint16_t *in, float *out, int64_t n, hipStream_t stream);

// One element-balanced product (eb.hip): equal spans of stored entries per
// wavefront, partial rows at span ends combined through carry slots.
struct EbArgs {
    const int32_t *rowptr;
    const int32_t *colind;
    const void *vals;
    const void *B;
    float *C;
    int64_t M;
    int64_t K;
    int64_t N;
    int64_t waves;        // spans (wavefronts) of the launch
    float *carry_val;     // [2 * waves * N] partial rows: head and tail slot
    uint64_t *arrive;     // [waves] arrival counters, tagged with epoch
    uint32_t *queues;     // the stream's product queue counters: this call
                          // clears the set of epoch + 1 (PlanBuffers::queues)
    uint32_t epoch;       // this call's epoch (words with another tag are 0)
};

// Enqueue the element-balanced kernel (one launch; start/stop attached).
hipError_t launch_eb(const WorkerConfig &cfg, const EbArgs &a, hipStream_t stream,
                     hipEvent_t start, hipEvent_t stop);
int64_t eb_waves();

// Plain descriptors for the plan export.
struct LongRow {
    int32_t row;
    int32_t first_chunk;
    int32_t n_chunks;
};

struct Chunk {
    int32_t row;
    int32_t p0;
    int32_t p1;
    int32_t long_idx;
};

// Copy the tagged plan of a finished plan-only launch into plain device
// arrays (at most `cap` records each; a record whose word does not carry
// `epoch` is written as -1).  counts_out[6] gets n_short, n_medium, n_long,
// n_chunks, n_hub, n_hub * n_slabs; hub chunks in item order (slab-major),
// their bounds found by the product's own search over colind.  Enqueued on
// `stream`.
hipError_t launch_plan_export(const int32_t *rowptr, const int32_t *colind,
                              Thresholds th,
                              const PlanBuffers &pb, uint32_t epoch,
                              int64_t cap, int32_t *medium_out,
                              LongRow *long_out, Chunk *chunk_out,
                              int32_t *hub_out, Chunk *hub_chunk_out,
                              int64_t *counts_out, hipStream_t stream);

}  // namespace sdl
