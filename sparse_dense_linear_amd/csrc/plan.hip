// plan.hip -- the plan on its own (for the plan export used by tests), the
// launch of a call, and the plan export.
//
// A call is one launch (worker.hip): its first workgroups compute the plan
// (plan_device.h) and the rest compute the product.  The plan-only kernel
// here runs the same plan blocks without a product.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "internal.h"
#include "plan_device.h"

namespace sdl {

PlanShape plan_shape(int64_t M)
{
    // Whole rounds of kPlanRoundRows rows per tile, at most kPlanMaxTiles
    // tiles (so summing the counts of earlier tiles stays a few loads per
    // lane).
    int64_t per = (M + kPlanMaxTiles - 1) / kPlanMaxTiles;
    per = (per + kPlanRoundRows - 1) / kPlanRoundRows * kPlanRoundRows;
    PlanShape s;
    s.tile_rows = per < kPlanRoundRows ? kPlanRoundRows : per;
    s.n_tiles = (M + s.tile_rows - 1) / s.tile_rows;
    return s;
}

namespace {

// One workgroup per plan block, one wavefront per plan tile.
__global__ __launch_bounds__(kPlanBlockWaves * kWave) void plan_kernel(WorkerArgs a)
{
    __shared__ PlanBlockLds lds;
    PlanCtx pc;
    pc.rowptr = a.rowptr;
    pc.C = a.C;
    pc.M = a.M;
    pc.N = a.N;
    pc.th = a.th;
    pc.pb = a.plan;
    pc.sh = a.shape;
    pc.epoch = a.epoch;
    pc.lane = threadIdx.x & (kWave - 1);
    plan_block(pc, blockIdx.x, threadIdx.x / kWave, lds);
}

constexpr int kExportBlock = 256;

__device__ inline int32_t untag(uint64_t w, uint32_t epoch)
{
    return tag_is(w, epoch) ? (int32_t)(uint32_t)w : -1;
}

__global__ __launch_bounds__(kExportBlock) void plan_export_kernel(
    const int32_t *__restrict__ rowptr, Thresholds th,
    PlanBuffers pb, uint32_t epoch, int64_t cap, int32_t *medium_out,
    LongRow *long_out, Chunk *chunk_out, int32_t *hub_out, int64_t *counts_out)
{
    const int64_t n_med = untag(pb.counts[0], epoch);
    const int64_t n_long = untag(pb.counts[1], epoch);
    const int64_t n_ch = untag(pb.counts[2], epoch);
    const int64_t n_hub = untag(pb.counts[4], epoch);
    const int64_t i = (int64_t)blockIdx.x * kExportBlock + threadIdx.x;
    if (i == 0) {
        counts_out[0] = untag(pb.counts[3], epoch);
        counts_out[1] = n_med;
        counts_out[2] = n_long;
        counts_out[3] = n_ch;
        counts_out[4] = n_hub;
        counts_out[5] = n_hub < 0 ? -1 : n_hub * th.n_slabs;
    }
    if (i >= cap)
        return;
    if (i < n_med)
        medium_out[i] = untag(pb.medium_rows[i], epoch);
    if (i < n_hub)
        hub_out[i] = untag(*hub_slot(pb, i), epoch);
    if (i < n_long) {
        LongRow lr;
        lr.row = untag(pb.long_row[i], epoch);
        lr.first_chunk = untag(pb.long_first[i], epoch);
        const int64_t len = lr.row < 0 ? 0 : (int64_t)rowptr[lr.row + 1] - rowptr[lr.row];
        lr.n_chunks = (int32_t)((len + th.chunk_nnz - 1) / th.chunk_nnz);
        long_out[i] = lr;
    }
    if (i < n_ch) {
        // owning long row: last whose first chunk is <= i
        int64_t lo = 0, hi = n_long - 1;
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) >> 1;
            if (untag(pb.long_first[mid], epoch) <= i)
                lo = mid;
            else
                hi = mid - 1;
        }
        Chunk ch;
        ch.long_idx = (int32_t)lo;
        int64_t row, k;
        if (i < pb.chunk_cap) {
            // the table entry is what the product reads
            row = untag(pb.chunk_row[i], epoch);
            k = untag(pb.chunk_k[i], epoch);
        } else {
            row = untag(pb.long_row[lo], epoch);
            k = i - untag(pb.long_first[lo], epoch);
        }
        ch.row = (int32_t)row;
        if (row >= 0 && k >= 0) {
            const int64_t start = rowptr[row];
            const int64_t len = (int64_t)rowptr[row + 1] - start;
            const int64_t n = (len + th.chunk_nnz - 1) / th.chunk_nnz;
            int64_t p0, p1;
            chunk_bounds(start, len, n, k, &p0, &p1);
            ch.p0 = (int32_t)p0;
            ch.p1 = (int32_t)p1;
        } else {
            ch.p0 = ch.p1 = -1;
        }
        chunk_out[i] = ch;
    }
}

// Hub chunks in item order (slab-major), one wavefront each, bounds found
// by the same search the product uses (slab_bounds).
__global__ __launch_bounds__(kExportBlock) void hub_chunk_export_kernel(
    const int32_t *__restrict__ rowptr, const int32_t *__restrict__ colind,
    Thresholds th, PlanBuffers pb, uint32_t epoch, int64_t cap, Chunk *out)
{
    const int64_t c = (int64_t)blockIdx.x * (kExportBlock / kWave) + threadIdx.x / kWave;
    const int64_t n_hub = untag(pb.counts[4], epoch);
    if (n_hub <= 0 || c >= cap || c >= n_hub * th.n_slabs)
        return;
    const int64_t s = c / n_hub, l = c - s * n_hub;
    Chunk ch;
    ch.long_idx = (int32_t)l;
    ch.row = untag(*hub_slot(pb, l), epoch);
    ch.p0 = ch.p1 = -1;
    if (ch.row >= 0) {
        const int64_t start = rowptr[ch.row], end = rowptr[ch.row + 1];
        const int64_t t0 = s * (int64_t)th.slab_rows, t1 = t0 + th.slab_rows;
        int64_t p0, p1;
        slab_bounds(colind, start, end, (int32_t)(t0 < INT32_MAX ? t0 : INT32_MAX),
                    (int32_t)(t1 < INT32_MAX ? t1 : INT32_MAX), &p0, &p1);
        ch.p0 = (int32_t)(s == 0 ? start : p0);
        ch.p1 = (int32_t)(s + 1 >= th.n_slabs ? end : p1);
    }
    if ((threadIdx.x & (kWave - 1)) == 0)
        out[c] = ch;
}

}  // namespace

hipError_t launch_call(const WorkerConfig &cfg, const WorkerArgs &a,
                       hipStream_t s, hipEvent_t e0, hipEvent_t e1);

hipError_t launch_worker(const WorkerConfig &cfg, const WorkerArgs &a,
                         hipStream_t stream, hipEvent_t start, hipEvent_t stop)
{
    if (a.C != nullptr)
        return launch_call(cfg, a, stream, start, stop);
    // plan only
    const int64_t blocks = (a.shape.n_tiles + kPlanBlockWaves - 1) / kPlanBlockWaves;
    hipExtLaunchKernelGGL(plan_kernel, dim3((unsigned)blocks),
                          dim3(kPlanBlockWaves * kWave), 0, stream, start, stop, 0, a);
    return hipGetLastError();
}

hipError_t launch_plan_export(const int32_t *rowptr, const int32_t *colind,
                              Thresholds th,
                              const PlanBuffers &pb, uint32_t epoch,
                              int64_t cap, int32_t *medium_out,
                              LongRow *long_out, Chunk *chunk_out,
                              int32_t *hub_out, Chunk *hub_chunk_out,
                              int64_t *counts_out, hipStream_t stream)
{
    const int64_t n = cap > 1 ? cap : 1;
    const int64_t blocks = (n + kExportBlock - 1) / kExportBlock;
    hipLaunchKernelGGL(plan_export_kernel, dim3((unsigned)blocks),
                       dim3(kExportBlock), 0, stream, rowptr, th, pb, epoch,
                       cap, medium_out, long_out, chunk_out, hub_out, counts_out);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || cap == 0 || colind == nullptr)
        return err;
    const int64_t waves_per_block = kExportBlock / kWave;
    const int64_t hblocks = (cap + waves_per_block - 1) / waves_per_block;
    hipLaunchKernelGGL(hub_chunk_export_kernel, dim3((unsigned)hblocks),
                       dim3(kExportBlock), 0, stream, rowptr, colind, th, pb, epoch,
                       cap, hub_chunk_out);
    return hipGetLastError();
}

}  // namespace sdl
