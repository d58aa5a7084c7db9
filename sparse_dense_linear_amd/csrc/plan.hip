// plan.hip -- the plan kernel, the launch sequence of a call, and the plan
// export for tests.
//
// A call is two launches on its stream: the plan kernel (plan_device.h: one
// wavefront per tile) and the product kernel (worker.hip), which reads the
// finished plan.
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

// One wavefront per plan tile.
__global__ __launch_bounds__(kBlock) void plan_kernel(WorkerArgs a)
{
    __shared__ PlanLds lds[kWavesPerBlock];
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    if (t >= a.shape.n_tiles)
        return;
    PlanCtx pc;
    pc.rowptr = a.rowptr;
    pc.C = a.C;
    pc.M = a.M;
    pc.N = a.N;
    pc.th = a.th;
    pc.pb = a.plan;
    pc.sh = a.shape;
    pc.epoch = a.epoch;
    pc.lane = lane;
    plan_tile(pc, t, lds[threadIdx.x / kWave]);
}

constexpr int kExportBlock = 256;

__device__ inline int32_t untag(uint64_t w, uint32_t epoch)
{
    return tag_is(w, epoch) ? (int32_t)(uint32_t)w : -1;
}

__global__ __launch_bounds__(kExportBlock) void plan_export_kernel(
    const int32_t *__restrict__ rowptr, int64_t M, Thresholds th,
    PlanBuffers pb, uint32_t epoch, int64_t cap, int32_t *medium_out,
    LongRow *long_out, Chunk *chunk_out, int64_t *counts_out)
{
    const int64_t n_med = untag(pb.counts[0], epoch);
    const int64_t n_long = untag(pb.counts[1], epoch);
    const int64_t n_ch = untag(pb.counts[2], epoch);
    const int64_t i = (int64_t)blockIdx.x * kExportBlock + threadIdx.x;
    if (i == 0) {
        counts_out[0] = untag(pb.counts[3], epoch);
        counts_out[1] = n_med;
        counts_out[2] = n_long;
        counts_out[3] = n_ch;
    }
    if (i >= cap)
        return;
    if (i < n_med)
        medium_out[i] = untag(pb.medium_rows[i], epoch);
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

}  // namespace

hipError_t launch_product(const WorkerConfig &cfg, const WorkerArgs &a,
                          hipStream_t s, hipEvent_t e0, hipEvent_t e1);

hipError_t launch_worker(const WorkerConfig &cfg, const WorkerArgs &a,
                         hipStream_t stream, hipEvent_t plan_start,
                         hipEvent_t work_start, hipEvent_t work_stop)
{
    if (a.shape.n_tiles > 0) {
        const int64_t blocks = (a.shape.n_tiles + kWavesPerBlock - 1) / kWavesPerBlock;
        hipExtLaunchKernelGGL(plan_kernel, dim3((unsigned)blocks), dim3(kBlock), 0,
                              stream, plan_start, nullptr, 0, a);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    if (a.C == nullptr)
        return hipSuccess;  // plan only
    return launch_product(cfg, a, stream, work_start, work_stop);
}

hipError_t launch_plan_export(const int32_t *rowptr, int64_t M, Thresholds th,
                              const PlanBuffers &pb, uint32_t epoch,
                              int64_t cap, int32_t *medium_out,
                              LongRow *long_out, Chunk *chunk_out,
                              int64_t *counts_out, hipStream_t stream)
{
    (void)M;
    const int64_t n = cap > 1 ? cap : 1;
    const int64_t blocks = (n + kExportBlock - 1) / kExportBlock;
    hipLaunchKernelGGL(plan_export_kernel, dim3((unsigned)blocks),
                       dim3(kExportBlock), 0, stream, rowptr, M, th, pb, epoch,
                       cap, medium_out, long_out, chunk_out, counts_out);
    return hipGetLastError();
}

}  // namespace sdl
