// plan.hip -- row-binning pass of the CSR sparse x dense product.
//
// Pages:
//   [Sgap]     "Sgap: Towards Efficient Sparse Tensor Algebra Compilation
//              for GPU": survey of prior SpMM work (Yang et al. pick between
//              an nnz-balanced split and a row split) and the DA-SpMM points
//              EB (element balanced) and RB (row balanced).
//   [IntelMax] "Performance Optimization of Deep Learning Sparse Matrix
//              Kernels on Intel Max Series GPU", SDDMM implementation: the
//              nnzr non-zeros of a row are divided equally among NT workers.
//
// The pass sorts rows by length into three bins and cuts long rows into
// near-equal nnz chunks, so that the worker can give short rows a lane group
// each (row split), medium rows a wavefront each, and long rows several
// wavefronts (nnz split).  Output is a pure function of rowptr and the
// thresholds: lists are compacted in ascending row order with block-wide
// prefix sums, never with atomic appends.
//
// Two kernels over the same tiling of the rows:
//   plan_count   per tile: number of medium rows, long rows, chunks, short rows
//   plan_scatter per tile: offsets = sums over earlier tiles, then a prefix
//                sum inside the tile places every medium row, long row and
//                chunk; the last tile writes the totals.  Optionally zeroes
//                the C rows of long rows, which the worker accumulates into
//                with atomics.
#include <hip/hip_ext.h>

#include "internal.h"

namespace sdl {

PlanShape plan_shape(int64_t M)
{
    // At least 1024 rows per tile and at most kPlanMaxTiles tiles, so the
    // sum over earlier tiles in plan_scatter stays a few loads per thread.
    int64_t per = (M + kPlanMaxTiles - 1) / kPlanMaxTiles;
    per = (per + 1023) / 1024 * 1024;
    PlanShape s;
    s.tile_rows = per < 1024 ? 1024 : per;
    s.n_tiles = (M + s.tile_rows - 1) / s.tile_rows;
    return s;
}

namespace {

struct RowClass {
    int medium;
    int lng;
    int chunks;
};

__device__ inline RowClass classify(int64_t len, const Thresholds &th)
{
    RowClass c;
    c.medium = (len > th.short_max) && (len <= th.medium_max);
    c.lng = len > th.medium_max;
    // len < 2^31 and chunk_nnz < 2^31, so the 32-bit unsigned sum is exact
    c.chunks = c.lng ? (int)(((uint32_t)len + (uint32_t)th.chunk_nnz - 1u) /
                             (uint32_t)th.chunk_nnz) : 0;
    return c;
}

// Sum of v over the block (kPlanBlock threads).  red has kPlanBlock/64 slots.
__device__ inline int block_sum(int v, int *red)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    for (int off = kWave / 2; off > 0; off >>= 1)
        v += __shfl_xor(v, off);
    if (lane == 0)
        red[wid] = v;
    __syncthreads();
    int total = 0;
    for (int w = 0; w < kPlanBlock / kWave; ++w)
        total += red[w];
    __syncthreads();
    return total;
}

// Exclusive prefix sum of v over the block in thread order; *total gets the
// block sum.  red has kPlanBlock/64 slots.
__device__ inline int block_exclusive_scan(int v, int *total, int *red)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    int x = v;
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off)
            x += y;
    }
    if (lane == kWave - 1)
        red[wid] = x;
    __syncthreads();
    int before = 0, sum = 0;
    for (int w = 0; w < kPlanBlock / kWave; ++w) {
        const int t = red[w];
        if (w < wid)
            before += t;
        sum += t;
    }
    __syncthreads();
    *total = sum;
    return before + x - v;
}

// Rows handled per thread per round: a round covers kPlanBlock * 4 rows.
constexpr int kRowsPerThread = 4;
constexpr int64_t kRoundRows = (int64_t)kPlanBlock * kRowsPerThread;

// Extents of the kRowsPerThread consecutive rows a thread owns in a round
// (rows past r1 get length 0 and are flagged invalid).
struct RowQuad {
    int64_t start[kRowsPerThread];
    int64_t len[kRowsPerThread];
    bool valid[kRowsPerThread];
};

__device__ inline RowQuad load_quad(const int32_t *__restrict__ rowptr,
                                    int64_t rb, int64_t r1)
{
    RowQuad q;
    int64_t rp[kRowsPerThread + 1];
#pragma unroll
    for (int k = 0; k <= kRowsPerThread; ++k)
        rp[k] = rb + k <= r1 ? rowptr[rb + k] : 0;
#pragma unroll
    for (int k = 0; k < kRowsPerThread; ++k) {
        q.valid[k] = rb + k < r1;
        q.start[k] = rp[k];
        q.len[k] = q.valid[k] ? rp[k + 1] - rp[k] : 0;
    }
    return q;
}

__global__ __launch_bounds__(kPlanBlock) void plan_count_kernel(
    const int32_t *__restrict__ rowptr, int64_t M, int64_t tile_rows,
    Thresholds th, int32_t *__restrict__ tile_counts)
{
    __shared__ int red[kPlanBlock / kWave];
    const int64_t r0 = (int64_t)blockIdx.x * tile_rows;
    const int64_t r1 = r0 + tile_rows < M ? r0 + tile_rows : M;
    int med = 0, lng = 0, chunks = 0, shrt = 0;
    for (int64_t base = r0; base < r1; base += kRoundRows) {
        const RowQuad q = load_quad(rowptr, base + kRowsPerThread * threadIdx.x, r1);
#pragma unroll
        for (int k = 0; k < kRowsPerThread; ++k) {
            if (!q.valid[k])
                continue;
            const RowClass c = classify(q.len[k], th);
            med += c.medium;
            lng += c.lng;
            chunks += c.chunks;
            shrt += !(c.medium | c.lng);
        }
    }
    med = block_sum(med, red);
    lng = block_sum(lng, red);
    chunks = block_sum(chunks, red);
    shrt = block_sum(shrt, red);
    if (threadIdx.x == 0) {
        int32_t *out = tile_counts + 4 * (int64_t)blockIdx.x;
        out[0] = med;
        out[1] = lng;
        out[2] = chunks;
        out[3] = shrt;
    }
}

__global__ __launch_bounds__(kPlanBlock) void plan_scatter_kernel(
    const int32_t *__restrict__ rowptr, int64_t M, int64_t tile_rows,
    int64_t n_tiles, Thresholds th, PlanBuffers pb, float *__restrict__ C,
    int64_t N, int zero_long)
{
    __shared__ int red[kPlanBlock / kWave];
    // This round's long rows: row, first chunk (relative to the round),
    // chunk count, first position and length.
    __shared__ int ll_row[kRoundRows];
    __shared__ int ll_cfirst[kRoundRows];
    __shared__ int ll_n[kRoundRows];
    __shared__ int ll_start[kRoundRows];
    __shared__ int ll_len[kRoundRows];
    const int64_t b = blockIdx.x;
    const int32_t *tc = pb.tile_counts;
    const int64_t r0 = b * tile_rows;
    const int64_t r1 = r0 + tile_rows < M ? r0 + tile_rows : M;

    // Issue the first round's row loads before summing the earlier tiles.
    RowQuad q = load_quad(rowptr, r0 + kRowsPerThread * threadIdx.x, r1);

    // Offsets of this tile = sums over all earlier tiles.
    int med_off = 0, long_off = 0, chunk_off = 0, short_off = 0;
    for (int64_t t = threadIdx.x; t < b; t += kPlanBlock) {
        med_off += tc[4 * t + 0];
        long_off += tc[4 * t + 1];
        chunk_off += tc[4 * t + 2];
        short_off += tc[4 * t + 3];
    }
    med_off = block_sum(med_off, red);
    long_off = block_sum(long_off, red);
    chunk_off = block_sum(chunk_off, red);
    short_off = block_sum(short_off, red);
    if (b == n_tiles - 1 && threadIdx.x == 0) {
        PlanCounts total;
        total.n_medium = med_off + tc[4 * b + 0];
        total.n_long = long_off + tc[4 * b + 1];
        total.n_chunks = chunk_off + tc[4 * b + 2];
        total.n_short = short_off + tc[4 * b + 3];
        *pb.counts = total;
    }

    for (int64_t base = r0; base < r1; base += kRoundRows) {
        const int64_t rb = base + kRowsPerThread * threadIdx.x;
        if (base != r0)
            q = load_quad(rowptr, rb, r1);
        RowClass c[kRowsPerThread];
        int my_flags = 0, my_chunks = 0;
#pragma unroll
        for (int k = 0; k < kRowsPerThread; ++k) {
            c[k] = q.valid[k] ? classify(q.len[k], th) : RowClass{0, 0, 0};
            my_flags += c[k].medium | (c[k].lng << 16);
            my_chunks += c[k].chunks;
        }
        // medium and long counts share one scan (a round has < 2^16 rows)
        int flags_total, chunk_total;
        const int flags = block_exclusive_scan(my_flags, &flags_total, red);
        int cpos = block_exclusive_scan(my_chunks, &chunk_total, red);
        int mpos = med_off + (flags & 0xFFFF);
        int lpos = flags >> 16;
#pragma unroll
        for (int k = 0; k < kRowsPerThread; ++k) {
            const int64_t r = rb + k;
            if (c[k].medium)
                pb.medium_rows[mpos++] = (int32_t)r;
            if (c[k].lng) {
                LongRow lr;
                lr.row = (int32_t)r;
                lr.first_chunk = chunk_off + cpos;
                lr.n_chunks = c[k].chunks;
                pb.long_rows[long_off + lpos] = lr;
                ll_row[lpos] = (int)r;
                ll_cfirst[lpos] = cpos;
                ll_n[lpos] = c[k].chunks;
                ll_start[lpos] = (int)q.start[k];
                ll_len[lpos] = (int)q.len[k];
                ++lpos;
                cpos += c[k].chunks;
            }
        }
        const int n_long_here = flags_total >> 16;
        if (n_long_here > 0) {
            __syncthreads();
            // Chunk descriptors of this round, all threads together: chunk x
            // belongs to the last long row whose first chunk is <= x.
            for (int x = threadIdx.x; x < chunk_total; x += kPlanBlock) {
                const int64_t ci = (int64_t)chunk_off + x;
                if (ci >= pb.chunk_cap)
                    break;
                int lo = 0, hi = n_long_here - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (ll_cfirst[mid] <= x)
                        lo = mid;
                    else
                        hi = mid - 1;
                }
                Chunk ch;
                ch.row = ll_row[lo];
                ch.long_idx = long_off + lo;
                chunk_bounds(ll_start[lo], ll_len[lo], ll_n[lo], x - ll_cfirst[lo],
                             &ch.p0, &ch.p1);
                pb.chunks[ci] = ch;
            }
            // Clear the C rows of this round's long rows.
            if (zero_long) {
                // one row per wavefront at a time, lanes across the columns
                const int lane = threadIdx.x & (kWave - 1);
                for (int x = threadIdx.x / kWave; x < n_long_here;
                     x += kPlanBlock / kWave) {
                    float *crow = C + (int64_t)ll_row[x] * N;
                    for (int64_t n = lane; n < N; n += kWave)
                        crow[n] = 0.0f;
                }
            }
            __syncthreads();
        }
        med_off += flags_total & 0xFFFF;
        long_off += n_long_here;
        chunk_off += chunk_total;
    }
}

}  // namespace

hipError_t launch_plan(const int32_t *rowptr, int64_t M, Thresholds th,
                       const PlanBuffers &buf, float *C, int64_t N,
                       hipStream_t stream, hipEvent_t start, hipEvent_t stop)
{
    const PlanShape s = plan_shape(M);
    if (s.n_tiles == 0)
        return hipSuccess;
    hipExtLaunchKernelGGL(plan_count_kernel, dim3((unsigned)s.n_tiles),
                          dim3(kPlanBlock), 0, stream, start, nullptr, 0,
                          rowptr, M, s.tile_rows, th, buf.tile_counts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    hipExtLaunchKernelGGL(plan_scatter_kernel, dim3((unsigned)s.n_tiles),
                          dim3(kPlanBlock), 0, stream, nullptr, stop, 0,
                          rowptr, M, s.tile_rows, s.n_tiles, th, buf, C, N,
                          C != nullptr ? 1 : 0);
    return hipGetLastError();
}

namespace {

__global__ __launch_bounds__(kPlanBlock) void chunk_expand_kernel(
    const int32_t *__restrict__ rowptr, PlanBuffers pb, int64_t count,
    Chunk *__restrict__ out)
{
    const int64_t c = (int64_t)blockIdx.x * kPlanBlock + threadIdx.x;
    if (c < count)
        out[c] = resolve_chunk(c, pb, pb.counts->n_long, rowptr);
}

}  // namespace

hipError_t launch_chunk_expand(const int32_t *rowptr, Thresholds th,
                               const PlanBuffers &buf, int64_t count,
                               Chunk *out, hipStream_t stream)
{
    (void)th;
    if (count <= 0)
        return hipSuccess;
    const int64_t blocks = (count + kPlanBlock - 1) / kPlanBlock;
    hipLaunchKernelGGL(chunk_expand_kernel, dim3((unsigned)blocks),
                       dim3(kPlanBlock), 0, stream, rowptr, buf, count, out);
    return hipGetLastError();
}

}  // namespace sdl
