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
#include "internal.h"

namespace sdl {

PlanShape plan_shape(int64_t M)
{
    // At least 1024 rows per tile and at most kPlanMaxTiles tiles, so the
    // sum over earlier tiles in plan_scatter stays a few loads per thread.
    int64_t per = (M + kPlanMaxTiles - 1) / kPlanMaxTiles;
    per = (per + kPlanBlock - 1) / kPlanBlock * kPlanBlock;
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
    c.chunks = c.lng ? (int)((len + th.chunk_nnz - 1) / th.chunk_nnz) : 0;
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

__global__ __launch_bounds__(kPlanBlock) void plan_count_kernel(
    const int32_t *__restrict__ rowptr, int64_t M, int64_t tile_rows,
    Thresholds th, int32_t *__restrict__ tile_counts)
{
    __shared__ int red[kPlanBlock / kWave];
    const int64_t r0 = (int64_t)blockIdx.x * tile_rows;
    const int64_t r1 = r0 + tile_rows < M ? r0 + tile_rows : M;
    int med = 0, lng = 0, chunks = 0, shrt = 0;
    for (int64_t r = r0 + threadIdx.x; r < r1; r += kPlanBlock) {
        const int64_t len = (int64_t)rowptr[r + 1] - rowptr[r];
        const RowClass c = classify(len, th);
        med += c.medium;
        lng += c.lng;
        chunks += c.chunks;
        shrt += !(c.medium | c.lng);
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
    __shared__ int long_list[kPlanBlock];
    const int64_t b = blockIdx.x;
    const int32_t *tc = pb.tile_counts;

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

    const int64_t r0 = b * tile_rows;
    const int64_t r1 = r0 + tile_rows < M ? r0 + tile_rows : M;
    for (int64_t base = r0; base < r1; base += kPlanBlock) {
        const int64_t r = base + threadIdx.x;
        int64_t start = 0, len = 0;
        if (r < r1) {
            start = rowptr[r];
            len = (int64_t)rowptr[r + 1] - start;
        }
        const RowClass c = r < r1 ? classify(len, th) : RowClass{0, 0, 0};
        // medium and long flags share one scan: counts per round fit 16 bits
        int flags_total, chunk_total;
        const int flags = block_exclusive_scan(c.medium | (c.lng << 16),
                                               &flags_total, red);
        const int cpos = block_exclusive_scan(c.chunks, &chunk_total, red);
        if (c.medium)
            pb.medium_rows[med_off + (flags & 0xFFFF)] = (int32_t)r;
        if (c.lng) {
            const int li = long_off + (flags >> 16);
            const int first = chunk_off + cpos;
            LongRow lr;
            lr.row = (int32_t)r;
            lr.first_chunk = first;
            lr.n_chunks = c.chunks;
            pb.long_rows[li] = lr;
            for (int k = 0; k < c.chunks; ++k) {
                const int64_t ci = (int64_t)first + k;
                if (ci >= pb.chunk_cap)
                    break;
                Chunk ch;
                ch.row = (int32_t)r;
                ch.long_idx = li;
                chunk_bounds(start, len, c.chunks, k, &ch.p0, &ch.p1);
                pb.chunks[ci] = ch;
            }
            long_list[flags >> 16] = (int)(r - base);
        }
        med_off += flags_total & 0xFFFF;
        long_off += flags_total >> 16;
        chunk_off += chunk_total;
        // Clear the C rows of this round's long rows, all threads together.
        const int n_long_here = flags_total >> 16;
        if (zero_long && n_long_here > 0) {
            __syncthreads();
            for (int q = 0; q < n_long_here; ++q) {
                float *crow = C + (base + long_list[q]) * N;
                for (int64_t n = threadIdx.x; n < N; n += kPlanBlock)
                    crow[n] = 0.0f;
            }
            __syncthreads();
        }
    }
}

}  // namespace

hipError_t launch_plan(const int32_t *rowptr, int64_t M, Thresholds th,
                       const PlanBuffers &buf, float *C, int64_t N,
                       hipStream_t stream)
{
    const PlanShape s = plan_shape(M);
    if (s.n_tiles == 0)
        return hipSuccess;
    hipLaunchKernelGGL(plan_count_kernel, dim3((unsigned)s.n_tiles),
                       dim3(kPlanBlock), 0, stream, rowptr, M, s.tile_rows,
                       th, buf.tile_counts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    hipLaunchKernelGGL(plan_scatter_kernel, dim3((unsigned)s.n_tiles),
                       dim3(kPlanBlock), 0, stream, rowptr, M, s.tile_rows,
                       s.n_tiles, th, buf, C, N, C != nullptr ? 1 : 0);
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
