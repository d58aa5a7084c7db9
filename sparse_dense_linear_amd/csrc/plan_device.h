// plan_device.h -- the row plan, computed by the plan kernel.
//
// Pages:
//   [Sgap]     "Sgap: Towards Efficient Sparse Tensor Algebra Compilation
//              for GPU": prior-work survey (Yang et al. choose between an
//              nnz-balanced split and a row split) and the DA-SpMM points EB
//              (element balanced) and RB (row balanced).
//   [IntelMax] "Performance Optimization of Deep Learning Sparse Matrix
//              Kernels on Intel Max Series GPU", SDDMM implementation: the
//              nnzr non-zeros of a row are divided equally among NT workers.
//
// The plan sorts rows by length into three kinds and cuts long rows into
// near-equal nnz chunks, so that the product can give short rows a lane
// group each (row split), medium rows a wavefront each, and long rows
// several wavefronts (nnz split).  Its lists are a pure function of rowptr
// and the thresholds: ascending row order, placed by prefix sums.
//
// The rows are cut into n_tiles tiles and one wavefront plans each tile:
//   1. count the tile's medium rows, long rows and chunks and publish the
//      three counts;
//   2. add up the counts of all earlier tiles; a count that is not visible
//      yet after a few polls is recomputed by this wavefront from rowptr
//      (counting is idempotent), so no wavefront ever waits for another;
//   3. write the tile's entries of the lists (for long rows: clear their C
//      rows, then publish the rows and their chunks); the last tile also
//      publishes the totals.
// The product kernel runs after the plan kernel has ended, on the same
// stream.  Every published word is tagged with the call's epoch (see
// PlanBuffers), and the product skips an entry that does not carry it.
#pragma once

#include "internal.h"

namespace sdl {

constexpr int kPlanPolls = 8;  // polls for an earlier tile's counts

// ------------------------------------------------------- tagged words

__device__ inline uint64_t tag_load(const uint64_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline void tag_store(uint64_t *p, uint32_t epoch, uint32_t v)
{
    __hip_atomic_store(p, ((uint64_t)epoch << 32) | v, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline bool tag_is(uint64_t w, uint32_t epoch)
{
    return (uint32_t)(w >> 32) == epoch;
}

// ------------------------------------------------------------ context

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
    // len < 2^31 and chunk_nnz < 2^31: the 32-bit unsigned sum is exact
    c.chunks = c.lng ? (int)(((uint32_t)len + (uint32_t)th.chunk_nnz - 1u) /
                             (uint32_t)th.chunk_nnz)
                     : 0;
    return c;
}

// Per-wavefront LDS list of one plan round's long rows.
struct PlanLds {
    int row[kPlanRoundRows];
    int cfirst[kPlanRoundRows];   // first chunk, relative to the round
};

struct PlanCtx {
    const int32_t *rowptr;
    float *C;          // null: do not clear long rows (plan only)
    int64_t M;
    int64_t N;
    Thresholds th;
    PlanBuffers pb;
    PlanShape sh;
    uint32_t epoch;
    int lane;
};

__device__ inline int wave_sum_i(int v)
{
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1)
        v += __shfl_xor(v, off);
    return v;
}

__device__ inline int wave_excl_scan_i(int v, int lane)
{
    int x = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off)
            x += y;
    }
    return x - v;
}

// The kPlanLaneRows consecutive rows of this lane in a round starting at
// `base`, classified (rows at or past r1 count as nothing).
struct LaneRows {
    int64_t start[kPlanLaneRows];
    int64_t len[kPlanLaneRows];
    RowClass rc[kPlanLaneRows];
};

__device__ inline LaneRows lane_rows(const PlanCtx &c, int64_t base, int64_t r1)
{
    LaneRows q;
    const int64_t rb = base + (int64_t)kPlanLaneRows * c.lane;
    int64_t rp[kPlanLaneRows + 1];
#pragma unroll
    for (int k = 0; k <= kPlanLaneRows; ++k)
        rp[k] = rb + k <= r1 ? c.rowptr[rb + k] : 0;
#pragma unroll
    for (int k = 0; k < kPlanLaneRows; ++k) {
        const bool valid = rb + k < r1;
        q.start[k] = rp[k];
        q.len[k] = valid ? rp[k + 1] - rp[k] : 0;
        q.rc[k] = valid ? classify(q.len[k], c.th) : RowClass{0, 0, 0};
    }
    return q;
}

__device__ inline void tile_range(const PlanCtx &c, int64_t t, int64_t *r0, int64_t *r1)
{
    *r0 = t * c.sh.tile_rows;
    *r1 = *r0 + c.sh.tile_rows < c.M ? *r0 + c.sh.tile_rows : c.M;
}

// Counts of tile t: medium rows, long rows, chunks (wave-uniform).
__device__ inline void count_tile(const PlanCtx &c, int64_t t, int *med,
                                  int *lng, int *chunks)
{
    int64_t r0, r1;
    tile_range(c, t, &r0, &r1);
    int m = 0, l = 0, ch = 0;
    for (int64_t base = r0; base < r1; base += kPlanRoundRows) {
        const LaneRows q = lane_rows(c, base, r1);
#pragma unroll
        for (int k = 0; k < kPlanLaneRows; ++k) {
            m += q.rc[k].medium;
            l += q.rc[k].lng;
            ch += q.rc[k].chunks;
        }
    }
    *med = wave_sum_i(m);
    *lng = wave_sum_i(l);
    *chunks = wave_sum_i(ch);
}

// Sums of the counts of tiles 0 .. t-1.  Counts not visible after a few
// polls are recomputed here.
__device__ inline void prefix_before(const PlanCtx &c, int64_t t, int *med,
                                     int *lng, int *chunks)
{
    int sm = 0, sl = 0, sc = 0;
    for (int64_t jb = 0; jb < t; jb += kWave) {
        const int64_t j = jb + c.lane;
        bool ready = j >= t;
        int vm = 0, vl = 0, vc = 0;
        for (int poll = 0; poll < kPlanPolls; ++poll) {
            if (!ready) {
                const uint64_t w0 = tag_load(c.pb.agg + 3 * j + 0);
                const uint64_t w1 = tag_load(c.pb.agg + 3 * j + 1);
                const uint64_t w2 = tag_load(c.pb.agg + 3 * j + 2);
                if (tag_is(w0, c.epoch) && tag_is(w1, c.epoch) && tag_is(w2, c.epoch)) {
                    vm = (int)(uint32_t)w0;
                    vl = (int)(uint32_t)w1;
                    vc = (int)(uint32_t)w2;
                    ready = true;
                }
            }
            if (__ballot(!ready) == 0)
                break;
            __builtin_amdgcn_s_sleep(1);
        }
        // recount whatever is still missing, one tile at a time
        uint64_t missing = __ballot(!ready);
        while (missing) {
            const int l = __builtin_ctzll(missing);
            missing &= missing - 1;
            int m, lg, ch;
            count_tile(c, jb + l, &m, &lg, &ch);
            if (c.lane == l) {
                vm = m;
                vl = lg;
                vc = ch;
            }
        }
        sm += vm;
        sl += vl;
        sc += vc;
    }
    *med = wave_sum_i(sm);
    *lng = wave_sum_i(sl);
    *chunks = wave_sum_i(sc);
}

// Plan tile t.  Never waits for another wavefront.
__device__ inline void plan_tile(const PlanCtx &c, int64_t t, PlanLds &L)
{
    int64_t r0, r1;
    tile_range(c, t, &r0, &r1);
    const bool one_round = r1 - r0 <= kPlanRoundRows;
    LaneRows q = lane_rows(c, r0, r1);

    // 1. publish this tile's counts
    int own_med, own_long, own_chunks;
    if (one_round) {
        int m = 0, l = 0, ch = 0;
#pragma unroll
        for (int k = 0; k < kPlanLaneRows; ++k) {
            m += q.rc[k].medium;
            l += q.rc[k].lng;
            ch += q.rc[k].chunks;
        }
        own_med = wave_sum_i(m);
        own_long = wave_sum_i(l);
        own_chunks = wave_sum_i(ch);
    } else {
        count_tile(c, t, &own_med, &own_long, &own_chunks);
    }
    if (c.lane == 0) {
        tag_store(c.pb.agg + 3 * t + 0, c.epoch, (uint32_t)own_med);
        tag_store(c.pb.agg + 3 * t + 1, c.epoch, (uint32_t)own_long);
        tag_store(c.pb.agg + 3 * t + 2, c.epoch, (uint32_t)own_chunks);
    }

    // 2. offsets from the earlier tiles
    int med_off, long_off, chunk_off;
    prefix_before(c, t, &med_off, &long_off, &chunk_off);
    if (t == c.sh.n_tiles - 1 && c.lane == 0) {
        const int n_med = med_off + own_med, n_long = long_off + own_long;
        tag_store(c.pb.counts + 0, c.epoch, (uint32_t)n_med);
        tag_store(c.pb.counts + 1, c.epoch, (uint32_t)n_long);
        tag_store(c.pb.counts + 2, c.epoch, (uint32_t)(chunk_off + own_chunks));
        tag_store(c.pb.counts + 3, c.epoch, (uint32_t)(c.M - n_med - n_long));
    }

    // 3. the tile's entries, a round of kPlanRoundRows rows at a time
    for (int64_t base = r0; base < r1; base += kPlanRoundRows) {
        if (base != r0)
            q = lane_rows(c, base, r1);
        int my_med = 0, my_long = 0, my_chunks = 0;
#pragma unroll
        for (int k = 0; k < kPlanLaneRows; ++k) {
            my_med += q.rc[k].medium;
            my_long += q.rc[k].lng;
            my_chunks += q.rc[k].chunks;
        }
        int mpos = wave_excl_scan_i(my_med, c.lane);
        int lpos = wave_excl_scan_i(my_long, c.lane);
        int cpos = wave_excl_scan_i(my_chunks, c.lane);
        const int round_med = __shfl(mpos + my_med, kWave - 1);
        const int round_long = __shfl(lpos + my_long, kWave - 1);
        const int round_chunks = __shfl(cpos + my_chunks, kWave - 1);
        const int64_t rb = base + (int64_t)kPlanLaneRows * c.lane;
#pragma unroll
        for (int k = 0; k < kPlanLaneRows; ++k) {
            if (q.rc[k].medium)
                tag_store(c.pb.medium_rows + med_off + mpos++, c.epoch, (uint32_t)(rb + k));
            if (q.rc[k].lng) {
                L.row[lpos] = (int)(rb + k);
                L.cfirst[lpos] = cpos;
                ++lpos;
                cpos += q.rc[k].chunks;
            }
        }
        if (round_long > 0) {
            // Clear the C rows of this round's long rows (the product adds
            // their chunks into them with atomics).
            if (c.C != nullptr) {
                for (int x = 0; x < round_long; ++x) {
                    float *crow = c.C + (int64_t)L.row[x] * c.N;
                    for (int64_t n = c.lane; n < c.N; n += kWave)
                        crow[n] = 0.0f;
                }
            }
            for (int x = c.lane; x < round_long; x += kWave) {
                tag_store(c.pb.long_row + long_off + x, c.epoch, (uint32_t)L.row[x]);
                tag_store(c.pb.long_first + long_off + x, c.epoch,
                          (uint32_t)(chunk_off + L.cfirst[x]));
            }
            // Chunk table: chunk x of the round belongs to the last long row
            // whose first chunk is <= x.
            for (int x = c.lane; x < round_chunks; x += kWave) {
                const int64_t ci = (int64_t)chunk_off + x;
                if (ci >= c.pb.chunk_cap)
                    break;
                int lo = 0, hi = round_long - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (L.cfirst[mid] <= x)
                        lo = mid;
                    else
                        hi = mid - 1;
                }
                tag_store(c.pb.chunk_row + ci, c.epoch, (uint32_t)L.row[lo]);
                tag_store(c.pb.chunk_k + ci, c.epoch, (uint32_t)(x - L.cfirst[lo]));
            }
        }
        med_off += round_med;
        long_off += round_long;
        chunk_off += round_chunks;
    }
}

}  // namespace sdl
