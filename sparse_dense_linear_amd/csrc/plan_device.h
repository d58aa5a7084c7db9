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
// The plan sorts rows by length into four kinds and cuts long rows into
// near-equal nnz chunks, so that the product can give short rows a lane
// group each (row split), medium rows a wavefront each, and long rows
// several wavefronts (nnz split).  Hub rows (the longest) are listed only:
// the product cuts them at column-slab boundaries itself (slab_bound).
// The lists are a pure function of rowptr and the thresholds: ascending row
// order, placed by prefix sums.
//
// The rows are cut into n_tiles tiles, one wavefront per tile, and the
// tiles are grouped kPlanBlockWaves to a workgroup (a plan block):
//   1. each wavefront counts its tile's medium rows, long rows, chunks and
//      hub rows;
//      the block adds them up in LDS and publishes the block's totals;
//   2. one wavefront adds up the totals of all earlier blocks; a total that
//      is not visible yet after a few polls is recomputed by this wavefront
//      from rowptr (counting is idempotent), so no workgroup ever waits for
//      another;
//   3. each wavefront writes its tile's entries of the lists (for long and
//      hub rows: clear their C rows, then publish the rows and chunks);
//      the last block also publishes the totals.
// Plan blocks are the first workgroups of the same launch as the product,
// so the product reads the plan while it is being written: every published
// word is tagged with the call's epoch (see PlanBuffers), and the product
// polls for the tag of each word it needs.
#pragma once

#include "internal.h"

namespace sdl {

constexpr int kPlanPolls = 8;  // polls for an earlier block's counts

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

// Wait until this wavefront's earlier global stores and atomics have
// completed (vmcnt counts stores as well as loads on gfx9-family parts).
// Device-coherent stores that have completed are visible device-wide, so a
// tagged word stored after this point is only seen after them.  This is the
// ordering step of the compiler's own release sequence without its L2
// write-back, which only plain (non-coherent) stores need.
__device__ inline void wait_stores_done()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt untouched
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ------------------------------------------------------------ context

struct RowClass {
    int medium;
    int lng;
    int chunks;
    int hub;
};

__device__ inline RowClass classify(int64_t len, const Thresholds &th)
{
    RowClass c;
    c.medium = (len > th.short_max) && (len <= th.medium_max);
    c.lng = (len > th.medium_max) && (len <= th.hub_top);
    c.hub = len > th.hub_top;
    // len < 2^31 and chunk_nnz < 2^31: the 32-bit unsigned sum is exact
    c.chunks = c.lng ? (int)(((uint32_t)len + (uint32_t)th.chunk_nnz - 1u) /
                             (uint32_t)th.chunk_nnz)
                     : 0;
    return c;
}

// Per-wavefront LDS list of one plan round's long and hub rows.
struct PlanLds {
    int row[kPlanRoundRows];
    int cfirst[kPlanRoundRows];   // first chunk, relative to the round
    int hub[kPlanRoundRows];
};

// Hub row l of the plan (stored from the back of the long-row array).
__device__ inline uint64_t *hub_slot(const PlanBuffers &pb, int64_t l)
{
    return pb.long_row + (pb.rows - 1 - l);
}

// First position of [lo, hi) whose column is >= t, for a row whose columns
// ascend -- the bound of a column slab of a hub row.  A 32-ary search run
// by one half of the wavefront: lanes 0-31 search for t0, lanes 32-63 for
// t1 (both halves search the same row).  Each step evaluates "column < t"
// at 32 split points inside the interval and keeps the part up to the first
// split point where it fails; an interval of at most 32 positions is
// checked whole.  For a row whose columns do not ascend the result is still
// a position in [lo, hi], and it never decreases as t grows (two targets
// agree on every test until the first split point where the smaller one
// fails and the larger one does not, and there the smaller keeps the part
// at or below that point and the larger the part above it), so bounds
// computed for the slab starts s * slab_rows, s = 0, 1, ..., tile the row.
// Called by all 64 lanes; *b0 and *b1 are wave-uniform.
__device__ inline void slab_bounds(const int32_t *colind, int64_t lo, int64_t hi,
                                   int32_t t0, int32_t t1, int64_t *b0, int64_t *b1)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int half = lane >> 5;
    const int i = lane & 31;
    const int32_t t = half ? t1 : t0;
    const int32_t *row = colind + lo;
    // positions relative to lo (a row holds fewer than 2^31 entries); the
    // bound is in [l, h]
    uint32_t l = 0, h = (uint32_t)(hi - lo);
    bool done = false;
    while (__ballot(!done) != 0) {
        const uint32_t n = h - l;
        const bool whole = n <= 32;
        // split point of this lane: every position of a short interval, or
        // l + (i+1) n / 33 (strictly increasing, inside (l, h)) otherwise
        const uint32_t m = whole ? l + i : l + (uint32_t)(((uint64_t)(i + 1) * n) / 33);
        const bool use = !done && (!whole || (uint32_t)i < n);
        const bool below = use ? row[m] < t : true;
        const uint64_t fails = __ballot(use && !below);
        const uint32_t mine = (uint32_t)(fails >> (32 * half));
        const uint32_t first = mine ? (uint32_t)__builtin_ctz(mine) : 32u;
        if (!done) {
            if (whole) {
                l = first < n ? l + first : h;
                done = true;
            } else {
                const uint32_t nl = first == 0 ? l : l + (uint32_t)(((uint64_t)first * n) / 33) + 1;
                const uint32_t nh = first == 32 ? h : l + (uint32_t)(((uint64_t)(first + 1) * n) / 33);
                l = nl;
                h = nh;
            }
        }
    }
    *b0 = lo + (int64_t)__shfl(l, 0);
    *b1 = lo + (int64_t)__shfl(l, 32);
}

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
    (void)lane;
    return wave_exclusive_sum(v);
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
        q.rc[k] = valid ? classify(q.len[k], c.th) : RowClass{0, 0, 0, 0};
    }
    return q;
}

__device__ inline void tile_range(const PlanCtx &c, int64_t t, int64_t *r0, int64_t *r1)
{
    *r0 = t * c.sh.tile_rows;
    *r1 = *r0 + c.sh.tile_rows < c.M ? *r0 + c.sh.tile_rows : c.M;
}

// The counts the plan keeps per tile and per block, in this order.
struct PlanCounts {
    int v[kPlanCounts];   // medium rows, long rows, chunks, hub rows
};

__device__ inline void add_row(PlanCounts &n, const RowClass &rc)
{
    n.v[0] += rc.medium;
    n.v[1] += rc.lng;
    n.v[2] += rc.chunks;
    n.v[3] += rc.hub;
}

__device__ inline PlanCounts wave_sum_counts(PlanCounts n)
{
#pragma unroll
    for (int k = 0; k < kPlanCounts; ++k)
        n.v[k] = wave_sum_i(n.v[k]);
    return n;
}

// Counts of tile t (wave-uniform).
__device__ inline PlanCounts count_tile(const PlanCtx &c, int64_t t)
{
    int64_t r0, r1;
    tile_range(c, t, &r0, &r1);
    PlanCounts n{};
    for (int64_t base = r0; base < r1; base += kPlanRoundRows) {
        const LaneRows q = lane_rows(c, base, r1);
#pragma unroll
        for (int k = 0; k < kPlanLaneRows; ++k)
            add_row(n, q.rc[k]);
    }
    return wave_sum_counts(n);
}

// Counts of plan block b (its kPlanBlockWaves tiles), wave-uniform.
__device__ inline PlanCounts count_block(const PlanCtx &c, int64_t b)
{
    PlanCounts n{};
    const int64_t t0 = b * kPlanBlockWaves;
    for (int64_t t = t0; t < t0 + kPlanBlockWaves && t < c.sh.n_tiles; ++t) {
        const PlanCounts tc = count_tile(c, t);
#pragma unroll
        for (int k = 0; k < kPlanCounts; ++k)
            n.v[k] += tc.v[k];
    }
    return n;
}

// Sums of the published counts of plan blocks 0 .. b-1: lane l reads
// blocks l, l + 64, ... (all loads of a poll in flight together).  Counts
// not visible after a few polls are recomputed here from rowptr.
__device__ inline PlanCounts block_prefix(const PlanCtx &c, int64_t b)
{
    PlanCounts v{};
    if (b > 0) {
        uint32_t need = 0;  // bit i: block lane + 64 i is still to be read
#pragma unroll
        for (int i = 0; i < kPlanPrefixLoads; ++i)
            need |= (c.lane + kWave * i < b) ? 1u << i : 0u;
        for (int poll = 0; poll < kPlanPolls && __ballot(need != 0) != 0; ++poll) {
            if (poll > 0)
                __builtin_amdgcn_s_sleep(2);
            uint64_t wd[kPlanPrefixLoads][kPlanCounts];
#pragma unroll
            for (int i = 0; i < kPlanPrefixLoads; ++i) {
                const int64_t jb = c.lane + kWave * i;
                const int64_t jj = jb < b ? jb : b - 1;
#pragma unroll
                for (int k = 0; k < kPlanCounts; ++k)
                    wd[i][k] = tag_load(c.pb.agg + k * kPlanMaxBlocks + jj);
            }
#pragma unroll
            for (int i = 0; i < kPlanPrefixLoads; ++i) {
                bool got = (need >> i) & 1u;
#pragma unroll
                for (int k = 0; k < kPlanCounts; ++k)
                    got = got && tag_is(wd[i][k], c.epoch);
                if (got) {
#pragma unroll
                    for (int k = 0; k < kPlanCounts; ++k)
                        v.v[k] += (int)(uint32_t)wd[i][k];
                    need &= ~(1u << i);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kPlanPrefixLoads; ++i) {
            uint64_t missing = __ballot((need >> i) & 1u);
            while (missing) {
                const int l = __builtin_ctzll(missing);
                missing &= missing - 1;
                const PlanCounts bc = count_block(c, l + (int64_t)kWave * i);
                if (c.lane == l) {
#pragma unroll
                    for (int k = 0; k < kPlanCounts; ++k)
                        v.v[k] += bc.v[k];
                }
            }
        }
    }
    return wave_sum_counts(v);
}

// Block-shared state of the plan kernel.
struct PlanBlockLds {
    PlanLds wave[kPlanBlockWaves];
    int cnt[kPlanCounts][kPlanBlockWaves];   // per tile
    int off[kPlanCounts];                    // offsets of this block in the lists
};

// Clear the C rows rows[0 .. n) (the product adds their chunks into them with
// device atomics as soon as they are published, so the zeros must have
// reached device scope first: they are written as device-coherent atomic
// stores, and the caller publishes the rows only after this returns).
__device__ inline void clear_rows(const PlanCtx &c, const int *rows, int n)
{
    for (int x = 0; x < n; ++x) {
        float *crow = c.C + (int64_t)rows[x] * c.N;
        for (int64_t k = c.lane; k < c.N; k += kWave)
            __hip_atomic_store(crow + k, 0.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    wait_stores_done();
}

// Plan block b: wavefront w of the block plans tile b * kPlanBlockWaves + w.
// Called by every thread of the block (it synchronises the block).
__device__ inline void plan_block(const PlanCtx &c, int64_t b, int w, PlanBlockLds &S)
{
    const int64_t t = b * kPlanBlockWaves + w;
    const bool active = t < c.sh.n_tiles;
    int64_t r0 = 0, r1 = 0;
    LaneRows q{};
    bool one_round = false;

    // 1. this tile's counts, gathered in LDS
    PlanCounts own{};
    if (active) {
        tile_range(c, t, &r0, &r1);
        one_round = r1 - r0 <= kPlanRoundRows;
        if (one_round) {
            q = lane_rows(c, r0, r1);
#pragma unroll
            for (int k = 0; k < kPlanLaneRows; ++k)
                add_row(own, q.rc[k]);
            own = wave_sum_counts(own);
        } else {
            own = count_tile(c, t);
        }
    }
    if (c.lane == 0) {
#pragma unroll
        for (int k = 0; k < kPlanCounts; ++k)
            S.cnt[k][w] = own.v[k];
    }
    __syncthreads();

    // 2. block totals, this tile's place in the block, the block's place
    int tot[kPlanCounts] = {}, pre[kPlanCounts] = {};
#pragma unroll
    for (int i = 0; i < kPlanBlockWaves; ++i) {
#pragma unroll
        for (int k = 0; k < kPlanCounts; ++k) {
            const int v = S.cnt[k][i];
            tot[k] += v;
            pre[k] += i < w ? v : 0;
        }
    }
    if (w == 0) {
        if (c.lane == 0) {
#pragma unroll
            for (int k = 0; k < kPlanCounts; ++k)
                tag_store(c.pb.agg + k * kPlanMaxBlocks + b, c.epoch, (uint32_t)tot[k]);
        }
        const PlanCounts bp = block_prefix(c, b);
        if (c.lane == 0) {
#pragma unroll
            for (int k = 0; k < kPlanCounts; ++k)
                S.off[k] = bp.v[k];
            if ((b + 1) * kPlanBlockWaves >= c.sh.n_tiles) {
                // last block: the totals of the whole plan
                const int n_med = bp.v[0] + tot[0], n_long = bp.v[1] + tot[1];
                const int n_hub = bp.v[3] + tot[3];
                tag_store(c.pb.counts + 0, c.epoch, (uint32_t)n_med);
                tag_store(c.pb.counts + 1, c.epoch, (uint32_t)n_long);
                tag_store(c.pb.counts + 2, c.epoch, (uint32_t)(bp.v[2] + tot[2]));
                tag_store(c.pb.counts + 3, c.epoch,
                          (uint32_t)(c.M - n_med - n_long - n_hub));
                tag_store(c.pb.counts + 4, c.epoch, (uint32_t)n_hub);
            }
        }
    }
    __syncthreads();
    if (!active)
        return;
    int med_off = S.off[0] + pre[0];
    int long_off = S.off[1] + pre[1];
    int chunk_off = S.off[2] + pre[2];
    int hub_off = S.off[3] + pre[3];
    PlanLds &L = S.wave[w];

    // 3. the tile's entries, a round of kPlanRoundRows rows at a time
    for (int64_t base = r0; base < r1; base += kPlanRoundRows) {
        if (base != r0 || !one_round)
            q = lane_rows(c, base, r1);
        PlanCounts mine{};
#pragma unroll
        for (int k = 0; k < kPlanLaneRows; ++k)
            add_row(mine, q.rc[k]);
        int mpos = wave_excl_scan_i(mine.v[0], c.lane);
        int lpos = wave_excl_scan_i(mine.v[1], c.lane);
        int cpos = wave_excl_scan_i(mine.v[2], c.lane);
        int hpos = wave_excl_scan_i(mine.v[3], c.lane);
        const int round_med = __shfl(mpos + mine.v[0], kWave - 1);
        const int round_long = __shfl(lpos + mine.v[1], kWave - 1);
        const int round_chunks = __shfl(cpos + mine.v[2], kWave - 1);
        const int round_hub = __shfl(hpos + mine.v[3], kWave - 1);
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
            if (q.rc[k].hub)
                L.hub[hpos++] = (int)(rb + k);
        }
        if (round_long > 0 || round_hub > 0) {
            // The C rows of long and hub rows are cleared before their
            // entries are published (the product adds into them).
            if (c.C != nullptr) {
                clear_rows(c, L.row, round_long);
                clear_rows(c, L.hub, round_hub);
            }
            for (int x = c.lane; x < round_long; x += kWave) {
                tag_store(c.pb.long_row + long_off + x, c.epoch, (uint32_t)L.row[x]);
                tag_store(c.pb.long_first + long_off + x, c.epoch,
                          (uint32_t)(chunk_off + L.cfirst[x]));
            }
            for (int x = c.lane; x < round_hub; x += kWave)
                tag_store(hub_slot(c.pb, hub_off + x), c.epoch, (uint32_t)L.hub[x]);
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
        hub_off += round_hub;
    }
}

}  // namespace sdl
