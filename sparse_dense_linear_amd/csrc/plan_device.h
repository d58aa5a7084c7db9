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
// The rows are cut into n_tiles tiles, one wavefront per tile, and the
// tiles are grouped kPlanBlockWaves to a workgroup (a plan block):
//   1. each wavefront counts its tile's medium rows, long rows and chunks;
//      the block adds them up in LDS and publishes the block's totals;
//   2. one wavefront adds up the totals of all earlier blocks; a total that
//      is not visible yet after a few polls is recomputed by this wavefront
//      from rowptr (counting is idempotent), so no workgroup ever waits for
//      another;
//   3. each wavefront writes its tile's entries of the lists (for long
//      rows: clear their C rows, then publish the rows and their chunks);
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

// Counts of plan block b (its kPlanBlockWaves tiles), wave-uniform.
__device__ inline void count_block(const PlanCtx &c, int64_t b, int *med,
                                   int *lng, int *chunks)
{
    int m = 0, l = 0, ch = 0;
    const int64_t t0 = b * kPlanBlockWaves;
    for (int64_t t = t0; t < t0 + kPlanBlockWaves && t < c.sh.n_tiles; ++t) {
        int tm, tl, tc;
        count_tile(c, t, &tm, &tl, &tc);
        m += tm;
        l += tl;
        ch += tc;
    }
    *med = m;
    *lng = l;
    *chunks = ch;
}

// Sums of the published counts of plan blocks 0 .. b-1: lane l reads
// blocks l, l + 64, ... (all loads of a poll in flight together).  Counts
// not visible after a few polls are recomputed here from rowptr.
__device__ inline void block_prefix(const PlanCtx &c, int64_t b, int *med,
                                    int *lng, int *chunks)
{
    int vm = 0, vl = 0, vc = 0;
    if (b > 0) {
        uint32_t need = 0;  // bit i: block lane + 64 i is still to be read
#pragma unroll
        for (int i = 0; i < kPlanPrefixLoads; ++i)
            need |= (c.lane + kWave * i < b) ? 1u << i : 0u;
        for (int poll = 0; poll < kPlanPolls && __ballot(need != 0) != 0; ++poll) {
            if (poll > 0)
                __builtin_amdgcn_s_sleep(2);
            uint64_t wd[kPlanPrefixLoads][3];
#pragma unroll
            for (int i = 0; i < kPlanPrefixLoads; ++i) {
                const int64_t jb = c.lane + kWave * i;
                const int64_t jj = jb < b ? jb : b - 1;
#pragma unroll
                for (int k = 0; k < 3; ++k)
                    wd[i][k] = tag_load(c.pb.agg + k * kPlanMaxBlocks + jj);
            }
#pragma unroll
            for (int i = 0; i < kPlanPrefixLoads; ++i) {
                const bool got = ((need >> i) & 1u) && tag_is(wd[i][0], c.epoch) &&
                                 tag_is(wd[i][1], c.epoch) && tag_is(wd[i][2], c.epoch);
                if (got) {
                    vm += (int)(uint32_t)wd[i][0];
                    vl += (int)(uint32_t)wd[i][1];
                    vc += (int)(uint32_t)wd[i][2];
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
                int m, lg, ch;
                count_block(c, l + (int64_t)kWave * i, &m, &lg, &ch);
                if (c.lane == l) {
                    vm += m;
                    vl += lg;
                    vc += ch;
                }
            }
        }
    }
    *med = wave_sum_i(vm);
    *lng = wave_sum_i(vl);
    *chunks = wave_sum_i(vc);
}

// Block-shared state of the plan kernel.
struct PlanBlockLds {
    PlanLds wave[kPlanBlockWaves];
    int cnt[3][kPlanBlockWaves];   // per tile: medium, long, chunks
    int off[3];                    // offsets of this block in the lists
};

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
    int own_med = 0, own_long = 0, own_chunks = 0;
    if (active) {
        tile_range(c, t, &r0, &r1);
        one_round = r1 - r0 <= kPlanRoundRows;
        if (one_round) {
            q = lane_rows(c, r0, r1);
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
    }
    if (c.lane == 0) {
        S.cnt[0][w] = own_med;
        S.cnt[1][w] = own_long;
        S.cnt[2][w] = own_chunks;
    }
    __syncthreads();

    // 2. block totals, this tile's place in the block, the block's place
    int tot[3] = {0, 0, 0}, pre[3] = {0, 0, 0};
#pragma unroll
    for (int i = 0; i < kPlanBlockWaves; ++i) {
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int v = S.cnt[k][i];
            tot[k] += v;
            pre[k] += i < w ? v : 0;
        }
    }
    if (w == 0) {
        if (c.lane == 0) {
            tag_store(c.pb.agg + b, c.epoch, (uint32_t)tot[0]);
            tag_store(c.pb.agg + kPlanMaxBlocks + b, c.epoch, (uint32_t)tot[1]);
            tag_store(c.pb.agg + 2 * kPlanMaxBlocks + b, c.epoch, (uint32_t)tot[2]);
        }
        int bm, bl, bc;
        block_prefix(c, b, &bm, &bl, &bc);
        if (c.lane == 0) {
            S.off[0] = bm;
            S.off[1] = bl;
            S.off[2] = bc;
            if ((b + 1) * kPlanBlockWaves >= c.sh.n_tiles) {
                // last block: the totals of the whole plan
                const int n_med = bm + tot[0], n_long = bl + tot[1];
                tag_store(c.pb.counts + 0, c.epoch, (uint32_t)n_med);
                tag_store(c.pb.counts + 1, c.epoch, (uint32_t)n_long);
                tag_store(c.pb.counts + 2, c.epoch, (uint32_t)(bc + tot[2]));
                tag_store(c.pb.counts + 3, c.epoch, (uint32_t)(c.M - n_med - n_long));
            }
        }
    }
    __syncthreads();
    if (!active)
        return;
    int med_off = S.off[0] + pre[0];
    int long_off = S.off[1] + pre[1];
    int chunk_off = S.off[2] + pre[2];
    PlanLds &L = S.wave[w];

    // 3. the tile's entries, a round of kPlanRoundRows rows at a time
    for (int64_t base = r0; base < r1; base += kPlanRoundRows) {
        if (base != r0 || !one_round)
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
            // The product (same launch) adds into these rows with device
            // atomics as soon as their chunks are published, so the zeros
            // must have reached device scope first: they are written as
            // device-coherent atomic stores, and the chunk entries are
            // published only after those stores have completed.
            if (c.C != nullptr) {
                for (int x = 0; x < round_long; ++x) {
                    float *crow = c.C + (int64_t)L.row[x] * c.N;
                    for (int64_t n = c.lane; n < c.N; n += kWave)
                        __hip_atomic_store(crow + n, 0.0f, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                }
                wait_stores_done();
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
