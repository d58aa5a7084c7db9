// worker_impl.h -- gather-scale-accumulate kernels of the CSR sparse x dense
// product C = A * B on gfx950 (templates; each worker_*.hip file
// instantiates a share of the variants, so they compile in parallel).
//
// Pages:
//   [IntelMax] "Performance Optimization of Deep Learning Sparse Matrix
//              Kernels on Intel Max Series GPU": the SpMM operation (Fig. 5,
//              Algorithm 2) -- per stored entry, scale a gathered row of B and
//              add it to the output row (a SAXPY) -- and its ESIMD kernel
//              (Figs. 9-10): a chunk of column indices and values is loaded
//              once, the next chunk is prefetched, the inner loop unrolled.
//   [Sgap]     "Sgap: Towards Efficient Sparse Tensor Algebra Compilation for
//              GPU": atomic parallelism <row|nnz, col> with reduction
//              parallelism r; row-balanced and element-balanced points with
//              a coarsened column factor; zero extension (lanes past the end
//              of a row contribute zeros to the group reduction); grouped
//              atomic adds; and the prior-work survey (Ge-SpMM's coalesced
//              row caching: a sparse row chunk staged in fast memory and
//              reused across the dense columns).
//
// Execution model (one wavefront = 64 lanes):
//   * Lanes form R = 64/G groups of G lanes.  Within a group, lane j covers
//     the B/C columns (k*G + j)*VEC .. +VEC-1 for k < NV, so every gathered
//     row of B is read, and every row of C written, as contiguous 16-byte
//     vectors across the group.
//   * colind/vals of the entries being worked on are loaded once with
//     coalesced loads, one entry per lane, and reach the lanes that cover
//     the N columns from there: by lane shuffles for a medium row or chunk,
//     through LDS (staged with their rows) for a short tile.
//   * One launch per call: the first workgroups compute the plan
//     (plan_device.h) while the others start on short tiles; then every
//     wavefront takes items from 64 work queues (see call_kernel).  Four
//     kinds of work item:
//       hub chunk   the entries of a hub row (the longest rows) whose
//                   columns fall in one slab of B's rows; each XCD takes the
//                   chunks of its own range of slabs, slab after slab, so
//                   they gather from its L2; added into C with atomics;
//       long chunk  (row, p0, p1) from the plan: the R groups split the
//                   chunk's entries, their partial rows are summed by
//                   butterfly shuffles, and group 0 adds the result to C
//                   with fp32 atomics (the row was cleared by the plan);
//       medium row  from the plan: as a chunk over the whole row, but the
//                   result is stored, not added;
//       short tile  a block of T consecutive rows in natural order.  The
//                   entries of its short rows are staged in LDS in one round
//                   (column, value and the row they belong to); each group
//                   then streams the entries of its own P consecutive rows in
//                   batches of U gathers that run across row boundaries,
//                   storing a row of C when its last entry is consumed (one
//                   row per group at a time: RB with coarsened columns).
//                   Rows that are not short are skipped: they belong to the
//                   other two kinds.
//   * Within an item, U gathers per lane are issued back to back before any
//     of them is consumed.
//   * FusedMM form (Shape::FUSED; [IntelMax] FusedMM operation, Fig. 6,
//     Algorithm 3): the same items, with each entry's value formed by its
//     lane group as <X_i, Y_j> where it is used instead of read from vals.
#pragma once

#include <hip/hip_ext.h>

#include <atomic>

#include "gather.h"
#include "internal.h"
#include "plan_device.h"
#include "spmm.h"

namespace sdl {
namespace {

// One wavefront accumulates positions [p0, p1) (p1 > p0) of one row: 64-entry
// chunks of colind/vals are loaded coalesced, one entry per lane (the next
// chunk prefetched into registers while the current one is consumed), and
// group g consumes entries g*G .. g*G+G-1 of each chunk, reading them from
// the lanes that hold them.  FusedMM: the values are formed from row `row`
// of X (held by each lane for its columns) and the entries' rows of Y.
template <class S>
__device__ inline void wave_range(const WorkerArgs &a, int lane, int g,
                                  int64_t row, int64_t p0, int64_t p1,
                                  const BSrc &src, const BSrc &ysrc,
                                  const LaneCols<S> &lc, uint32_t row_bytes,
                                  float (&acc)[S::NV][S::VEC])
{
    zero_acc<S>(acc);
    typename BLoad<S::DT, S::VEC>::raw x[S::NV];
    if constexpr (S::FUSED)
        load_x_row<S>((const char *)a.dot_rows, row, row_bytes, lc, x);
    // positions past the range read the range's last entry (valid address)
    int64_t p = p0 + lane < p1 ? p0 + lane : p1 - 1;
    int32_t nc = a.colind[p];
    float nvv = 0.0f;
    if constexpr (!S::FUSED)
        nvv = load_val<S::DT>(a.vals, p);
    for (int64_t base = p0; base < p1; base += kWave) {
        const int n = p1 - base < kWave ? (int)(p1 - base) : kWave;
        const int32_t col = nc;
        const float val = nvv;
        const int64_t nb = base + kWave;
        if (nb < p1) {
            p = nb + lane < p1 ? nb + lane : p1 - 1;
            nc = a.colind[p];
            if constexpr (!S::FUSED)
                nvv = load_val<S::DT>(a.vals, p);
        }
        int cnt = n - g * S::G;
        cnt = cnt < 0 ? 0 : (cnt > S::G ? S::G : cnt);
        if constexpr (S::FUSED)
            consume_lanes_fused<S>(col, g * S::G, cnt, src, ysrc, row_bytes, lc, x, acc);
        else
            consume_lanes<S>(col, val, g * S::G, cnt, src, row_bytes, lc, acc);
    }
}

// Row and position range of chunk ci if its plan entries are published:
// from the chunk table, or past its end from the long-row list (binary
// search for the last long row whose first chunk is <= ci).  Never waits.
__device__ inline bool chunk_ready(const WorkerArgs &a, int64_t ci,
                                   int64_t n_long, int64_t *row, int64_t *p0,
                                   int64_t *p1)
{
    uint64_t wr, wk;
    if (ci < a.plan.chunk_cap) {
        wr = __shfl(tag_load(a.plan.chunk_row + ci), 0);
        wk = __shfl(tag_load(a.plan.chunk_k + ci), 0);
        if (!tag_is(wr, a.epoch) || !tag_is(wk, a.epoch))
            return false;
    } else {
        int64_t lo = 0, hi = n_long - 1;
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) >> 1;
            const uint64_t wf = __shfl(tag_load(a.plan.long_first + mid), 0);
            if (!tag_is(wf, a.epoch))
                return false;
            if ((int64_t)(uint32_t)wf <= ci)
                lo = mid;
            else
                hi = mid - 1;
        }
        wr = __shfl(tag_load(a.plan.long_row + lo), 0);
        const uint64_t wf = __shfl(tag_load(a.plan.long_first + lo), 0);
        if (!tag_is(wr, a.epoch) || !tag_is(wf, a.epoch))
            return false;
        wk = (uint64_t)(ci - (int64_t)(uint32_t)wf);
    }
    const int64_t r = (uint32_t)wr;
    const int64_t start = a.rowptr[r];
    const int64_t len = (int64_t)a.rowptr[r + 1] - start;
    const int64_t n = (len + a.th.chunk_nnz - 1) / a.th.chunk_nnz;
    chunk_bounds(start, len, n, (int64_t)(uint32_t)wk, p0, p1);
    *row = r;
    return true;
}

// Row of medium item i if published.  Never waits.
__device__ inline bool medium_ready(const WorkerArgs &a, int64_t i, int64_t *row)
{
    const uint64_t w = __shfl(tag_load(a.plan.medium_rows + i), 0);
    if (!tag_is(w, a.epoch))
        return false;
    *row = (uint32_t)w;
    return true;
}


// Add one column pass of a row's partial sums into C with device atomics.
// After reduce_groups every group holds the sums; group 0 lays each of its
// vectors out in the wavefront's LDS area in column order, and then all 64
// lanes add 64 consecutive floats per instruction, so each atomic
// instruction covers whole 256-byte spans of the row (adding straight from
// the lanes' vectors would touch one float per 16 bytes per instruction and
// send every float to memory in a separate sector).
template <class S>
__device__ inline void add_row_atomic(WaveStage &ws, float *C, int64_t row,
                                      int64_t N, int64_t col0, int g, int j,
                                      int lane, const float (&acc)[S::NV][S::VEC])
{
    float *f = reinterpret_cast<float *>(ws.ent);   // G * VEC <= 512 floats
    float *crow = C + row * N + col0;
    const int64_t left = N - col0;                  // columns of the pass
#pragma unroll
    for (int k = 0; k < S::NV; ++k) {
        const int64_t cbase = (int64_t)k * S::G * S::VEC;   // vector k's columns
        if (cbase >= left)
            break;
        __builtin_amdgcn_wave_barrier();   // earlier reads of the area are done
        if (g == 0) {
#pragma unroll
            for (int x = 0; x < S::VEC; ++x)
                f[j * S::VEC + x] = acc[k][x];
        }
        __builtin_amdgcn_wave_barrier();   // the vectors are in place
        for (int c = lane; c < S::G * S::VEC; c += kWave)
            if (cbase + c < left)
                unsafeAtomicAdd(crow + cbase + c, f[c]);
    }
    __builtin_amdgcn_wave_barrier();
}

// One wavefront accumulates row `row` over positions [p0, p1) and stores
// (medium row) or atomically adds (long-row or hub chunk) the result.
template <class S, bool ATOMIC>
__device__ void do_range(const WorkerArgs &a, WaveStage &ws, int lane, int g,
                         int j, int64_t row, int64_t p0, int64_t p1,
                         const BSrc &src, const BSrc &ysrc, uint32_t row_bytes)
{
    for (int64_t col0 = 0; col0 < a.N; col0 += S::COLS) {
        const LaneCols<S> lc = lane_cols<S>(a.N, col0, j);
        float acc[S::NV][S::VEC];
        wave_range<S>(a, lane, g, row, p0, p1, src, ysrc, lc, row_bytes, acc);
        reduce_groups<S>(acc);
        if constexpr (ATOMIC)
            add_row_atomic<S>(ws, a.C, row, a.N, col0, g, j, lane, acc);
        else if (g == 0)
            emit_row<S, false>(a.C, row, a.N, col0, j, acc);
    }
}

// FusedMM form of issue() for a short tile: for each of the U staged
// entries (slots past n repeat entry q) the gathers of Y_j and D_j and the
// load of this lane's slice of X_i (rows are consecutive, so these mostly hit
// the cache) are issued first; then each entry's value <X_i, Y_j> is formed
// and the D_j vectors go into bt as the rows to accumulate.
template <class S>
__device__ inline void issue_fused(Batch<S> &bt, const WaveStage &ws,
                                   const WorkerArgs &a, int64_t r0, int q,
                                   int n, const BSrc &dsrc, const BSrc &ysrc,
                                   uint32_t row_bytes, const LaneCols<S> &lc)
{
    typedef BLoad<S::DT, S::VEC> L;
    typename L::raw yb[S::U][S::NV], xb[S::U][S::NV];
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
        const int e = u < n ? q + u : q;
        const int32_t c = ws.ent[e].col;
        const char *xrow = (const char *)a.dot_rows + (uint64_t)(r0 + ws.rid[e]) * row_bytes;
#pragma unroll
        for (int k = 0; k < S::NV; ++k) {
            yb[u][k] = load_row_vec<S>(ysrc, c, row_bytes, lc, k);
            xb[u][k] = L::load(xrow + lc.ofs[k]);
            bt.buf[u][k] = load_row_vec<S>(dsrc, c, row_bytes, lc, k);
        }
    }
#pragma unroll
    for (int u = 0; u < S::U; ++u)
        bt.v[u] = group_dot<S>(xb[u], yb[u], lc);
}

// One short tile: rows r0 .. r0+T-1 with T = P*R; group g owns rows
// g*P .. g*P+P-1 of the tile.
template <class S>
__device__ void do_short_tile(const WorkerArgs &a, WaveStage &ws, int lane,
                              int g, int j, int64_t r0, int P,
                              const BSrc &src, const BSrc &ysrc,
                              uint32_t row_bytes)
{
    const int T = P * S::R;
    const int64_t r = r0 + lane;
    const bool in_tile = lane < T && r < a.M;
    int32_t s = 0, len = 0;
    if (in_tile) {
        s = a.rowptr[r];
        len = a.rowptr[r + 1] - s;
    }
    const bool shrt = in_tile && len <= a.th.short_max;
    const int slen = shrt ? len : 0;
    const int off = wave_exclusive_sum(slen);

    // Stage the tile's short entries, flattened in row order: entry e goes
    // to lane e % 64.  The lane finds the row holding e (the last lane l with
    // off_l <= e; such a lane has slen_l > 0) by a binary search over the
    // lanes' offsets, so each round is one coalesced load per lane however
    // the entries are spread over rows.
    const int total = __shfl(off + slen, kWave - 1);
    // All loads first (slot i holds entry i*64 + lane), then the LDS
    // stores, so the whole tile is staged in one memory round trip.
    int scol[kStageSlots];
    float sval[kStageSlots];
    int srow[kStageSlots];
#pragma unroll
    for (int i = 0; i < kStageSlots; ++i) {
        if (i * kWave < total) {  // wave-uniform
            const int e = i * kWave + lane < total ? i * kWave + lane : total - 1;
            int l = 0;
#pragma unroll
            for (int step = kWave / 2; step > 0; step >>= 1) {
                const int cand = l + step;
                if (__shfl(off, cand) <= e)
                    l = cand;
            }
            const int64_t p = (int64_t)__shfl(s, l) + (e - __shfl(off, l));
            scol[i] = a.colind[p];
            sval[i] = S::FUSED ? 0.0f : load_val<S::DT>(a.vals, p);
            srow[i] = l;
        }
    }
    // every lane has read the previous tile's entries
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < kStageSlots; ++i) {
        const int e = i * kWave + lane;
        if (i * kWave < total && e < total) {
            Entry en;
            en.col = scol[i];
            en.val = sval[i];
            ws.ent[e] = en;
            ws.rid[e] = (uint8_t)srow[i];
        }
    }
    // the tile is staged before any lane reads it
    __builtin_amdgcn_wave_barrier();

    const int first = g * P;
    const int beg = __shfl(off, first);
    const int end = __shfl(off + slen, first + P - 1);
    const int empty = (shrt && len == 0) ? 1 : 0;

    for (int64_t col0 = 0; col0 < a.N; col0 += S::COLS) {
        const LaneCols<S> lc = lane_cols<S>(a.N, col0, j);
        // Empty short rows are rows of zeros.
        for (int q = 0; q < P; ++q) {
            if (__shfl(empty, first + q)) {
                float z[S::NV][S::VEC];
                zero_acc<S>(z);
                emit_row<S, false>(a.C, r0 + first + q, a.N, col0, j, z);
            }
        }
        float acc[S::NV][S::VEC];
        zero_acc<S>(acc);
        for (int q = beg; q < end; q += S::U) {
            const int n = end - q < S::U ? end - q : S::U;
            Batch<S> bt;
            if constexpr (S::FUSED)
                issue_fused<S>(bt, ws, a, r0, q, n, src, ysrc, row_bytes, lc);
            else
                issue<S>(bt, ws.ent, q, n, src, row_bytes, lc);
#pragma unroll
            for (int u = 0; u < S::U; ++u) {
                accumulate<S>(bt, u, u < n, acc);
                if (u < n) {
                    const int rr = ws.rid[q + u];
                    if (q + u + 1 == end || ws.rid[q + u + 1] != rr) {
                        emit_row<S, false>(a.C, r0 + rr, a.N, col0, j, acc);
                        zero_acc<S>(acc);
                    }
                }
            }
        }
    }
}

// Workgroups are handed to the 8 XCDs round-robin (block b runs on XCD
// b % 8).  Renumber them so each XCD holds a contiguous range of logical
// blocks, and so neighbouring work items share an L2.
__device__ inline int64_t xcd_logical_block(int64_t b, int64_t nb)
{
    const int64_t per = nb / 8, rem = nb % 8;
    const int64_t x = b % 8, k = b / 8;
    return x * per + (x < rem ? x : rem) + k;
}

// Plan totals if this call's have been published (no waiting).
__device__ inline bool counts_ready(const WorkerArgs &a, int64_t *n_med,
                                    int64_t *n_long, int64_t *n_ch, int64_t *n_hub)
{
    const uint64_t w0 = __shfl(tag_load(a.plan.counts + 0), 0);
    const uint64_t w1 = __shfl(tag_load(a.plan.counts + 1), 0);
    const uint64_t w2 = __shfl(tag_load(a.plan.counts + 2), 0);
    const uint64_t w4 = __shfl(tag_load(a.plan.counts + 4), 0);
    if (!tag_is(w0, a.epoch) || !tag_is(w1, a.epoch) || !tag_is(w2, a.epoch) ||
        !tag_is(w4, a.epoch))
        return false;
    *n_med = (uint32_t)w0;
    *n_long = (uint32_t)w1;
    *n_ch = (uint32_t)w2;
    *n_hub = (uint32_t)w4;
    return true;
}

// Row of hub l if published.  Never waits.
__device__ inline bool hub_ready(const WorkerArgs &a, int64_t l, int64_t *row)
{
    const uint64_t w = __shfl(tag_load(hub_slot(a.plan, l)), 0);
    if (!tag_is(w, a.epoch))
        return false;
    *row = (uint32_t)w;
    return true;
}

// PAIR form items: medium rows 4u .. 4u+3 of the list, one row per 16-lane
// group.  Whether all of the item's plan words are published, and this
// lane's group's row (-1 past the end of the list).  Never waits.
struct PairItemRow {
    bool ok;
    int64_t row;   // this lane's group's row, -1 past the list
};
__device__ inline PairItemRow medium_item_ready(const WorkerArgs &a, int64_t u,
                                                int64_t n_med, int lane, int g)
{
    const int64_t m = 4 * u + (lane & 3);
    const uint64_t w = (lane < 4 && m < n_med) ? tag_load(a.plan.medium_rows + m) : 0;
    bool ok = true;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint64_t wt = __shfl(w, t);
        if (4 * u + t < n_med && !tag_is(wt, a.epoch))
            ok = false;
    }
    const uint64_t wg = __shfl(w, g);
    PairItemRow q;
    q.ok = ok;
    q.row = 4 * u + g < n_med ? (int64_t)(uint32_t)wg : -1;
    return q;
}

// One PAIR form item: group g accumulates its row over the column pass
// starting at col0 (its entries 16 at a time, one per lane of the group, read
// by shuffles within the group) and stores it.  Four rows per item instead
// of two (each then split over two groups) measured 6.43 -> 6.12 ms on the
// banded workload (A/B, one box): the item's plan words, row bounds and
// first entries are one round of loads for four rows.
template <class S>
__device__ void do_pair_item(const WorkerArgs &a, int g, int j, int64_t row, int64_t col0,
                             const BSrc &src, uint32_t row_bytes)
{
    static_assert(S::PAIR && S::R == 4 && S::NV == 1 && !S::FUSED, "PAIR shapes only");
    const bool has = row >= 0;
    int64_t p0 = 0, p1 = 0;
    if (has) {
        p0 = a.rowptr[row];
        p1 = a.rowptr[row + 1];
    }
    const int len = (int)(p1 - p0);
    int longest = len;
    longest = max(longest, __shfl_xor(longest, 16));
    longest = max(longest, __shfl_xor(longest, 32));
    const int n_chunks = (longest + S::G - 1) / S::G;
    const LaneCols<S> lc = lane_cols<S>(a.N, col0, j);
    float acc[S::NV][S::VEC];
    zero_acc<S>(acc);
    int32_t nc = 0;
    float nvv = 0.0f;
    if (has) {
        const int64_t p = p0 + j < p1 ? p0 + j : p1 - 1;
        nc = a.colind[p];
        nvv = load_val<S::DT>(a.vals, p);
    }
    for (int c = 0; c < n_chunks; ++c) {
        const int32_t col = nc;
        const float val = nvv;
        if (c + 1 < n_chunks && has) {
            const int64_t p = p0 + (int64_t)(c + 1) * S::G + j;
            const int64_t q = p < p1 ? p : p1 - 1;
            nc = a.colind[q];
            nvv = load_val<S::DT>(a.vals, q);
        }
        int cnt = len - c * S::G;
        cnt = cnt < 0 ? 0 : (cnt > S::G ? S::G : cnt);
        consume_lanes<S>(col, val, g * S::G, cnt, src, row_bytes, lc, acc);
    }
    if (has)
        emit_row<S, false>(a.C, row, a.N, col0, j, acc);
}

// Polls for a plan word, at most `polls` times.  The plan blocks are the
// first workgroups of the launch, each XCD starts its workgroups in order,
// and a plan block never waits, so the plan is running (and finishes)
// whenever a product wavefront runs; the bound (kWaitPolls, about a
// second) only guarantees that every wavefront exits.
template <class Ready>
__device__ inline bool wait_for(int32_t polls, Ready ready)
{
    for (int32_t i = 0; i < polls; ++i) {
        if (ready())
            return true;
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

// An item whose plan entry never became visible is left undone and counted.
__device__ inline void note_fault(const WorkerArgs &a, int lane)
{
    if (lane == 0)
        atomicAdd(a.plan.faults, 1u);
}

// How the product's work is cut, fixed by the host for one launch.
struct ProductShape {
    int passes;            // P of the static short tiles (T = P*R rows)
    int dyn_passes;        // P of the short tiles handed out by the queues
    int64_t first;         // static short tiles (one per product wavefront)
    int64_t rows_static;   // rows [0, rows_static) are in static tiles
    int64_t n_dyn_tiles;   // short tiles over rows [rows_static, M)
    int64_t plan_blocks;   // workgroups that compute the plan
    int64_t plan_grid;     // plan_blocks rounded up to a multiple of 8
    int64_t static_waves;  // product wavefronts
};

// One queued item: [0, n_ch) long-row chunks (the heaviest items first),
// then, for the product, the short tiles after the static ones and last the
// medium rows; for FusedMM medium rows before short tiles.  Ending on medium
// rows (one wavefront per row, every gather slot busy) drains the queues
// faster than ending on short tiles (a few rows per lane group, batches
// part empty): measured 6 % faster on the power-law workload; FusedMM,
// with two gathers per entry, measured the other way.
template <class S>
__device__ inline void do_item(const WorkerArgs &a, const ProductShape &ps,
                               WaveStage &ws, int lane, int g, int j,
                               int64_t d, int64_t n_ch, int64_t n_med,
                               int64_t n_long, const BSrc &src,
                               const BSrc &ysrc, uint32_t row_bytes)
{
    int64_t row = 0, p0 = 0, p1 = 0;
    if (d < n_ch) {
        // The row was cleared (device-coherent stores, completed) before its
        // chunk was published; the atomic adds address it through the
        // published row, so they come after the clearing.
        if (wait_for(a.wait_polls, [&]() { return chunk_ready(a, d, n_long, &row, &p0, &p1); }))
            do_range<S, true>(a, ws, lane, g, j, row, p0, p1, src, ysrc, row_bytes);
        else
            note_fault(a, lane);
    } else {
        // medium rows, then short tiles (FusedMM); short tiles, then medium
        // rows (product)
        const int64_t e = d - n_ch;
        const int64_t m = S::FUSED ? e : e - ps.n_dyn_tiles;
        if (m >= 0 && m < n_med) {
            if (wait_for(a.wait_polls, [&]() { return medium_ready(a, m, &row); }))
                do_range<S, false>(a, ws, lane, g, j, row, a.rowptr[row],
                                   a.rowptr[row + 1], src, ysrc, row_bytes);
            else
                note_fault(a, lane);
        } else {
            const int64_t t = S::FUSED ? e - n_med : e;
            do_short_tile<S>(a, ws, lane, g, j,
                             ps.rows_static + t * (int64_t)(ps.dyn_passes * S::R),
                             ps.dyn_passes, src, ysrc, row_bytes);
        }
    }
}

// Hub chunk c = s * n_hub + l: the entries of hub row l whose columns lie
// in slab s, [s * slab_rows, (s + 1) * slab_rows) -- found by slab_bounds
// on the row's columns -- added into the row (cleared by the plan) with
// atomics.  Hub chunks of neighbouring slabs go to the same XCD (see
// call_kernel), so the rows of B one slab holds are gathered from that
// XCD's L2 by all the hubs' chunks of the slab.
template <class S>
__device__ inline void do_hub(const WorkerArgs &a, WaveStage &ws, int lane,
                              int g, int j, int64_t c, int64_t n_hub,
                              const BSrc &src, const BSrc &ysrc, uint32_t row_bytes)
{
    const int64_t s = c / n_hub, l = c - s * n_hub;
    int64_t row = 0;
    if (!wait_for(a.wait_polls, [&]() { return hub_ready(a, l, &row); })) {
        note_fault(a, lane);
        return;
    }
    const int64_t start = a.rowptr[row], end = a.rowptr[row + 1];
    const int64_t ns = a.th.n_slabs;
    const int64_t t0 = s * (int64_t)a.th.slab_rows, t1 = t0 + a.th.slab_rows;
    int64_t p0, p1;
    slab_bounds(a.colind, start, end, (int32_t)(t0 < INT32_MAX ? t0 : INT32_MAX),
                (int32_t)(t1 < INT32_MAX ? t1 : INT32_MAX), &p0, &p1);
    if (s == 0)
        p0 = start;
    if (s + 1 >= ns)
        p1 = end;
    if (p1 > p0)
        do_range<S, true>(a, ws, lane, g, j, row, p0, p1, src, ysrc, row_bytes);
}

// Workgroups beyond the first kSmallJobBlocks product workgroups leave at
// once when the whole call gathers less than kSmallJobBytes (nnz * N *
// element size): the uniform 1024-row workload (2 MB) took 9.5 -> 7.3 us
// per launch (same box).  The launch keeps its full size, so that a matrix
// of few but long rows still gets the whole GPU.
constexpr int64_t kSmallJobBlocks = 64;
constexpr int64_t kSmallJobBytes = (int64_t)16 << 20;

// Items per wavefront of a queue above which the next grab overlaps the
// current item.  Measured (A/B on one box): the pruned 4096-row matrices,
// about one medium row per wavefront, 88 -> 77 us (fp32) and 76 -> 58 us
// (bf16) without the early grab; power-law (about 4 items per wavefront)
// 58.0 -> 56.2 us and FusedMM 107.3 -> 105.2 us; the banded matrix (about
// 1000 per wavefront) 2.7 % slower without it, so it keeps it.
constexpr int64_t kGrabAheadItems = 16;

// One launch per call, sized to the workgroups that fit at once.
// Workgroups [0, plan_blocks) first compute the plan (plan_device.h);
// [plan_blocks, plan_grid) pad that part to a multiple of the 8 XCDs.
// Product workgroups (the rest) start with one short tile each (static:
// logical product wavefront w takes tile w, for w < first), which needs no
// plan.  Then every wavefront, the planners included, takes the remaining
// items from kQueues work queues: queue q first hands out its XCD's hub
// chunks (see below), then items q, q + kQueues, ... of the list
// [long-row chunks | short tiles | medium rows], so every queue holds the
// same mix, and a wavefront that started late or drew slow items simply
// takes fewer.
template <class S>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(S::MIN_WAVES)))
void call_kernel(WorkerArgs a, ProductShape ps)
{
    if (a.vals_relative)  // entry p's value sits at vals[p - rowptr[0]]
        a.vals = (const char *)a.vals - (int64_t)a.rowptr[0] * S::ESZ;
    __shared__ union {
        WaveStage stage[kWavesPerBlock];
        PlanBlockLds plan;
    } lds;
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wid;
    const bool planner = (int64_t)blockIdx.x < ps.plan_grid;
    if (planner) {
        if ((int64_t)blockIdx.x < ps.plan_blocks) {
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
            plan_block(pc, blockIdx.x, wid, lds.plan);
        }
        // Clear the queue counters of the next epoch on this stream (the
        // call before this one, which used them, has ended).  Every call
        // that takes an epoch does this, the element-balanced kernel too, so
        // a product call always finds its set cleared.
        if (blockIdx.x == 0 && wid == 0)
            for (int q = lane; q < kQueues; q += kWave)
                a.plan.queues[((a.epoch + 1) & 1) * kQueues * kQueueStride +
                              q * kQueueStride] = 0;
        __syncthreads();  // the block's LDS now serves the product
    }
    // Values read from an array of vals_count entries (the SDDMM values of
    // FusedMM's two-launch route): a pattern with more stored entries than
    // that (an nnz below rowptr[M] - rowptr[0]) is refused before any value
    // is read, and counted as a fault.
    if (a.vals_relative && (int64_t)a.rowptr[a.M] - a.rowptr[0] > a.vals_count) {
        note_fault(a, lane);
        return;
    }

    const int g = lane / S::G;
    const int j = lane % S::G;
    WaveStage &ws = lds.stage[wid];
    const uint32_t row_bytes = (uint32_t)(a.N * S::ESZ);
    BSrc src;
    src.base = (const char *)a.B;
    if constexpr (S::BUF)
        src.rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<void *>(a.B), (short)0,
            (int)(uint32_t)(a.K * a.N * S::ESZ), kBufferWord3);
    // FusedMM: Y (K x N, like B) is gathered the same way.
    BSrc ysrc = src;
    if constexpr (S::FUSED) {
        ysrc.base = (const char *)a.dot_cols;
        if constexpr (S::BUF)
            ysrc.rsrc = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<void *>(a.dot_cols), (short)0,
                (int)(uint32_t)(a.K * a.N * S::ESZ), kBufferWord3);
    }

    if (!planner) {
        // plan_grid is a multiple of 8, so product block b runs on XCD b % 8
        const int64_t w = xcd_logical_block((int64_t)blockIdx.x - ps.plan_grid,
                                            (int64_t)gridDim.x - ps.plan_grid) *
                              kWavesPerBlock + wid;
        if (w < ps.first) {
            do_short_tile<S>(a, ws, lane, g, j, w * (int64_t)(ps.passes * S::R),
                             ps.passes, src, ysrc, row_bytes);
        } else if ((int64_t)blockIdx.x >= ps.plan_grid + kSmallJobBlocks &&
                   ((int64_t)a.rowptr[a.M] - a.rowptr[0]) * a.N * S::ESZ < kSmallJobBytes) {
            // A small job (a few MB of gathers in all) needs no more than the
            // first kSmallJobBlocks product workgroups (with every workgroup
            // of the plan they cover all kQueues queues): the others leave
            // at once instead of waiting for the plan to find nothing to do.
            return;
        }
    }

    int64_t n_med = 0, n_long = 0, n_ch = 0, n_hub = 0;
    if (!wait_for(a.wait_polls, [&]() { return counts_ready(a, &n_med, &n_long, &n_ch, &n_hub); })) {
        note_fault(a, lane);
        n_med = n_long = n_ch = n_hub = 0;
    }
    // PAIR form: medium rows leave the shared list for the PAIR items below
    const int64_t n_med_list = S::PAIR ? 0 : n_med;
    const int64_t n_dyn = n_ch + n_med_list + ps.n_dyn_tiles;
    // One item per grab: consecutive items go to different wavefronts at
    // about the same time, so the whole GPU sweeps the item list in order
    // (rows that share columns of B, as in banded matrices, are gathered
    // together).  Grabs are device atomics on kQueues counters.
    const int64_t q = gw % kQueues;
    uint32_t *ctr = a.plan.queues + ((a.epoch & 1) * kQueues + q) * kQueueStride;
    // Hub chunks come first and stay on one XCD per slab range: the waves
    // of queue q belong to blocks q/4 mod 16, which run on XCD x = (q/4) mod
    // 8 (blocks go to the XCDs round-robin), and XCD x's 8 queues (index k)
    // hand out the hub chunks of slabs [x*ns/8, (x+1)*ns/8) slab by slab:
    // chunk s_lo*n_hub + k + 8i is the queue's i-th.  So each XCD sweeps its
    // own eighth of B's rows, one slab at a time, for all hubs.
    const int64_t ns = a.th.n_slabs;
    const int x = (int)((q >> 2) & 7);
    const int k = (int)(((q >> 5) << 2) | (q & 3));
    const int64_t s_lo = (int64_t)x * ns / 8, s_hi = (int64_t)(x + 1) * ns / 8;
    const int64_t hub_base = s_lo * n_hub + k;
    const int64_t n_xh = (s_hi - s_lo) * n_hub;          // the XCD's hub chunks
    const int64_t n_qh = n_xh > k ? (n_xh - k + 7) / 8 : 0;  // this queue's
    // A call whose every item was a static tile grabs nothing (the uniform
    // 1024-row workload).
    if (n_hub == 0 && n_med == 0 && n_dyn == 0)
        return;
    // Lane 0 holds the next grabbed index; it is read (and waited for) only
    // at the top of the next round, so the grab overlaps the current item.
    uint32_t next = 0;
    if (lane == 0)
        next = atomicAdd(ctr, 1u);
    int64_t i = __builtin_amdgcn_readfirstlane(next);
    while (i < n_qh) {
        if (lane == 0)
            next = atomicAdd(ctr, 1u);
        do_hub<S>(a, ws, lane, g, j, hub_base + 8 * i, n_hub, src, ysrc, row_bytes);
        i = __builtin_amdgcn_readfirstlane(next);
    }
    // PAIR form: then the medium rows, four consecutive ones per item and
    // one column half per item.  XCDs 0-3 take the first half of B's
    // columns and XCDs 4-7 the second, each XCD a contiguous quarter of the
    // items in row order (its 8 queues interleaved), so the rows of B that
    // neighbouring rows gather (a band) are read from that XCD's L2 at half
    // the width: a window of B rows twice as tall fits it.
    int64_t n_qp = 0;
    if constexpr (S::PAIR) {
        const int64_t n_items = (n_med + 3) / 4;   // four rows each
        const int64_t u_lo = (int64_t)(x & 3) * n_items / 4;
        const int64_t u_hi = (int64_t)((x & 3) + 1) * n_items / 4;
        n_qp = u_hi - u_lo > k ? (u_hi - u_lo - k + 7) / 8 : 0;
        const int64_t col0 = (int64_t)(x >> 2) * S::COLS;
        const bool pahead =
            n_qp > kGrabAheadItems * ((int64_t)gridDim.x * kWavesPerBlock / kQueues);
        while (i - n_qh < n_qp) {
            const int64_t u = u_lo + k + 8 * (i - n_qh);
            if (pahead && lane == 0)
                next = atomicAdd(ctr, 1u);
            PairItemRow ir;
            ir.ok = false;
            ir.row = -1;
            if (wait_for(a.wait_polls, [&]() {
                    ir = medium_item_ready(a, u, n_med, lane, g);
                    return ir.ok;
                }))
                do_pair_item<S>(a, g, j, ir.row, col0, src, row_bytes);
            else
                note_fault(a, lane);
            if (!pahead && lane == 0)
                next = atomicAdd(ctr, 1u);
            i = __builtin_amdgcn_readfirstlane(next);
        }
    }
    // then queue q hands out items q, q + kQueues, ... of the rest.  The
    // next grab is issued before the current item only when the queue holds
    // many items per wavefront (then its latency would recur item after
    // item); with few, a grab made early reserves an item that no idle
    // wavefront may take, and the first wavefronts to arrive take two items
    // each while later ones find the queue empty.
    int64_t d = q + (int64_t)kQueues * (i - n_qh - n_qp);
    const int64_t n_q = n_dyn > q ? (n_dyn - q + kQueues - 1) / kQueues : 0;
    const bool ahead =
        n_q > kGrabAheadItems * ((int64_t)gridDim.x * kWavesPerBlock / kQueues);
    while (d < n_dyn) {
        if (ahead && lane == 0)
            next = atomicAdd(ctr, 1u);
        do_item<S>(a, ps, ws, lane, g, j, d, n_ch, n_med_list, n_long, src, ysrc, row_bytes);
        if (!ahead && lane == 0)
            next = atomicAdd(ctr, 1u);
        d = q + (int64_t)kQueues *
                ((int64_t)__builtin_amdgcn_readfirstlane(next) - n_qh - n_qp);
    }
}

// Short tiles handed out by the queues hold 1/kDynTileDiv of the rows of
// the static ones (at least R rows).  Measured on the power-law workload:
// 2 for the product (1 and 4 are 3-5 % slower), 4 for FusedMM (3 % faster
// than 2; its tiles are last in the queues).
template <class S>
constexpr int kDynTileDiv = S::FUSED ? 4 : 2;

template <class S>
hipError_t launch_shape(const WorkerArgs &a, hipStream_t stream,
                        hipEvent_t start, hipEvent_t stop)
{
    // Workgroups of this variant that fit on the GPU at once; queried once
    // (several host threads may race to store the same value).
    static std::atomic<int> resident_cache{0};
    int resident_blocks = resident_cache.load(std::memory_order_relaxed);
    if (resident_blocks == 0) {
        int dev = 0, per_cu = 0, cus = 0;
        hipError_t err = hipGetDevice(&dev);
        if (err == hipSuccess)
            err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (err == hipSuccess)
            err = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, reinterpret_cast<const void *>(call_kernel<S>), kBlock, 0);
        if (err != hipSuccess)
            return err;
        resident_blocks = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
        resident_cache.store(resident_blocks, std::memory_order_relaxed);
    }
    ProductShape ps;
    // Plan workgroups first (padded to a multiple of the 8 XCDs), product
    // workgroups in the remaining slots, so that every workgroup starts at
    // once.
    ps.plan_blocks = (a.shape.n_tiles + kPlanBlockWaves - 1) / kPlanBlockWaves;
    ps.plan_grid = (ps.plan_blocks + 7) / 8 * 8;
    int64_t product_blocks = resident_blocks - ps.plan_grid;
    if (product_blocks < 8)
        product_blocks = 8;
    ps.static_waves = product_blocks * kWavesPerBlock;
    // Short tiles: P rows per group (T = P*R rows, at most 64), at most 8,
    // small enough that the staged entries fit (T * short_max <= kShortCap),
    // and fewer when M is too small to give every product wavefront a tile.
    const int64_t smax = a.th.short_max > 1 ? a.th.short_max : 1;
    int64_t max_passes = kWave / S::R < 8 ? kWave / S::R : 8;
    if (max_passes > kShortCap / (S::R * smax))
        max_passes = kShortCap / (S::R * smax);
    if (max_passes < 1)
        return hipErrorInvalidValue;  // short_max above the group capacity
    int64_t passes = a.M / ((int64_t)S::R * ps.static_waves);
    passes = passes < 1 ? 1 : (passes > max_passes ? max_passes : passes);
    ps.passes = (int)passes;
    ps.dyn_passes = (int)(passes / kDynTileDiv<S> > 1 ? passes / kDynTileDiv<S> : 1);
    const int64_t ts = passes * S::R, td = (int64_t)ps.dyn_passes * S::R;
    const int64_t n_static = (a.M + ts - 1) / ts;
    ps.first = n_static < ps.static_waves ? n_static : ps.static_waves;
    ps.rows_static = ps.first * ts < a.M ? ps.first * ts : a.M;
    ps.n_dyn_tiles = (a.M - ps.rows_static + td - 1) / td;
    const int64_t blocks = ps.plan_grid + product_blocks;
    hipExtLaunchKernelGGL(call_kernel<S>, dim3((unsigned)blocks), dim3(kBlock),
                          0, stream, start, stop, 0, a, ps);
    return hipGetLastError();
}

// The PAIR form for rows of B two column passes of 16 lanes wide.
template <int DT, int VEC, bool BUF>
hipError_t launch_pair(int group, const WorkerArgs &a, hipStream_t s, hipEvent_t e0,
                       hipEvent_t e1)
{
    if (group != 16)
        return hipErrorInvalidValue;
    return launch_shape<Shape<DT, VEC, 16, 1, BUF, false, true>>(a, s, e0, e1);
}

template <int DT, int VEC, bool BUF, bool FUSED = false>
hipError_t launch_vec(int group, int nv, const WorkerArgs &a, hipStream_t s,
                      hipEvent_t e0, hipEvent_t e1)
{
    switch (group) {
    case 1: return launch_shape<Shape<DT, VEC, 1, 1, BUF, FUSED>>(a, s, e0, e1);
    case 2: return launch_shape<Shape<DT, VEC, 2, 1, BUF, FUSED>>(a, s, e0, e1);
    case 4: return launch_shape<Shape<DT, VEC, 4, 1, BUF, FUSED>>(a, s, e0, e1);
    case 8: return launch_shape<Shape<DT, VEC, 8, 1, BUF, FUSED>>(a, s, e0, e1);
    case 16: return launch_shape<Shape<DT, VEC, 16, 1, BUF, FUSED>>(a, s, e0, e1);
    case 32: return launch_shape<Shape<DT, VEC, 32, 1, BUF, FUSED>>(a, s, e0, e1);
    case 64:
        if (nv == 1) return launch_shape<Shape<DT, VEC, 64, 1, BUF, FUSED>>(a, s, e0, e1);
        if (nv == 2) return launch_shape<Shape<DT, VEC, 64, 2, BUF, FUSED>>(a, s, e0, e1);
        return launch_shape<Shape<DT, VEC, 64, 4, BUF, FUSED>>(a, s, e0, e1);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace
}  // namespace sdl
