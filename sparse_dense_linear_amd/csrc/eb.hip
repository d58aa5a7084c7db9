// eb.hip -- element-balanced sparse x dense product: a single pass over the
// stored entries with no row plan, gfx950.
//
// Page: [Sgap] "Sgap: Towards Efficient Sparse Tensor Algebra Compilation
// for GPU": the element-balanced (EB) points of atomic parallelism, where
// each worker takes a fixed number of non-zeros regardless of rows, and the
// grouped segmented reduction that combines the partial sums of entries
// that share a row.  Here the combination is deterministic (no atomics):
//
//   * the stored entries are split into equal spans, one per wavefront
//     (whole 64-entry batches; the count comes from rowptr on the device);
//   * a batch's 64 entries are staged in LDS with their rows (row found by
//     a 64-ary search at the span start, then a 64-row window search);
//   * per step, lane group g takes U consecutive entries and streams them
//     with all U gathers in flight, storing every row that starts and ends
//     inside those entries, and keeping the partial of its first row (head)
//     and of its last row (tail);
//   * the groups' heads and tails are then added in entry order into the
//     wavefront's open row (a segmented reduction across the groups); a row
//     that closes inside the span is stored;
//   * the span's first row, if it started in an earlier span, and its last
//     row, if it goes on past the span, are partial: each goes to a carry
//     slot of the wavefront (device-coherent stores), and the wavefront
//     then arrives on a counter of that row (tagged with the call's epoch);
//     the arrival that completes the row's count adds the row's slots in
//     span order and stores the row -- so the whole product is one launch;
//   * empty rows are zeroed by one wavefront each (before the first entry:
//     wavefront 0; between a span's entries: that span; starting exactly at
//     a span's end: that span).
// Every output element is the sum of its row's products in a fixed order,
// so results repeat bit for bit.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "gather.h"
#include "internal.h"
#include "plan_device.h"
#include "span.h"
#include "spmm.h"

namespace sdl {
namespace {

template <class S>
struct EbStep {
    // entries per group per step: U, but at most 64/R so a step fits a batch
    static constexpr int UE = S::U < kWave / S::R ? S::U : kWave / S::R;
    static constexpr int SU = S::R * UE;  // entries per step
};

// Zero rows [lo, hi) of C, the whole wavefront writing each row (rows of
// N floats, lanes over the columns).
__device__ void zero_rows(float *C, int64_t N, int64_t lo, int64_t hi, int lane)
{
    for (int64_t r = lo; r < hi; ++r)
        for (int64_t c = lane; c < N; c += kWave)
            C[r * N + c] = 0.0f;
}

// Zero the empty rows that follow row `last` and start at position p (no
// entries, rowptr == p): the run of such rows, 64 at a time.
__device__ void zero_empty_after(float *C, const int32_t *rowptr, int64_t M,
                                 int64_t N, int64_t last, int64_t p, int lane)
{
    for (int64_t r0 = last + 1; r0 < M; r0 += kWave) {
        const int64_t r = r0 + lane;
        const int64_t rc = r < M ? r : M - 1;  // rc + 1 <= M
        const bool empty_here = r < M && (int64_t)rowptr[rc] == p &&
                                (int64_t)rowptr[rc + 1] == p;
        // the empty rows at p form a prefix of the run
        const uint64_t m = __ballot(empty_here);
        const int cnt = __popcll(~m) == 0 ? kWave : __builtin_ctzll(~m);
        zero_rows(C, N, r0, r0 + cnt, lane);
        if (cnt < kWave)
            break;
    }
}

// Store this lane's columns of a partial row into carry slot `slot` with
// device-coherent stores (another XCD's wavefront may read it).
template <class S>
__device__ inline void store_partial(float *carry_val, int64_t slot, int64_t N,
                                     int64_t col0, int j,
                                     const float (&acc)[S::NV][S::VEC])
{
#pragma unroll
    for (int k = 0; k < S::NV; ++k) {
        const int64_t c = col0 + (int64_t)(k * S::G + j) * S::VEC;
        if (c >= N)
            continue;
#pragma unroll
        for (int x = 0; x < S::VEC; ++x)
            __hip_atomic_store(carry_val + slot * N + c + x, acc[k][x],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Count one arrival on a counter tagged with the call's epoch (a word with
// another tag counts as 0) and return the count including this arrival.
// Lock-free: a retry happens only when another arrival got in first.
__device__ inline uint32_t arrive(uint64_t *ctr, uint32_t epoch)
{
    uint64_t old = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int tries = 0; tries < (1 << 20); ++tries) {
        const uint32_t cnt = (uint32_t)(old >> 32) == epoch ? (uint32_t)old : 0u;
        const uint64_t nw = ((uint64_t)epoch << 32) | (uint64_t)(cnt + 1);
        if (__hip_atomic_compare_exchange_strong(ctr, &old, nw, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT))
            return cnt + 1;
    }
    return 0;  // not reached with the few arrivals a row has
}

// Row x was cut by span ends: its partials sit in the tail slot of the span
// holding its first entry (wa) and in the head slots of spans wa+1 .. wb.
// The wavefront whose arrival completes the count adds them in that order
// (8 coherent loads in flight) and stores the row.
__device__ void finish_split_row(const EbArgs &a, int64_t x, int64_t base,
                                 int64_t span, int lane)
{
    const int64_t wa = ((int64_t)a.rowptr[x] - base) / span;
    const int64_t wb = ((int64_t)a.rowptr[x + 1] - 1 - base) / span;
    int c_arr = 0;
    if (lane == 0)
        c_arr = (int)arrive(a.arrive + wa, a.epoch);
    c_arr = __shfl(c_arr, 0);
    if (c_arr != (int)(wb - wa + 1))
        return;
    const int64_t n = wb - wa + 1;  // slots: 2wa+1, then 2(wa+1), ..., 2wb
    constexpr int kAhead = 8;
    for (int64_t c = lane; c < a.N; c += kWave) {
        float v = 0.0f;
        for (int64_t t0 = 0; t0 < n; t0 += kAhead) {
            float xs[kAhead];
#pragma unroll
            for (int u = 0; u < kAhead; ++u) {
                const int64_t t = t0 + u < n ? t0 + u : n - 1;
                const int64_t slot = t == 0 ? 2 * wa + 1 : 2 * (wa + t);
                xs[u] = __hip_atomic_load(a.carry_val + slot * a.N + c,
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int u = 0; u < kAhead; ++u)
                v = t0 + u < n ? v + xs[u] : v;
        }
        a.C[x * a.N + c] = v;
    }
}

// Move group gg's slice of a partial row to every group (lane j of each
// group gets lane j of group gg).
template <class S>
__device__ inline void from_group(const float (&src)[S::NV][S::VEC], int gg,
                                  int j, float (&dst)[S::NV][S::VEC])
{
#pragma unroll
    for (int k = 0; k < S::NV; ++k)
#pragma unroll
        for (int x = 0; x < S::VEC; ++x)
            dst[k][x] = __shfl(src[k][x], gg * S::G + j);
}

template <class S>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4)))
void eb_kernel(EbArgs a)
{
    __shared__ Entry ent[kWavesPerBlock][kWave];
    __shared__ int32_t erow[kWavesPerBlock][kWave];
    typedef EbStep<S> E;
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int g = lane / S::G;
    const int j = lane % S::G;
    const int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + wid;
    // Every call on a stream takes the next epoch, and a planned product
    // call draws from the queue counter set of its epoch's parity, which the
    // call before it must clear: this call clears the set of epoch + 1 (no
    // call on the stream is using it now).
    if (w == 0)
        for (int q = lane; q < kQueues; q += kWave)
            a.queues[(((a.epoch + 1) & 1) * kQueues + q) * kQueueStride] = 0;
    if (w >= a.waves)
        return;
    const int32_t *rowptr = a.rowptr;
    const int64_t base = rowptr[0];
    const int64_t nnz = (int64_t)rowptr[a.M] - base;
    int64_t span = (nnz + a.waves - 1) / a.waves;
    span = (span + kWave - 1) / kWave * kWave;
    span = span < kWave ? kWave : span;
    const int64_t s0 = w * span < nnz ? w * span : nnz;
    const int64_t s1 = s0 + span < nnz ? s0 + span : nnz;

    if (nnz == 0) {
        // no entries at all: every row is a zero row
        if (w == 0)
            zero_rows(a.C, a.N, 0, a.M, lane);
        return;
    }
    if (s0 >= s1)
        return;
    // Empty rows are zeroed by one wavefront each: wavefront 0 takes those
    // before the first stored entry, a span takes those between its own
    // entries (found while walking) and those that start exactly at its end
    // (after its last row, if that row ends there; the last span's are the
    // trailing empty rows).

    const uint32_t row_bytes = (uint32_t)(a.N * S::ESZ);
    BSrc src;
    src.base = (const char *)a.B;
    if constexpr (S::BUF)
        src.rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<void *>(a.B), (short)0,
            (int)(uint32_t)(a.K * a.N * S::ESZ), kBufferWord3);
    const int64_t r_first = find_row(rowptr, a.M, base + s0, lane);
    const bool first_partial = (int64_t)rowptr[r_first] < base + s0;
    if (w == 0)
        zero_rows(a.C, a.N, 0, r_first, lane);  // rows before the first entry
    Entry *st = ent[wid];
    int32_t *rw = erow[wid];
    int64_t r_last = r_first;  // row of the span's last entry

    for (int64_t col0 = 0; col0 < a.N; col0 += S::COLS) {
        const LaneCols<S> lc = lane_cols<S>(a.N, col0, j);
        int64_t i_cur = r_first;
        int64_t open_row = -1;
        float acc_open[S::NV][S::VEC];
        zero_acc<S>(acc_open);

        // Close the open row: a carry if it is the span's first row and began
        // in an earlier span, else a stored row.
        auto flush_open = [&]() {
            if (open_row < 0)
                return;
            if (open_row == r_first && first_partial) {
                if (g == 0)
                    store_partial<S>(a.carry_val, 2 * w, a.N, col0, j, acc_open);
            } else if (g == 0) {
                emit_row<S, false>(a.C, open_row, a.N, col0, j, acc_open);
            }
        };

        // the first batch's entries and row window, loaded ahead
        int64_t pe = base + (lane < s1 - s0 ? s0 + lane : s1 - 1);
        int32_t ncol = a.colind[pe];
        float nval = load_val<S::DT>(a.vals, pe);
        int64_t nwin = rowptr[i_cur + 1 + lane < a.M ? i_cur + 1 + lane : a.M];
        int64_t prev_last = r_first;  // row of the previous batch's last entry

        for (int64_t e0 = s0; e0 < s1; e0 += kWave) {
            const int nb = s1 - e0 < kWave ? (int)(s1 - e0) : kWave;
            Entry en;
            en.col = ncol;
            en.val = nval;
            const int64_t row = row_in_window(rowptr, a.M, i_cur, pe, lane, nwin);
            i_cur = __shfl(row, kWave - 1);
            // the next batch's loads go out before this batch's gathers
            const int64_t e1 = e0 + kWave;
            if (e1 < s1) {
                pe = base + (lane < s1 - e1 ? e1 + lane : s1 - 1);
                ncol = a.colind[pe];
                nval = load_val<S::DT>(a.vals, pe);
                nwin = rowptr[i_cur + 1 + lane < a.M ? i_cur + 1 + lane : a.M];
            }
            if (col0 == 0) {
                // rows skipped between consecutive entries have no entries
                const int64_t before = lane == 0 ? prev_last : __shfl_up(row, 1);
                const bool gap = lane < nb && row > before + 1;
                uint64_t m = __ballot(gap);
                while (m != 0) {
                    const int l = __builtin_ctzll(m);
                    m &= m - 1;
                    const int64_t hi = __shfl(row, l);
                    const int64_t lo = (l == 0 ? prev_last : __shfl(row, l - 1)) + 1;
                    zero_rows(a.C, a.N, lo, hi, lane);
                }
            }
            prev_last = i_cur;
            __builtin_amdgcn_wave_barrier();  // the previous batch is consumed
            st[lane] = en;
            rw[lane] = (int32_t)row;
            __builtin_amdgcn_wave_barrier();  // staged before any lane reads

            for (int st0 = 0; st0 < nb; st0 += E::SU) {
                const int k0 = st0 + g * E::UE;
                int n = nb - k0;
                n = n < 0 ? 0 : (n > E::UE ? E::UE : n);
                const int q = k0 < nb ? k0 : nb - 1;
                Batch<S> bt;
                issue<S>(bt, st, q, n, src, row_bytes, lc);
                float acc[S::NV][S::VEC], hacc[S::NV][S::VEC];
                zero_acc<S>(acc);
                zero_acc<S>(hacc);
                bool changed = false;
                const int32_t hrow = rw[q];
                int32_t prev = hrow;
#pragma unroll
                for (int u = 0; u < E::UE; ++u) {
                    const bool on = u < n;
                    const int32_t r = rw[on ? q + u : q];
                    if (on && u > 0 && r != prev) {
                        if (!changed) {
#pragma unroll
                            for (int k = 0; k < S::NV; ++k)
#pragma unroll
                                for (int x = 0; x < S::VEC; ++x)
                                    hacc[k][x] = acc[k][x];
                            changed = true;
                        } else {
                            // a row that starts and ends inside these entries
                            emit_row<S, false>(a.C, prev, a.N, col0, j, acc);
                        }
                        zero_acc<S>(acc);
                    }
                    accumulate<S>(bt, u, on, acc);
                    prev = on ? r : prev;
                }
                const int32_t trow = prev;

                // segmented reduction across the groups, in entry order
                for (int gg = 0; gg < S::R; ++gg) {
                    const int ng = __shfl(n, gg * S::G);
                    if (ng == 0)
                        continue;
                    const bool ch = __shfl((int)changed, gg * S::G) != 0;
                    const int32_t hr = __shfl(hrow, gg * S::G);
                    const int32_t tr = __shfl(trow, gg * S::G);
                    float part[S::NV][S::VEC];
                    if (ch) {
                        from_group<S>(hacc, gg, j, part);
                        if (hr == open_row) {
#pragma unroll
                            for (int k = 0; k < S::NV; ++k)
#pragma unroll
                                for (int x = 0; x < S::VEC; ++x)
                                    acc_open[k][x] += part[k][x];
                        } else {
                            flush_open();
#pragma unroll
                            for (int k = 0; k < S::NV; ++k)
#pragma unroll
                                for (int x = 0; x < S::VEC; ++x)
                                    acc_open[k][x] = part[k][x];
                        }
                        open_row = hr;
                        flush_open();  // the head row ended inside group gg
                        from_group<S>(acc, gg, j, acc_open);
                        open_row = tr;
                    } else {
                        from_group<S>(acc, gg, j, part);
                        if (tr == open_row) {
#pragma unroll
                            for (int k = 0; k < S::NV; ++k)
#pragma unroll
                                for (int x = 0; x < S::VEC; ++x)
                                    acc_open[k][x] += part[k][x];
                        } else {
                            flush_open();
#pragma unroll
                            for (int k = 0; k < S::NV; ++k)
#pragma unroll
                                for (int x = 0; x < S::VEC; ++x)
                                    acc_open[k][x] = part[k][x];
                            open_row = tr;
                        }
                    }
                }
            }
        }

        r_last = i_cur;

        // The last open row: if it goes on past the span it is partial (the
        // head slot if it is also the span's first, partial row -- the whole
        // span lies inside it -- else the tail slot).
        if ((int64_t)rowptr[open_row + 1] > base + s1) {
            if (open_row == r_first && first_partial)
                flush_open();
            else if (g == 0)
                store_partial<S>(a.carry_val, 2 * w + 1, a.N, col0, j, acc_open);
        } else {
            flush_open();
        }
    }

    // Rows cut by this span's ends: arrive once per row; the last arrival
    // adds the row's partials and stores it.
    const bool tail_split = (int64_t)rowptr[r_last + 1] > base + s1 &&
                            !(r_last == r_first && first_partial);
    if (first_partial || tail_split) {
        wait_stores_done();  // the partials are visible device-wide first
        if (first_partial)
            finish_split_row(a, r_first, base, span, lane);
        if (tail_split)
            finish_split_row(a, r_last, base, span, lane);
    }
    // empty rows that start where this span ends (the last row ends there)
    if ((int64_t)rowptr[r_last + 1] == base + s1)
        zero_empty_after(a.C, rowptr, a.M, a.N, r_last, base + s1, lane);
}

template <class S>
hipError_t launch_eb_shape(const EbArgs &a0, hipStream_t stream, hipEvent_t e0,
                           hipEvent_t e1)
{
    EbArgs a = a0;
    const int64_t blocks = (a.waves + kWavesPerBlock - 1) / kWavesPerBlock;
    hipExtLaunchKernelGGL(eb_kernel<S>, dim3((unsigned)blocks), dim3(kBlock), 0,
                          stream, e0, e1, 0, a);
    return hipGetLastError();
}

template <int DT, int VEC, bool BUF>
hipError_t launch_eb_vec(int group, int nv, const EbArgs &a, hipStream_t s,
                         hipEvent_t e0, hipEvent_t e1)
{
    switch (group) {
    case 1: return launch_eb_shape<Shape<DT, VEC, 1, 1, BUF>>(a, s, e0, e1);
    case 2: return launch_eb_shape<Shape<DT, VEC, 2, 1, BUF>>(a, s, e0, e1);
    case 4: return launch_eb_shape<Shape<DT, VEC, 4, 1, BUF>>(a, s, e0, e1);
    case 8: return launch_eb_shape<Shape<DT, VEC, 8, 1, BUF>>(a, s, e0, e1);
    case 16: return launch_eb_shape<Shape<DT, VEC, 16, 1, BUF>>(a, s, e0, e1);
    case 32: return launch_eb_shape<Shape<DT, VEC, 32, 1, BUF>>(a, s, e0, e1);
    case 64:
        if (nv == 1) return launch_eb_shape<Shape<DT, VEC, 64, 1, BUF>>(a, s, e0, e1);
        if (nv == 2) return launch_eb_shape<Shape<DT, VEC, 64, 2, BUF>>(a, s, e0, e1);
        return launch_eb_shape<Shape<DT, VEC, 64, 4, BUF>>(a, s, e0, e1);
    default: return hipErrorInvalidValue;
    }
}

template <bool BUF>
hipError_t launch_eb_dtype(const WorkerConfig &cfg, const EbArgs &a,
                           hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    if (cfg.dtype == SPMM_DTYPE_F32) {
        switch (cfg.vec) {
        case 4: return launch_eb_vec<SPMM_DTYPE_F32, 4, BUF>(cfg.group, cfg.nv, a, s, e0, e1);
        case 2: return launch_eb_vec<SPMM_DTYPE_F32, 2, BUF>(cfg.group, cfg.nv, a, s, e0, e1);
        case 1: return launch_eb_vec<SPMM_DTYPE_F32, 1, BUF>(cfg.group, cfg.nv, a, s, e0, e1);
        }
    } else {
        switch (cfg.vec) {
        case 8: return launch_eb_vec<SPMM_DTYPE_BF16, 8, BUF>(cfg.group, cfg.nv, a, s, e0, e1);
        case 4: return launch_eb_vec<SPMM_DTYPE_BF16, 4, BUF>(cfg.group, cfg.nv, a, s, e0, e1);
        case 2: return launch_eb_vec<SPMM_DTYPE_BF16, 2, BUF>(cfg.group, cfg.nv, a, s, e0, e1);
        case 1: return launch_eb_vec<SPMM_DTYPE_BF16, 1, BUF>(cfg.group, cfg.nv, a, s, e0, e1);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_eb(const WorkerConfig &cfg, const EbArgs &a, hipStream_t s,
                     hipEvent_t e0, hipEvent_t e1)
{
    const int esz = cfg.dtype == SPMM_DTYPE_BF16 ? 2 : 4;
    const uint64_t b_bytes = (uint64_t)a.K * (uint64_t)a.N * (uint64_t)esz;
    if (b_bytes <= kBufMaxBytes)
        return launch_eb_dtype<true>(cfg, a, s, e0, e1);
    return launch_eb_dtype<false>(cfg, a, s, e0, e1);
}

int64_t eb_waves()
{
    // one span per wavefront slot of the GPU (4 per SIMD, 4 SIMDs per
    // compute unit); with fewer resident, the rest run later (no wavefront
    // of this kernel waits for another)
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return (int64_t)cus * 16;
}

}  // namespace sdl
