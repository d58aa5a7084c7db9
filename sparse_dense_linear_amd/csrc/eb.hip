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
//     row, if it goes on past the span, are partial: they go to two carry
//     slots per wavefront, and a second small kernel adds the carries of
//     each row in slot order and stores the row;
//   * the empty rows that start inside a span are written as zero rows by
//     that span's wavefront.
// Every output element is the sum of its row's products in a fixed order,
// so results repeat bit for bit.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "gather.h"
#include "internal.h"
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

// Zero rows [lo, hi) that hold no entries; group g takes every R-th empty
// row found.
template <class S>
__device__ void zero_empty_rows(const EbArgs &a, int64_t lo, int64_t hi,
                                int lane, int g, int j)
{
    for (int64_t r0 = lo; r0 < hi; r0 += kWave) {
        const int64_t r = r0 + lane;
        const int64_t rc = r < hi ? r : hi - 1;  // rc + 1 <= hi <= M
        const bool empty = r < hi && a.rowptr[rc + 1] == a.rowptr[rc];
        uint64_t m = __ballot(empty);
        for (int k = 0; m != 0; ++k) {
            const int bit = __builtin_ctzll(m);
            m &= m - 1;
            if (k % S::R != g)
                continue;
            float z[S::NV][S::VEC];
            zero_acc<S>(z);
            for (int64_t col0 = 0; col0 < a.N; col0 += S::COLS)
                emit_row<S, false>(a.C, r0 + bit, a.N, col0, j, z);
        }
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
__global__ __launch_bounds__(kBlock) void eb_kernel(EbArgs a)
{
    __shared__ Entry ent[kWavesPerBlock][kWave];
    __shared__ int32_t erow[kWavesPerBlock][kWave];
    typedef EbStep<S> E;
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int g = lane / S::G;
    const int j = lane % S::G;
    const int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + wid;
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
    const int64_t last_wave = nnz == 0 ? 0 : (nnz - 1) / span;

    // carry slots 2w (head) and 2w+1 (tail): unused unless written below
    if (lane == 0) {
        a.carry_row[2 * w] = -1;
        a.carry_row[2 * w + 1] = -1;
    }
    // empty rows starting in this span (the last span also takes those at
    // position nnz, i.e. trailing empty rows)
    if (w <= last_wave) {
        const int64_t lo = w == 0 ? 0 : lower_row(rowptr, a.M, base + s0, lane);
        const int64_t hi = w == last_wave ? a.M : lower_row(rowptr, a.M, base + s1, lane);
        zero_empty_rows<S>(a, lo, hi, lane, g, j);
    }
    if (s0 >= s1)
        return;

    const uint32_t row_bytes = (uint32_t)(a.N * S::ESZ);
    BSrc src;
    src.base = (const char *)a.B;
    if constexpr (S::BUF)
        src.rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<void *>(a.B), (short)0,
            (int)(uint32_t)(a.K * a.N * S::ESZ), kBufferWord3);
    const int64_t r_first = find_row(rowptr, a.M, base + s0, lane);
    const bool first_partial = (int64_t)rowptr[r_first] < base + s0;
    Entry *st = ent[wid];
    int32_t *rw = erow[wid];

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
                    emit_row<S, false>(a.carry_val, 2 * w, a.N, col0, j, acc_open);
                if (lane == 0)
                    a.carry_row[2 * w] = (int32_t)open_row;
            } else if (g == 0) {
                emit_row<S, false>(a.C, open_row, a.N, col0, j, acc_open);
            }
        };

        for (int64_t e0 = s0; e0 < s1; e0 += kWave) {
            const int nb = s1 - e0 < kWave ? (int)(s1 - e0) : kWave;
            const int64_t pe = base + (lane < nb ? e0 + lane : s1 - 1);
            Entry en;
            en.col = a.colind[pe];
            en.val = load_val<S::DT>(a.vals, pe);
            const int64_t row = row_in_window(rowptr, a.M, i_cur, pe, lane);
            i_cur = __shfl(row, kWave - 1);
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
                issue<S>(bt, st, q, n > 0 ? n : 1, src, row_bytes, lc);
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

        // The last open row: a tail carry if it goes on past the span.
        if ((int64_t)rowptr[open_row + 1] > base + s1) {
            if (open_row == r_first && first_partial) {
                // the whole span lies inside one row: the partial is the head
                // carry, and a zero tail carry keeps the row's slots adjacent
                flush_open();
                float z[S::NV][S::VEC];
                zero_acc<S>(z);
                if (g == 0)
                    emit_row<S, false>(a.carry_val, 2 * w + 1, a.N, col0, j, z);
            } else if (g == 0) {
                emit_row<S, false>(a.carry_val, 2 * w + 1, a.N, col0, j, acc_open);
            }
            if (lane == 0)
                a.carry_row[2 * w + 1] = (int32_t)open_row;
        } else {
            flush_open();
        }
    }
}

// Rows split across spans: slot s starts a run if it holds a row and the
// slot before it holds another; the run's slots are added in slot order and
// the row is stored.  One wavefront per slot.
__global__ __launch_bounds__(kBlock) void eb_fixup(const int32_t *carry_row,
                                                   const float *carry_val,
                                                   float *C, int64_t slots,
                                                   int64_t N)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t s = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    if (s >= slots)
        return;
    const int32_t r = carry_row[s];
    if (r < 0 || (s > 0 && carry_row[s - 1] == r))
        return;
    int64_t e = s + 1;
    while (e < slots && carry_row[e] == r)
        ++e;
    for (int64_t c = lane; c < N; c += kWave) {
        float v = 0.0f;
        for (int64_t t = s; t < e; ++t)
            v += carry_val[t * N + c];
        C[(int64_t)r * N + c] = v;
    }
}

template <class S>
hipError_t launch_eb_shape(const EbArgs &a0, hipStream_t stream, hipEvent_t e0,
                           hipEvent_t e1)
{
    EbArgs a = a0;
    const int64_t blocks = (a.waves + kWavesPerBlock - 1) / kWavesPerBlock;
    hipExtLaunchKernelGGL(eb_kernel<S>, dim3((unsigned)blocks), dim3(kBlock), 0,
                          stream, e0, nullptr, 0, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    const int64_t slots = 2 * a.waves;
    const int64_t fblocks = (slots + kWavesPerBlock - 1) / kWavesPerBlock;
    hipExtLaunchKernelGGL(eb_fixup, dim3((unsigned)fblocks), dim3(kBlock), 0, stream,
                          nullptr, e1, 0, a.carry_row, a.carry_val, a.C, slots, a.N);
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
    if (b_bytes < 0xFFFFFFFFull)
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
