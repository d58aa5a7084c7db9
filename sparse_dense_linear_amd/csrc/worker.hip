// worker.hip -- gather-scale-accumulate kernels of the CSR sparse x dense
// product C = A * B on gfx950.
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
//   * colind/vals of the entries being worked on are staged in LDS, loaded
//     once with coalesced loads and then read (as broadcasts) by the lanes
//     that cover the N columns.
//   * Three kinds of work item, all handled by one grid-stride kernel:
//       long chunk  (row, p0, p1) from the plan: the R groups split the
//                   chunk's entries, their partial rows are summed by
//                   butterfly shuffles, and group 0 adds the result to C
//                   with fp32 atomics (the row was zeroed by the plan);
//       medium row  from the plan: as a chunk over the whole row, but the
//                   result is stored, not added;
//       short tile  a block of consecutive rows in natural order: each group
//                   takes one row per pass (one row per group: RB with
//                   coarsened columns); rows that are not short are skipped,
//                   they belong to the other two kinds.
//   * Within an item, U gathers per lane are issued back to back before any
//     of them is consumed.
#include "internal.h"
#include "spmm.h"

namespace sdl {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Loads of VEC consecutive elements of B and their exact widening to fp32.
template <int DT, int VEC> struct BLoad;

template <> struct BLoad<SPMM_DTYPE_F32, 4> {
    typedef f32x4 raw;
    static __device__ raw load(const void *p) { return *(const f32x4 *)p; }
    static __device__ void widen(const raw &r, float (&o)[4])
    { o[0] = r.x; o[1] = r.y; o[2] = r.z; o[3] = r.w; }
};
template <> struct BLoad<SPMM_DTYPE_F32, 2> {
    typedef f32x2 raw;
    static __device__ raw load(const void *p) { return *(const f32x2 *)p; }
    static __device__ void widen(const raw &r, float (&o)[2])
    { o[0] = r.x; o[1] = r.y; }
};
template <> struct BLoad<SPMM_DTYPE_F32, 1> {
    typedef float raw;
    static __device__ raw load(const void *p) { return *(const float *)p; }
    static __device__ void widen(const raw &r, float (&o)[1]) { o[0] = r; }
};
template <> struct BLoad<SPMM_DTYPE_BF16, 8> {
    typedef u32x4 raw;
    static __device__ raw load(const void *p) { return *(const u32x4 *)p; }
    static __device__ void widen(const raw &r, float (&o)[8])
    {
        o[0] = bf16_lo(r.x); o[1] = bf16_hi(r.x);
        o[2] = bf16_lo(r.y); o[3] = bf16_hi(r.y);
        o[4] = bf16_lo(r.z); o[5] = bf16_hi(r.z);
        o[6] = bf16_lo(r.w); o[7] = bf16_hi(r.w);
    }
};
template <> struct BLoad<SPMM_DTYPE_BF16, 4> {
    typedef u32x2 raw;
    static __device__ raw load(const void *p) { return *(const u32x2 *)p; }
    static __device__ void widen(const raw &r, float (&o)[4])
    {
        o[0] = bf16_lo(r.x); o[1] = bf16_hi(r.x);
        o[2] = bf16_lo(r.y); o[3] = bf16_hi(r.y);
    }
};
template <> struct BLoad<SPMM_DTYPE_BF16, 2> {
    typedef uint32_t raw;
    static __device__ raw load(const void *p) { return *(const uint32_t *)p; }
    static __device__ void widen(const raw &r, float (&o)[2])
    { o[0] = bf16_lo(r); o[1] = bf16_hi(r); }
};
template <> struct BLoad<SPMM_DTYPE_BF16, 1> {
    typedef uint16_t raw;
    static __device__ raw load(const void *p) { return *(const uint16_t *)p; }
    static __device__ void widen(const raw &r, float (&o)[1])
    { o[0] = __uint_as_float((uint32_t)r << 16); }
};

template <int DT> struct ElemSize;
template <> struct ElemSize<SPMM_DTYPE_F32> { static constexpr int v = 4; };
template <> struct ElemSize<SPMM_DTYPE_BF16> { static constexpr int v = 2; };

// A stored entry as staged in LDS: column and value (already fp32).
struct Entry {
    int32_t col;
    float val;
};

template <int DT> __device__ inline float load_val(const void *vals, int64_t p);
template <> __device__ inline float load_val<SPMM_DTYPE_F32>(const void *vals, int64_t p)
{ return ((const float *)vals)[p]; }
template <> __device__ inline float load_val<SPMM_DTYPE_BF16>(const void *vals, int64_t p)
{ return __uint_as_float((uint32_t)((const uint16_t *)vals)[p] << 16); }

// Compile-time shape of one worker variant.
template <int DT_, int VEC_, int G_, int NV_>
struct Shape {
    static constexpr int DT = DT_;
    static constexpr int VEC = VEC_;
    static constexpr int G = G_;
    static constexpr int NV = NV_;
    static constexpr int R = kWave / G_;          // groups per wavefront
    static constexpr int COLS = G_ * VEC_ * NV_;  // columns per column pass
    static constexpr int U = NV_ == 1 ? 8 : (NV_ == 2 ? 4 : 2);  // gathers in flight
};

// Group-local SAXPY over cnt staged entries: acc += val * B[col, cols of lane].
template <class S>
__device__ inline void consume(const Entry *st, int cnt, const void *B,
                               int64_t N, int64_t col0, int j,
                               float (&acc)[S::NV][S::VEC])
{
    typedef BLoad<S::DT, S::VEC> L;
    const char *Bb = (const char *)B;
    for (int u = 0; u < cnt; u += S::U) {
        typename L::raw buf[S::U][S::NV];
        float v[S::U];
#pragma unroll
        for (int q = 0; q < S::U; ++q) {
            if (u + q < cnt) {
                const Entry e = st[u + q];
                v[q] = e.val;
                const int64_t rowoff = (int64_t)e.col * N + col0;
#pragma unroll
                for (int k = 0; k < S::NV; ++k) {
                    const int64_t c = (int64_t)(k * S::G + j) * S::VEC;
                    if (col0 + c < N)
                        buf[q][k] = L::load(Bb + (rowoff + c) * ElemSize<S::DT>::v);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < S::U; ++q) {
            if (u + q < cnt) {
#pragma unroll
                for (int k = 0; k < S::NV; ++k) {
                    const int64_t c = (int64_t)(k * S::G + j) * S::VEC;
                    if (col0 + c < N) {
                        float b[S::VEC];
                        L::widen(buf[q][k], b);
#pragma unroll
                        for (int x = 0; x < S::VEC; ++x)
                            acc[k][x] = fmaf(v[q], b[x], acc[k][x]);
                    }
                }
            }
        }
    }
}

template <class S>
__device__ inline void zero_acc(float (&acc)[S::NV][S::VEC])
{
#pragma unroll
    for (int k = 0; k < S::NV; ++k)
#pragma unroll
        for (int x = 0; x < S::VEC; ++x)
            acc[k][x] = 0.0f;
}

// Store (or atomically add) this lane's columns of one C row.
template <class S, bool ATOMIC>
__device__ inline void emit_row(float *C, int64_t row, int64_t N, int64_t col0,
                                int j, const float (&acc)[S::NV][S::VEC])
{
    float *crow = C + row * N + col0;
#pragma unroll
    for (int k = 0; k < S::NV; ++k) {
        const int64_t c = (int64_t)(k * S::G + j) * S::VEC;
        if (col0 + c >= N)
            continue;
        if constexpr (ATOMIC) {
#pragma unroll
            for (int x = 0; x < S::VEC; ++x)
                unsafeAtomicAdd(crow + c + x, acc[k][x]);
        } else if constexpr (S::VEC % 4 == 0) {
#pragma unroll
            for (int x = 0; x < S::VEC; x += 4) {
                f32x4 w = {acc[k][x], acc[k][x + 1], acc[k][x + 2], acc[k][x + 3]};
                *(f32x4 *)(crow + c + x) = w;
            }
        } else if constexpr (S::VEC == 2) {
            f32x2 w = {acc[k][0], acc[k][1]};
            *(f32x2 *)(crow + c) = w;
        } else {
            crow[c] = acc[k][0];
        }
    }
}

// Sum the partial rows of the R groups (butterfly over lane distance
// G, 2G, ...).  Groups that received no entries hold zeros.
template <class S>
__device__ inline void reduce_groups(float (&acc)[S::NV][S::VEC])
{
#pragma unroll
    for (int off = S::G; off < kWave; off <<= 1)
#pragma unroll
        for (int k = 0; k < S::NV; ++k)
#pragma unroll
            for (int x = 0; x < S::VEC; ++x)
                acc[k][x] += __shfl_xor(acc[k][x], off);
}

// One wavefront accumulates positions [p0, p1) of one row: 64-entry chunks
// of colind/vals are loaded coalesced (the next one prefetched into
// registers while the current one is consumed) and staged in LDS; group g
// consumes entries g*G .. g*G+G-1 of each chunk.
template <class S>
__device__ inline void wave_range(const WorkerArgs &a, Entry *st, int lane,
                                  int g, int j, int64_t p0, int64_t p1,
                                  int64_t col0, float (&acc)[S::NV][S::VEC])
{
    zero_acc<S>(acc);
    int32_t nc = 0;
    float nvv = 0.0f;
    if (p0 + lane < p1) {
        nc = a.colind[p0 + lane];
        nvv = load_val<S::DT>(a.vals, p0 + lane);
    }
    for (int64_t base = p0; base < p1; base += kWave) {
        const int n = p1 - base < kWave ? (int)(p1 - base) : kWave;
        if (lane < n) {
            Entry e;
            e.col = nc;
            e.val = nvv;
            st[lane] = e;
        }
        const int64_t nb = base + kWave;
        if (nb + lane < p1) {
            nc = a.colind[nb + lane];
            nvv = load_val<S::DT>(a.vals, nb + lane);
        }
        int cnt = n - g * S::G;
        cnt = cnt < 0 ? 0 : (cnt > S::G ? S::G : cnt);
        consume<S>(st + g * S::G, cnt, a.B, a.N, col0, j, acc);
    }
}

template <class S>
__device__ void do_chunk(const WorkerArgs &a, Entry *st, int lane, int g,
                         int j, int64_t c, int32_t n_long)
{
    const Chunk ch = resolve_chunk(c, a.plan, n_long, a.rowptr);
    for (int64_t col0 = 0; col0 < a.N; col0 += S::COLS) {
        float acc[S::NV][S::VEC];
        wave_range<S>(a, st, lane, g, j, ch.p0, ch.p1, col0, acc);
        reduce_groups<S>(acc);
        if (g == 0)
            emit_row<S, true>(a.C, ch.row, a.N, col0, j, acc);
    }
}

template <class S>
__device__ void do_medium(const WorkerArgs &a, Entry *st, int lane, int g,
                          int j, int64_t i)
{
    const int64_t row = a.plan.medium_rows[i];
    const int64_t p0 = a.rowptr[row];
    const int64_t p1 = a.rowptr[row + 1];
    for (int64_t col0 = 0; col0 < a.N; col0 += S::COLS) {
        float acc[S::NV][S::VEC];
        wave_range<S>(a, st, lane, g, j, p0, p1, col0, acc);
        reduce_groups<S>(acc);
        if (g == 0)
            emit_row<S, false>(a.C, row, a.N, col0, j, acc);
    }
}

// A short tile is `passes` passes of R consecutive rows (passes * R <= 64).
template <class S>
__device__ void do_short_tile(const WorkerArgs &a, Entry *st, int lane, int g,
                              int j, int64_t t, int passes)
{
    const int tile = passes * S::R;
    const int64_t r0 = t * tile;
    // lane l < tile holds the extent of row r0 + l
    int32_t s = 0, e = 0;
    if (lane < tile && r0 + lane < a.M) {
        s = a.rowptr[r0 + lane];
        e = a.rowptr[r0 + lane + 1];
    }
    Entry *sg = st + g * S::G;
#pragma unroll 1
    for (int pass = 0; pass < passes; ++pass) {
        const int src = pass * S::R + g;
        const int32_t start = __shfl(s, src);
        const int32_t end = __shfl(e, src);
        const int64_t row = r0 + src;
        if (row >= a.M || end - start > a.th.short_max)
            continue;  // past the end, or routed to the medium/long kinds
        for (int64_t col0 = 0; col0 < a.N; col0 += S::COLS) {
            float acc[S::NV][S::VEC];
            zero_acc<S>(acc);
            for (int32_t base = start; base < end; base += S::G) {
                const int cnt = end - base < S::G ? end - base : S::G;
                if (j < cnt) {
                    Entry en;
                    en.col = a.colind[base + j];
                    en.val = load_val<S::DT>(a.vals, base + j);
                    sg[j] = en;
                }
                consume<S>(sg, cnt, a.B, a.N, col0, j, acc);
            }
            emit_row<S, false>(a.C, row, a.N, col0, j, acc);
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

template <class S>
__global__ __launch_bounds__(kBlock) void worker_kernel(WorkerArgs a,
                                                        int64_t n_tiles,
                                                        int passes,
                                                        int64_t total_waves)
{
    __shared__ Entry stage[kWavesPerBlock][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int g = lane / S::G;
    const int j = lane % S::G;
    Entry *st = stage[wid];

    const PlanCounts pc = *a.plan.counts;
    const int64_t n_ch = pc.n_chunks;
    const int64_t n_med = pc.n_medium;
    const int64_t n_items = n_ch + n_med + n_tiles;
    const int64_t w0 = xcd_logical_block(blockIdx.x, gridDim.x) * kWavesPerBlock + wid;

    for (int64_t item = w0; item < n_items; item += total_waves) {
        if (item < n_ch)
            do_chunk<S>(a, st, lane, g, j, item, pc.n_long);
        else if (item < n_ch + n_med)
            do_medium<S>(a, st, lane, g, j, item - n_ch);
        else
            do_short_tile<S>(a, st, lane, g, j, item - n_ch - n_med, passes);
    }
}

template <class S>
hipError_t launch_shape(const WorkerArgs &a, hipStream_t stream)
{
    static int resident_blocks = 0;  // per variant: blocks that fit at once
    if (resident_blocks == 0) {
        int dev = 0, per_cu = 0, cus = 0;
        hipError_t err = hipGetDevice(&dev);
        if (err == hipSuccess)
            err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (err == hipSuccess)
            err = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, reinterpret_cast<const void *>(worker_kernel<S>), kBlock, 0);
        if (err != hipSuccess)
            return err;
        resident_blocks = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
    }
    // Short tiles: up to 8 passes of R rows (at most 64 rows), fewer when M
    // is too small to give every resident wavefront a tile.
    const int64_t resident_waves = (int64_t)resident_blocks * kWavesPerBlock;
    int64_t passes = a.M / ((int64_t)S::R * resident_waves);
    const int64_t max_passes = kWave / S::R < 8 ? kWave / S::R : 8;
    passes = passes < 1 ? 1 : (passes > max_passes ? max_passes : passes);
    const int64_t tile = passes * S::R;
    const int64_t n_tiles = (a.M + tile - 1) / tile;
    // Items: chunks (unknown on the host) + medium rows (<= M) + tiles.
    const int64_t want_waves = n_tiles + a.M;
    int64_t blocks = (want_waves + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks > resident_blocks)
        blocks = resident_blocks;
    if (blocks < 1)
        blocks = 1;
    hipLaunchKernelGGL(worker_kernel<S>, dim3((unsigned)blocks), dim3(kBlock),
                       0, stream, a, n_tiles, (int)passes,
                       blocks * kWavesPerBlock);
    return hipGetLastError();
}

template <int DT, int VEC>
hipError_t launch_vec(int group, int nv, const WorkerArgs &a, hipStream_t s)
{
    switch (group) {
    case 1: return launch_shape<Shape<DT, VEC, 1, 1>>(a, s);
    case 2: return launch_shape<Shape<DT, VEC, 2, 1>>(a, s);
    case 4: return launch_shape<Shape<DT, VEC, 4, 1>>(a, s);
    case 8: return launch_shape<Shape<DT, VEC, 8, 1>>(a, s);
    case 16: return launch_shape<Shape<DT, VEC, 16, 1>>(a, s);
    case 32: return launch_shape<Shape<DT, VEC, 32, 1>>(a, s);
    case 64:
        if (nv == 1) return launch_shape<Shape<DT, VEC, 64, 1>>(a, s);
        if (nv == 2) return launch_shape<Shape<DT, VEC, 64, 2>>(a, s);
        return launch_shape<Shape<DT, VEC, 64, 4>>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

WorkerConfig choose_worker(int dtype, int64_t N, const void *B, const float *C)
{
    const int esz = dtype == SPMM_DTYPE_BF16 ? 2 : 4;
    const uintptr_t bp = (uintptr_t)B, cp = (uintptr_t)C;
    // Widest lane vector (at most 16 bytes of B) that divides N and whose
    // B loads and C stores are aligned.
    int vec = 16 / esz;
    for (; vec > 1; vec /= 2) {
        const int64_t bbytes = (int64_t)vec * esz;
        const int64_t cbytes = (int64_t)vec * 4 < 16 ? (int64_t)vec * 4 : 16;
        if (N % vec == 0 && bp % bbytes == 0 && cp % cbytes == 0)
            break;
    }
    const int64_t vecs = (N + vec - 1) / vec;  // lane vectors per B row
    int group = 1;
    while (group < 64 && group < vecs)
        group *= 2;
    int64_t nv = (vecs + group - 1) / group;
    nv = nv <= 1 ? 1 : (nv <= 2 ? 2 : 4);
    WorkerConfig cfg;
    cfg.dtype = dtype;
    cfg.vec = vec;
    cfg.group = group;
    cfg.nv = (int)nv;
    return cfg;
}

hipError_t launch_worker(const WorkerConfig &cfg, const WorkerArgs &a,
                         hipStream_t s)
{
    if (cfg.dtype == SPMM_DTYPE_F32) {
        switch (cfg.vec) {
        case 4: return launch_vec<SPMM_DTYPE_F32, 4>(cfg.group, cfg.nv, a, s);
        case 2: return launch_vec<SPMM_DTYPE_F32, 2>(cfg.group, cfg.nv, a, s);
        case 1: return launch_vec<SPMM_DTYPE_F32, 1>(cfg.group, cfg.nv, a, s);
        }
    } else {
        switch (cfg.vec) {
        case 8: return launch_vec<SPMM_DTYPE_BF16, 8>(cfg.group, cfg.nv, a, s);
        case 4: return launch_vec<SPMM_DTYPE_BF16, 4>(cfg.group, cfg.nv, a, s);
        case 2: return launch_vec<SPMM_DTYPE_BF16, 2>(cfg.group, cfg.nv, a, s);
        case 1: return launch_vec<SPMM_DTYPE_BF16, 1>(cfg.group, cfg.nv, a, s);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace sdl
