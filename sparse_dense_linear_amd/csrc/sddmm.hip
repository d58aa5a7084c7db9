// sddmm.hip -- sampled dense-dense product (SDDMM) on a CSR pattern, gfx950.
//
// Page: [IntelMax] "Performance Optimization of Deep Learning Sparse Matrix
// Kernels on Intel Max Series GPU", the SDDMM operation (Fig. 3,
// Algorithm 1) and its ESIMD kernel: the stored entry p of row i, at column
// j = colind[p], gets the dot product of row C_i (C dense M x N) with row
// B_j (B dense K x N, i.e. column j of B^T).  The page splits a row's
// entries equally among NT workers; here every stored entry is its own unit
// of work, so the entries are split equally among all wavefronts
// regardless of rows (every entry costs the same: two row reads and a dot
// product), and no output is shared between wavefronts.
//
// One wavefront takes the span [s0, s1) of entry positions (relative to
// rowptr[0]) and walks it 64 entries at a time:
//   * the row of the span's first entry is found by a 64-ary search over
//     rowptr (each round, the 64 lanes probe 64 evenly spaced rows);
//   * for a batch of 64 entries (lane l: entry e0 + l), lane l also holds
//     rowptr[i_cur + 1 + l] of the current row window, and each lane finds
//     its entry's row by a binary search over that window (shuffles); a
//     batch that runs past 64 rows (empty rows) moves the window on;
//   * the 64 dot products are computed by R = 64/G groups of G lanes: for
//     entry k the group reads C_i and B_j as 16-byte vectors (one per lane,
//     VEC elements), multiplies them element-wise and sums the lane's part;
//     U entries per group are in flight at once, and when all of them lie in
//     one row (long rows) the C_i vector is loaded once for the U;
//   * the group adds its G parts with butterfly shuffles, and the 64 results
//     are gathered in LDS and written with one coalesced store; or, for one
//     64-lane group of fp32 rows, each lane keeps its parts of all 64 entries
//     and a reduce-scatter leaves entry u's total in one lane (63 shuffles
//     per lane instead of 6 per entry), summed in the butterfly's order.
#include <hip/hip_ext.h>

#include <atomic>
#include <hip/hip_runtime.h>

#include "internal.h"
#include "span.h"
#include "spmm.h"

namespace sdl {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// VEC consecutive elements of a dense row, widened exactly to fp32.
template <int DT, int VEC> struct RowLoad;

template <> struct RowLoad<SPMM_DTYPE_F32, 4> {
    static __device__ void load(const void *base, int64_t idx, float (&o)[4])
    {
        const f32x4 v = *(const f32x4 *)((const float *)base + idx);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
};
template <> struct RowLoad<SPMM_DTYPE_F32, 1> {
    static __device__ void load(const void *base, int64_t idx, float (&o)[1])
    { o[0] = ((const float *)base)[idx]; }
};
template <> struct RowLoad<SPMM_DTYPE_BF16, 8> {
    static __device__ void load(const void *base, int64_t idx, float (&o)[8])
    {
        const u32x4 v = *(const u32x4 *)((const uint16_t *)base + idx);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            o[2 * q] = __uint_as_float(w[q] << 16);
            o[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
        }
    }
};
template <> struct RowLoad<SPMM_DTYPE_BF16, 1> {
    static __device__ void load(const void *base, int64_t idx, float (&o)[1])
    { o[0] = __uint_as_float((uint32_t)((const uint16_t *)base)[idx] << 16); }
};

template <int DT_, int VEC_, int G_>
struct SdShape {
    static constexpr int DT = DT_;
    static constexpr int VEC = VEC_;
    static constexpr int G = G_;
    static constexpr int R = kWave / G_;   // groups per wavefront
    static constexpr int COLS = G_ * VEC_; // columns per pass over a row
    static constexpr int U = 4;            // entries per group in flight
    static constexpr int LOGG = G_ == 1 ? 0 : G_ == 2 ? 1 : G_ == 4 ? 2 : G_ == 8 ? 3
                              : G_ == 16 ? 4 : G_ == 32 ? 5 : 6;
    static_assert((1 << LOGG) == G_, "G is a power of two up to 64");
    static_assert(G_ % U == 0, "a group's G entries are a whole number of steps");
    // RS: one 64-lane group per wavefront, whose 64 dot products are
    // finished by a reduce-scatter (fp32 operands; with bf16 the 64 partial
    // sums per lane do not fit beside the wider loads).  It holds 64 partial
    // sums per lane: ask for registers that still allow 3 wavefronts per SIMD.
    static constexpr bool RS = G_ == kWave && DT_ == SPMM_DTYPE_F32;
    static constexpr int MIN_WAVES = RS ? 3 : 1;
};

// This lane's parts of NU dot products <C row ci[u], B row bj[u]> (offsets
// in elements): over the column passes, a chain of fused multiply-adds per
// vector; lanes past the end of the row read its last vector and contribute
// nothing.  ONE_ROW: all ci[u] are equal, and the C vector is loaded once.
template <class S, bool ONE_ROW, int NU>
__device__ inline void dots(const void *__restrict__ C, const void *__restrict__ B,
                            const int64_t *ci, const int64_t *bj, int64_t N,
                            int jl, float *part)
{
#pragma unroll
    for (int u = 0; u < NU; ++u)
        part[u] = 0.0f;
    for (int64_t col0 = 0; col0 < N; col0 += S::COLS) {
        const int64_t c = col0 + (int64_t)jl * S::VEC;
        const bool in = c < N;
        const int64_t cc = in ? c : N - S::VEC;
        constexpr int NC = ONE_ROW ? 1 : NU;
        if constexpr (S::DT == SPMM_DTYPE_BF16 && S::VEC == 8) {
            // bf16: one v_dot2 per pair of neighbouring columns (exact
            // products, fp32 sum), on the words as loaded
            u32x4 cw[NC], bw[NU];
#pragma unroll
            for (int u = 0; u < NC; ++u)
                cw[u] = *(const u32x4 *)((const uint16_t *)C + ci[u] + cc);
#pragma unroll
            for (int u = 0; u < NU; ++u)
                bw[u] = *(const u32x4 *)((const uint16_t *)B + bj[u] + cc);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const u32x4 c4 = cw[ONE_ROW ? 0 : u];
                const uint32_t cq[4] = {c4.x, c4.y, c4.z, c4.w};
                const uint32_t bq[4] = {bw[u].x, bw[u].y, bw[u].z, bw[u].w};
                float d = 0.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, cq[q]),
                                                        __builtin_bit_cast(bf16x2_t, bq[q]),
                                                        d, false);
                part[u] += in ? d : 0.0f;
            }
        } else {
            float cv[NC][S::VEC], bv[NU][S::VEC];
#pragma unroll
            for (int u = 0; u < NC; ++u)
                RowLoad<S::DT, S::VEC>::load(C, ci[u] + cc, cv[u]);
#pragma unroll
            for (int u = 0; u < NU; ++u)
                RowLoad<S::DT, S::VEC>::load(B, bj[u] + cc, bv[u]);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                float d = 0.0f;
#pragma unroll
                for (int x = 0; x < S::VEC; ++x)
                    d = __builtin_fmaf(cv[ONE_ROW ? 0 : u][x], bv[u][x], d);
                part[u] += in ? d : 0.0f;
            }
        }
    }
}

// Rows of C and B (element offsets) of group g's entries u0 .. u0+U-1 of
// the batch (entry k = u * R + g, held by lane k).
template <class S>
__device__ inline void entry_rows(int64_t row, int32_t col, int64_t N, int u0,
                                  int g, int64_t (&ci)[S::U], int64_t (&bj)[S::U])
{
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
        const int k = (u0 + u) * S::R + g;
        ci[u] = __shfl(row, k) * N;
        bj[u] = (int64_t)__shfl(col, k) * N;
    }
}

template <class S>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(S::MIN_WAVES)))
void sddmm_kernel(
    const int32_t *__restrict__ rowptr, const int32_t *__restrict__ colind,
    const void *__restrict__ C, const void *__restrict__ B,
    float *__restrict__ A, int64_t M, int64_t N, int64_t nnz, int64_t span)
{
    __shared__ float res[kWavesPerBlock][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int g = lane / S::G;
    const int jl = lane % S::G;
    const int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + wid;
    const int64_t base = rowptr[0];
    // Never go past the pattern itself, whatever nnz the caller passed: an
    // inconsistent nnz leaves values unwritten but reads nothing outside
    // colind and writes nothing outside A.
    const int64_t stored = (int64_t)rowptr[M] - base;
    const int64_t n = nnz < stored ? nnz : stored;
    const int64_t s0 = w * span;
    const int64_t s1 = s0 + span < n ? s0 + span : n;
    if (s0 >= s1)
        return;
    int64_t i_cur = find_row(rowptr, M, base + s0, lane);

    for (int64_t e0 = s0; e0 < s1; e0 += kWave) {
        const int64_t pe = base + (e0 + lane < s1 ? e0 + lane : s1 - 1);
        const int32_t col = colind[pe];

        const int64_t row = row_in_window(rowptr, M, i_cur, pe, lane);
        i_cur = __shfl(row, kWave - 1);

        if constexpr (S::RS) {
            // One group (the whole wavefront) takes all 64 entries; part[u]
            // is this lane's part of entry u's dot product.
            float part[S::G];
#pragma unroll
            for (int u0 = 0; u0 < S::G; u0 += S::U) {
                int64_t ci[S::U], bj[S::U];
                entry_rows<S>(row, col, N, u0, g, ci, bj);
                if (__all(ci[0] == ci[S::U - 1]))
                    dots<S, true, S::U>(C, B, ci, bj, N, jl, part + u0);
                else
                    dots<S, false, S::U>(C, B, ci, bj, N, jl, part + u0);
                // one step's loads at a time (the steps are unrolled only so
                // that part[] has fixed indices)
                __builtin_amdgcn_sched_barrier(0);
            }
            // Reduce-scatter over the 64 lanes: at each stage a lane keeps
            // half of its partial sums and sends the other half to the lane
            // that differs in one bit, adding what it receives.  The lowest
            // bit goes first, so each total is added up in the same order as
            // the butterfly below; the total of entry u ends in lane
            // bitrev(u).  63 shuffles per lane instead of 6 per entry.
#pragma unroll
            for (int b = 0; b < S::LOGG; ++b) {
                const int h = 1 << b;                 // partner distance
                const int half = S::G >> (b + 1);     // values kept after this stage
                const bool upper = (jl & h) != 0;
#pragma unroll
                for (int i = 0; i < half; ++i) {
                    const float send = upper ? part[i] : part[i + half];
                    const float keep = upper ? part[i + half] : part[i];
                    part[i] = keep + __shfl_xor(send, h);
                }
            }
            const int u = (int)(__builtin_bitreverse32((uint32_t)jl) >> (32 - S::LOGG));
            const int64_t eu = e0 + (int64_t)u * S::R + g;
            if (eu < s1)
                __builtin_nontemporal_store(part[0], A + eu);  // written once
        } else {
            // Group g takes entries k = u * R + g; each step's U dot products
            // are finished by a butterfly over the group's lanes (lane l adds
            // lane l ^ 1, then l ^ 2, ...), and the 64 results are gathered in
            // LDS for one coalesced store.
            for (int u0 = 0; u0 < S::G; u0 += S::U) {
                int64_t ci[S::U], bj[S::U];
                entry_rows<S>(row, col, N, u0, g, ci, bj);
                float part[S::U];
                if (__all(ci[0] == ci[S::U - 1]))
                    dots<S, true, S::U>(C, B, ci, bj, N, jl, part);
                else
                    dots<S, false, S::U>(C, B, ci, bj, N, jl, part);
                // this batch's results go to res only after every lane has
                // read the previous batch's
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int u = 0; u < S::U; ++u) {
                    float d = part[u];
#pragma unroll
                    for (int off = 1; off < S::G; off <<= 1)
                        d += __shfl_xor(d, off);
                    if (jl == 0)
                        res[wid][(u0 + u) * S::R + g] = d;
                }
            }
            __builtin_amdgcn_wave_barrier();  // all 64 results are in res
            if (e0 + lane < s1)
                __builtin_nontemporal_store(res[wid][lane], A + e0 + lane);
        }
    }
}

template <class S>
hipError_t launch_sd(const SddmmArgs &a, hipStream_t stream, hipEvent_t e0,
                     hipEvent_t e1)
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
                &per_cu, reinterpret_cast<const void *>(sddmm_kernel<S>), kBlock, 0);
        if (err != hipSuccess)
            return err;
        resident_blocks = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
        resident_cache.store(resident_blocks, std::memory_order_relaxed);
    }
    // Equal spans of whole 64-entry batches, one per resident wavefront
    // (fewer when there are fewer batches).
    const int64_t batches = (a.nnz + kWave - 1) / kWave;
    const int64_t waves_max = (int64_t)resident_blocks * kWavesPerBlock;
    const int64_t per_wave = (batches + waves_max - 1) / waves_max;
    const int64_t span = per_wave * kWave;
    const int64_t waves = (a.nnz + span - 1) / span;
    const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    hipExtLaunchKernelGGL(sddmm_kernel<S>, dim3((unsigned)blocks), dim3(kBlock), 0,
                          stream, e0, e1, 0, a.rowptr, a.colind, a.C, a.B, a.A,
                          a.M, a.N, a.nnz, span);
    return hipGetLastError();
}

template <int DT, int VEC>
hipError_t launch_sd_vec(int group, const SddmmArgs &a, hipStream_t s,
                         hipEvent_t e0, hipEvent_t e1)
{
    switch (group) {
    case 4: return launch_sd<SdShape<DT, VEC, 4>>(a, s, e0, e1);
    case 8: return launch_sd<SdShape<DT, VEC, 8>>(a, s, e0, e1);
    case 16: return launch_sd<SdShape<DT, VEC, 16>>(a, s, e0, e1);
    case 32: return launch_sd<SdShape<DT, VEC, 32>>(a, s, e0, e1);
    case 64: return launch_sd<SdShape<DT, VEC, 64>>(a, s, e0, e1);
    default: return hipErrorInvalidValue;
    }
}

__global__ __launch_bounds__(kBlock) void widen_bf16_kernel(const uint16_t *__restrict__ in,
                                                           float *__restrict__ out, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride)
        out[i] = __uint_as_float((uint32_t)in[i] << 16);
}

}  // namespace

hipError_t launch_widen_bf16(const uint16_t *in, float *out, int64_t n, hipStream_t stream)
{
    if (n <= 0)
        return hipSuccess;
    int64_t blocks = (n + kBlock - 1) / kBlock;
    if (blocks > 8192)
        blocks = 8192;  // grid-stride beyond that
    hipLaunchKernelGGL(widen_bf16_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, stream,
                       in, out, n);
    return hipGetLastError();
}

hipError_t launch_sddmm(const SddmmArgs &a, hipStream_t stream, hipEvent_t e0,
                        hipEvent_t e1)
{
    // 16-byte vectors when N and both dense operands allow them.
    const int esz = a.dtype == SPMM_DTYPE_BF16 ? 2 : 4;
    const int wide = 16 / esz;
    const bool aligned = a.N % wide == 0 && ((uintptr_t)a.C) % 16 == 0 &&
                         ((uintptr_t)a.B) % 16 == 0;
    const int vec = aligned ? wide : 1;
    const int64_t vecs = (a.N + vec - 1) / vec;
    int group = 4;
    while (group < 64 && group < vecs)
        group *= 2;
    if (a.dtype == SPMM_DTYPE_F32)
        return vec == 4 ? launch_sd_vec<SPMM_DTYPE_F32, 4>(group, a, stream, e0, e1)
                        : launch_sd_vec<SPMM_DTYPE_F32, 1>(group, a, stream, e0, e1);
    return vec == 8 ? launch_sd_vec<SPMM_DTYPE_BF16, 8>(group, a, stream, e0, e1)
                    : launch_sd_vec<SPMM_DTYPE_BF16, 1>(group, a, stream, e0, e1);
}

}  // namespace sdl
