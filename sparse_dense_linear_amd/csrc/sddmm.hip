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
//     VEC elements), multiplies them element-wise, sums the lane's part,
//     and the group adds its G parts with butterfly shuffles; U entries per
//     group are in flight at once;
//   * the 64 results are gathered in LDS and written with one coalesced
//     store.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "internal.h"
#include "span.h"
#include "spmm.h"

namespace sdl {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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
    static_assert((kWave / R) % U == 0, "a batch is a whole number of steps");
};

template <class S>
__global__ __launch_bounds__(kBlock) void sddmm_kernel(
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
        const int64_t e = e0 + lane;
        const bool live = e < s1;
        const int64_t pe = base + (live ? e : s1 - 1);
        const int32_t col = colind[pe];

        const int64_t row = row_in_window(rowptr, M, i_cur, pe, lane);
        i_cur = __shfl(row, kWave - 1);

        // The 64 dot products: group g takes entries k = u * R + g.
        for (int u0 = 0; u0 < kWave / S::R; u0 += S::U) {
            float part[S::U];
#pragma unroll
            for (int u = 0; u < S::U; ++u)
                part[u] = 0.0f;
            int64_t ci[S::U], bj[S::U];
#pragma unroll
            for (int u = 0; u < S::U; ++u) {
                const int k = (u0 + u) * S::R + g;
                ci[u] = __shfl(row, k) * N;
                bj[u] = (int64_t)__shfl(col, k) * N;
            }
            for (int64_t col0 = 0; col0 < N; col0 += S::COLS) {
                // lanes past the end of the row read its last vector and
                // contribute nothing
                const int64_t c = col0 + (int64_t)jl * S::VEC;
                const bool in = c < N;
                const int64_t cc = in ? c : N - S::VEC;
                float cv[S::U][S::VEC], bv[S::U][S::VEC];
#pragma unroll
                for (int u = 0; u < S::U; ++u) {
                    RowLoad<S::DT, S::VEC>::load(C, ci[u] + cc, cv[u]);
                    RowLoad<S::DT, S::VEC>::load(B, bj[u] + cc, bv[u]);
                }
#pragma unroll
                for (int u = 0; u < S::U; ++u) {
                    float d = 0.0f;
#pragma unroll
                    for (int x = 0; x < S::VEC; ++x)
                        d = __builtin_fmaf(cv[u][x], bv[u][x], d);
                    part[u] += in ? d : 0.0f;
                }
            }
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
        if (live)
            A[e] = res[wid][lane];
    }
}

template <class S>
hipError_t launch_sd(const SddmmArgs &a, hipStream_t stream, hipEvent_t e0,
                     hipEvent_t e1)
{
    static int resident_blocks = 0;
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

}  // namespace

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
