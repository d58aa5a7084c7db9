// gather.h -- device building blocks shared by the product kernels: lane
// groups and their column layout, exact loads of B vectors (fp32 or bf16),
// the staged (column, value) entries, batches of U gathers issued without
// branches, accumulation, row stores and the reduction across groups, and
// the FusedMM pieces (a group's dot product <X_i, Y_j> formed where the
// value is used).
// Included by worker.hip and eb.hip (each keeps its own copy: everything
// here is in an anonymous namespace).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
// load() takes a flat address; load_buf() a byte offset into a buffer
// resource covering B (used when B is below 4 GiB: one 32-bit offset per
// gather instead of a 64-bit address).
template <int DT, int VEC> struct BLoad;

template <> struct BLoad<SPMM_DTYPE_F32, 4> {
    typedef f32x4 raw;
    static __device__ raw load(const void *p) { return *(const f32x4 *)p; }
    static __device__ raw load_buf(__amdgpu_buffer_rsrc_t r, uint32_t off)
    { return __builtin_bit_cast(raw, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0)); }
    static __device__ void widen(const raw &r, float (&o)[4])
    { o[0] = r.x; o[1] = r.y; o[2] = r.z; o[3] = r.w; }
};
template <> struct BLoad<SPMM_DTYPE_F32, 2> {
    typedef f32x2 raw;
    static __device__ raw load(const void *p) { return *(const f32x2 *)p; }
    static __device__ raw load_buf(__amdgpu_buffer_rsrc_t r, uint32_t off)
    { return __builtin_bit_cast(raw, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0)); }
    static __device__ void widen(const raw &r, float (&o)[2])
    { o[0] = r.x; o[1] = r.y; }
};
template <> struct BLoad<SPMM_DTYPE_F32, 1> {
    typedef float raw;
    static __device__ raw load(const void *p) { return *(const float *)p; }
    static __device__ raw load_buf(__amdgpu_buffer_rsrc_t r, uint32_t off)
    { return __builtin_bit_cast(raw, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0)); }
    static __device__ void widen(const raw &r, float (&o)[1]) { o[0] = r; }
};
template <> struct BLoad<SPMM_DTYPE_BF16, 8> {
    typedef u32x4 raw;
    static __device__ raw load(const void *p) { return *(const u32x4 *)p; }
    static __device__ raw load_buf(__amdgpu_buffer_rsrc_t r, uint32_t off)
    { return __builtin_bit_cast(raw, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0)); }
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
    static __device__ raw load_buf(__amdgpu_buffer_rsrc_t r, uint32_t off)
    { return __builtin_bit_cast(raw, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0)); }
    static __device__ void widen(const raw &r, float (&o)[4])
    {
        o[0] = bf16_lo(r.x); o[1] = bf16_hi(r.x);
        o[2] = bf16_lo(r.y); o[3] = bf16_hi(r.y);
    }
};
template <> struct BLoad<SPMM_DTYPE_BF16, 2> {
    typedef uint32_t raw;
    static __device__ raw load(const void *p) { return *(const uint32_t *)p; }
    static __device__ raw load_buf(__amdgpu_buffer_rsrc_t r, uint32_t off)
    { return __builtin_bit_cast(raw, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0)); }
    static __device__ void widen(const raw &r, float (&o)[2])
    { o[0] = bf16_lo(r); o[1] = bf16_hi(r); }
};
template <> struct BLoad<SPMM_DTYPE_BF16, 1> {
    typedef uint16_t raw;
    static __device__ raw load(const void *p) { return *(const uint16_t *)p; }
    static __device__ raw load_buf(__amdgpu_buffer_rsrc_t r, uint32_t off)
    { return __builtin_bit_cast(raw, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0)); }
    static __device__ void widen(const raw &r, float (&o)[1])
    { o[0] = __uint_as_float((uint32_t)r << 16); }
};

template <int DT> struct ElemSize;
template <> struct ElemSize<SPMM_DTYPE_F32> { static constexpr int v = 4; };
template <> struct ElemSize<SPMM_DTYPE_BF16> { static constexpr int v = 2; };

// Word 3 of a raw buffer resource on the gfx9 family (gfx950): 32-bit
// elements, no swizzle; with stride 0 the record count is a byte count and
// loads past it return zero.
constexpr int kBufferWord3 = 0x00020000;

// A stored entry as staged in LDS: column and value (already fp32).
struct Entry {
    int32_t col;
    float val;
};

// Per-wavefront LDS staging area.  A short tile stages at most kShortCap
// entries (the host sizes tiles so that T * short_max <= kShortCap); medium
// rows and long chunks use the first 64 entries.
constexpr int kStageSlots = kShortCap / kWave;  // staged entries per lane

struct WaveStage {
    Entry ent[kShortCap];
    uint8_t rid[kShortCap];   // row of the entry within its tile
};

template <int DT> __device__ inline float load_val(const void *vals, int64_t p);
template <> __device__ inline float load_val<SPMM_DTYPE_F32>(const void *vals, int64_t p)
{ return ((const float *)vals)[p]; }
template <> __device__ inline float load_val<SPMM_DTYPE_BF16>(const void *vals, int64_t p)
{ return __uint_as_float((uint32_t)((const uint16_t *)vals)[p] << 16); }

// Compile-time shape of one worker variant.  FUSED: the FusedMM variant,
// whose entry values are computed on the fly (two gathers per entry, so
// half as many entries in flight).  Every variant runs at 4 wavefronts per
// SIMD: 16 gathers in flight per lane for whole fp32 rows of 256 columns at
// 3 wavefronts per SIMD measured 5-11 % slower than 8 at 4 (pruned 4096^2,
// N = 192 and 256), once queues stopped reserving items ahead.
// PAIR: the product form for a B larger than the Infinity Cache whose rows
// are two column passes wide: medium rows are taken four at a time, one
// column half per item (see call_kernel).
template <int DT_, int VEC_, int G_, int NV_, bool BUF_, bool FUSED_ = false,
          bool PAIR_ = false>
struct Shape {
    static constexpr bool BUF = BUF_;   // B addressed through a buffer resource
    static constexpr bool FUSED = FUSED_;
    static constexpr bool PAIR = PAIR_;
    static constexpr int DT = DT_;
    static constexpr int VEC = VEC_;
    static constexpr int G = G_;
    static constexpr int NV = NV_;
    static constexpr int R = kWave / G_;          // groups per wavefront
    static constexpr int COLS = G_ * VEC_ * NV_;  // columns per column pass
    static constexpr int U0 = NV_ == 1 ? 8 : (NV_ == 2 ? 4 : 2);
    static constexpr int U = FUSED_ ? (U0 / 2 > 1 ? U0 / 2 : 1) : U0;  // entries in flight
    static constexpr int MIN_WAVES = 4;   // wavefronts per SIMD
    static constexpr int ESZ = ElemSize<DT_>::v;
};

// Byte offsets (within a row of B) of this lane's NV vectors for the column
// pass starting at col0, and whether each lies inside the row.  Lanes past
// the end of the row read the row's last full vector instead, so every load
// has a valid address and none needs a branch.
template <class S>
struct LaneCols {
    int64_t ofs[S::NV];
    bool live[S::NV];
};

template <class S>
__device__ inline LaneCols<S> lane_cols(int64_t N, int64_t col0, int j)
{
    LaneCols<S> lc;
#pragma unroll
    for (int k = 0; k < S::NV; ++k) {
        const int64_t c = col0 + (int64_t)(k * S::G + j) * S::VEC;
        lc.live[k] = c < N;
        lc.ofs[k] = (c < N ? c : N - S::VEC) * S::ESZ;
    }
    return lc;
}

// Where B lives: a buffer resource (BUF) or a flat pointer.
struct BSrc {
    __amdgpu_buffer_rsrc_t rsrc;
    const char *base;
};

// One batch of up to U gathers of a lane group: the raw B vectors and the
// entry values.
template <class S>
struct Batch {
    typename BLoad<S::DT, S::VEC>::raw buf[S::U][S::NV];
    float v[S::U];
};

// Vector k of this lane's columns of row `row` of a K x N operand.
template <class S>
__device__ inline typename BLoad<S::DT, S::VEC>::raw
load_row_vec(const BSrc &src, int32_t row, uint32_t row_bytes,
             const LaneCols<S> &lc, int k)
{
    typedef BLoad<S::DT, S::VEC> L;
    if constexpr (S::BUF)
        return L::load_buf(src.rsrc, (uint32_t)row * row_bytes + (uint32_t)lc.ofs[k]);
    else
        return L::load(src.base + (uint64_t)(uint32_t)row * row_bytes + lc.ofs[k]);
}

// Gather slots with no entry.  For bf16 B read through a buffer resource
// (outside FusedMM, whose values come from gathered rows) such a slot is
// made a no-op at issue: value -0 and a load past the record count, which
// reads +0, so fma(-0, +0, acc) = acc + (-0) = acc for every acc, -0,
// infinities and NaN included, and the accumulation needs no select.
// Otherwise the slot repeats a valid entry and accumulate() selects the
// old acc.  Measured (same box, A/B): the pruned 4096-row bf16 product
// 53.1 -> 46.1 us and the skewed bf16 one 7.02 -> 6.66 ms, where the
// widening already costs one instruction per element; for fp32 B the
// selects-free form was 7-9 % slower (pruned, power-law; the loads past
// the record count alone cost nothing), so fp32 keeps the selects.
template <class S>
constexpr bool kSlotsZeroed = S::BUF && !S::FUSED && S::DT == SPMM_DTYPE_BF16;

template <class S>
__device__ inline typename BLoad<S::DT, S::VEC>::raw
load_slot_vec(const BSrc &src, int32_t row, uint32_t row_bytes,
              const LaneCols<S> &lc, int k, bool on)
{
    typedef BLoad<S::DT, S::VEC> L;
    if constexpr (kSlotsZeroed<S>)
        return L::load_buf(src.rsrc, on ? (uint32_t)row * row_bytes + (uint32_t)lc.ofs[k]
                                        : kNoRowOffset);
    else
        return load_row_vec<S>(src, row, row_bytes, lc, k);
}

// Issue the gathers of entries st[q .. q+n) (0 <= n <= U; st[q] exists)
// back to back, with no branches; slots past n are no-ops or repeat entry
// q (see kSlotsZeroed).
template <class S>
__device__ inline void issue(Batch<S> &bt, const Entry *st, int q, int n,
                             const BSrc &src, uint32_t row_bytes,
                             const LaneCols<S> &lc)
{
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
        const bool on = u < n;
        const Entry e = st[on ? q + u : q];
        bt.v[u] = kSlotsZeroed<S> && !on ? -0.0f : e.val;
#pragma unroll
        for (int k = 0; k < S::NV; ++k)
            bt.buf[u][k] = load_slot_vec<S>(src, e.col, row_bytes, lc, k, on);
    }
}

// acc += v * B-vector when `on`; otherwise acc is left as it was: a
// no-op slot adds -0, any other unused slot is a select, not a branch, so
// its value never matters.
template <class S>
__device__ inline void axpy(const typename BLoad<S::DT, S::VEC>::raw (&buf)[S::NV],
                            float v, bool on, float (&acc)[S::NV][S::VEC])
{
    typedef BLoad<S::DT, S::VEC> L;
#pragma unroll
    for (int k = 0; k < S::NV; ++k) {
        float b[S::VEC];
        L::widen(buf[k], b);
#pragma unroll
        for (int x = 0; x < S::VEC; ++x) {
            const float t = fmaf(v, b[x], acc[k][x]);
            acc[k][x] = kSlotsZeroed<S> || on ? t : acc[k][x];
        }
    }
}

template <class S>
__device__ inline void accumulate(const Batch<S> &bt, int u, bool on,
                                  float (&acc)[S::NV][S::VEC])
{
    axpy<S>(bt.buf[u], bt.v[u], on, acc);
}

// Two entries of one row at once, for bf16 B with zeroed slots: for each
// column, the two entries' elements of B are paired in one register (a
// byte permute) and added in with one v_dot2 (bf16 x bf16 products, exact,
// summed into the fp32 accumulator): two instructions per two products
// instead of four (two widenings, two multiply-adds).  Each dot pairs the
// same column of two entries, so a non-finite element stays in its column,
// and a zeroed slot's -0 x +0 adds -0.  Its rounding is not a single one:
// over 2^20 random cases its error stayed within 2.5 x 2^-24 of
// |a0 b0| + |a1 b1| + |acc| (two fp32 multiply-adds: within 2 x 2^-24),
// with denormals kept.  Measured (A/B, one box): pruned 4096-row bf16
// product 46.3 -> 43.4 us, skewed bf16 6.69 -> 6.45 ms.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <class S>
constexpr bool kPairDot = kSlotsZeroed<S> && (S::VEC == 2 || S::VEC == 4 || S::VEC == 8) &&
                          S::U % 2 == 0;

template <class S>
__device__ inline void accumulate_two(const Batch<S> &bt, int u, float (&acc)[S::NV][S::VEC])
{
    constexpr int D = S::VEC / 2;  // 32-bit words (column pairs) per vector
    // the two values as one bf16 pair: entry u low, entry u+1 high
    const uint32_t vv = __builtin_amdgcn_perm(__float_as_uint(bt.v[u + 1]),
                                              __float_as_uint(bt.v[u]), 0x07060302u);
    const bf16x2_t vp = __builtin_bit_cast(bf16x2_t, vv);
#pragma unroll
    for (int k = 0; k < S::NV; ++k) {
        uint32_t w0[D], w1[D];
        __builtin_memcpy(w0, &bt.buf[u][k], sizeof(w0));
        __builtin_memcpy(w1, &bt.buf[u + 1][k], sizeof(w1));
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const bf16x2_t lo = __builtin_bit_cast(bf16x2_t,
                __builtin_amdgcn_perm(w1[d], w0[d], 0x05040100u));
            const bf16x2_t hi = __builtin_bit_cast(bf16x2_t,
                __builtin_amdgcn_perm(w1[d], w0[d], 0x07060302u));
            acc[k][2 * d] = __builtin_amdgcn_fdot2_f32_bf16(lo, vp, acc[k][2 * d], false);
            acc[k][2 * d + 1] = __builtin_amdgcn_fdot2_f32_bf16(hi, vp, acc[k][2 * d + 1], false);
        }
    }
}

// Group-local SAXPY over entries first .. first+cnt-1 of a chunk held one
// per lane (lane k: column `col`, value `val`), read by lane shuffles:
// acc += val * B[col, this lane's columns], U gathers at a time.
template <class S>
__device__ inline void consume_lanes(int32_t col, float val, int first, int cnt,
                                     const BSrc &src, uint32_t row_bytes,
                                     const LaneCols<S> &lc, float (&acc)[S::NV][S::VEC])
{
    for (int u0 = 0; u0 < cnt; u0 += S::U) {
        const int n = cnt - u0 < S::U ? cnt - u0 : S::U;
        Batch<S> bt;
#pragma unroll
        for (int u = 0; u < S::U; ++u) {
            const bool on = u < n;
            const int from = first + (on ? u0 + u : u0);
            const int32_t c = __shfl(col, from);
            const float v = __shfl(val, from);
            bt.v[u] = kSlotsZeroed<S> && !on ? -0.0f : v;
#pragma unroll
            for (int k = 0; k < S::NV; ++k)
                bt.buf[u][k] = load_slot_vec<S>(src, c, row_bytes, lc, k, on);
        }
        if constexpr (kPairDot<S>) {
#pragma unroll
            for (int x = 0; x < S::U; x += 2)
                accumulate_two<S>(bt, x, acc);
        } else {
#pragma unroll
            for (int x = 0; x < S::U; ++x)
                accumulate<S>(bt, x, x < n, acc);
        }
    }
}

// FusedMM.  The value of an entry of row i at column j is <X_i, Y_j> (X the
// M x N row operand, Y the K x N column operand), formed by the lane group
// that holds the whole row (one column pass): each lane sums its vectors in
// order (a chain of fused multiply-adds per vector, vectors past the end of
// the row left out), then a butterfly over the group's G lanes adds the
// parts.  This is the SDDMM kernel's order when the two use the same group
// width, so the value is the SDDMM value bit for bit.  bf16 vectors of 8:
// the chain is one v_dot2 per pair of neighbouring columns (both operands
// bf16, exact products, fp32 sum), as in the SDDMM kernel.
template <class S>
__device__ inline float group_dot(const typename BLoad<S::DT, S::VEC>::raw (&x)[S::NV],
                                  const typename BLoad<S::DT, S::VEC>::raw (&y)[S::NV],
                                  const LaneCols<S> &lc)
{
    typedef BLoad<S::DT, S::VEC> L;
    float d = 0.0f;
#pragma unroll
    for (int k = 0; k < S::NV; ++k) {
        float dk = 0.0f;
        if constexpr (S::DT == SPMM_DTYPE_BF16 && S::VEC == 8) {
            uint32_t xw[4], yw[4];
            __builtin_memcpy(xw, &x[k], sizeof(xw));
            __builtin_memcpy(yw, &y[k], sizeof(yw));
#pragma unroll
            for (int q = 0; q < 4; ++q)
                dk = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xw[q]),
                                                     __builtin_bit_cast(bf16x2_t, yw[q]),
                                                     dk, false);
        } else {
            float xv[S::VEC], yv[S::VEC];
            L::widen(x[k], xv);
            L::widen(y[k], yv);
#pragma unroll
            for (int e = 0; e < S::VEC; ++e)
                dk = fmaf(xv[e], yv[e], dk);
        }
        d += lc.live[k] ? dk : 0.0f;
    }
#pragma unroll
    for (int off = 1; off < S::G; off <<= 1)
        d += __shfl_xor(d, off);
    return d;
}

// This lane's columns of row `row` of the M x N row operand (flat address),
// as loaded.
template <class S>
__device__ inline void load_x_row(const char *X, int64_t row, uint32_t row_bytes,
                                  const LaneCols<S> &lc,
                                  typename BLoad<S::DT, S::VEC>::raw (&x)[S::NV])
{
    typedef BLoad<S::DT, S::VEC> L;
#pragma unroll
    for (int k = 0; k < S::NV; ++k)
        x[k] = L::load(X + (uint64_t)row * row_bytes + lc.ofs[k]);
}

// FusedMM over entries first .. first+cnt-1 of a chunk held one per lane
// (column in lane k's `col`), all in the row whose X slice this lane holds:
// acc += <X_i, Y_j> * D_j.  Both gathers of a batch are issued before any
// value is formed.
template <class S>
__device__ inline void consume_lanes_fused(int32_t col, int first, int cnt,
                                           const BSrc &dsrc, const BSrc &ysrc,
                                           uint32_t row_bytes, const LaneCols<S> &lc,
                                           const typename BLoad<S::DT, S::VEC>::raw (&x)[S::NV],
                                           float (&acc)[S::NV][S::VEC])
{
    typedef typename BLoad<S::DT, S::VEC>::raw Raw;
    for (int u0 = 0; u0 < cnt; u0 += S::U) {
        const int n = cnt - u0 < S::U ? cnt - u0 : S::U;
        int32_t c[S::U];
        Raw yb[S::U][S::NV], db[S::U][S::NV];
#pragma unroll
        for (int u = 0; u < S::U; ++u) {
            c[u] = __shfl(col, first + (u < n ? u0 + u : u0));
#pragma unroll
            for (int k = 0; k < S::NV; ++k)
                yb[u][k] = load_row_vec<S>(ysrc, c[u], row_bytes, lc, k);
        }
#pragma unroll
        for (int u = 0; u < S::U; ++u)
#pragma unroll
            for (int k = 0; k < S::NV; ++k)
                db[u][k] = load_row_vec<S>(dsrc, c[u], row_bytes, lc, k);
#pragma unroll
        for (int u = 0; u < S::U; ++u)
            axpy<S>(db[u], group_dot<S>(x, yb[u], lc), u < n, acc);
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

// Store (or atomically add) this lane's columns of one C row.  Plain stores
// are nontemporal: C is written once and not read again by the call, so its
// lines need not displace gathered B rows from the caches (measured faster
// on every workload).
template <class S, bool ATOMIC>
__device__ inline void emit_row(float *C, int64_t row, int64_t N, int64_t col0,
                                int j, const float (&acc)[S::NV][S::VEC])
{
    // The lane's addresses are formed here at every call rather than kept
    // live across the caller's loops (they cost registers there, and the
    // spills a 128-register wavefront would need cost more than the few
    // instructions).
    __asm__ volatile("" : "+v"(j));
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
                __builtin_nontemporal_store(w, (f32x4 *)(crow + c + x));
            }
        } else if constexpr (S::VEC == 2) {
            f32x2 w = {acc[k][0], acc[k][1]};
            __builtin_nontemporal_store(w, (f32x2 *)(crow + c));
        } else {
            __builtin_nontemporal_store(acc[k][0], crow + c);
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

}  // namespace
}  // namespace sdl
