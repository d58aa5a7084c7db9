// span.h -- finding the rows of stored entries when the entries, not the
// rows, are split among wavefronts (SDDMM and the element-balanced product).
// All functions are wavefront-collective: every lane calls them together.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace sdl {
namespace {

// The row holding absolute position p: the last i in [0, M) with
// rowptr[i] <= p (rowptr[0] <= p < rowptr[M] is required).  64-ary search:
// each round narrows [lo, hi) to one of 64 equal parts.
__device__ inline int64_t find_row(const int32_t *rowptr, int64_t M, int64_t p,
                                   int lane)
{
    int64_t lo = 0, hi = M;  // rowptr[lo] <= p < rowptr[hi]
    while (hi - lo > 1) {
        const int64_t step = (hi - lo + kWave - 1) / kWave;
        const int64_t idx = lo + lane * step;
        const int64_t v = rowptr[idx < hi ? idx : hi - 1];
        // the probes are in ascending order, so the lanes with v <= p form
        // a prefix (lane 0 always: rowptr[lo] <= p)
        const int c = __popcll(__ballot(idx < hi && v <= p));
        const int64_t nlo = lo + (int64_t)(c - 1) * step;
        hi = nlo + step < hi ? nlo + step : hi;
        lo = nlo;
    }
    return lo;
}

// The first row i in [0, M] with rowptr[i] >= p.  Requires
// rowptr[0] <= p <= rowptr[M].  64-ary search keeping
// rowptr[lo] < p <= rowptr[hi].
__device__ inline int64_t lower_row(const int32_t *rowptr, int64_t M, int64_t p,
                                    int lane)
{
    if ((int64_t)rowptr[0] >= p)
        return 0;
    int64_t lo = 0, hi = M;
    while (hi - lo > 1) {
        const int64_t step = (hi - lo + kWave - 1) / kWave;
        const int64_t idx = lo + lane * step;
        const int64_t v = rowptr[idx < hi ? idx : hi - 1];
        // ascending probes: the lanes with v < p form a prefix (lane 0 always)
        const int c = __popcll(__ballot(idx < hi && v < p));
        const int64_t nlo = lo + (int64_t)(c - 1) * step;
        hi = nlo + step < hi ? nlo + step : hi;
        lo = nlo;
    }
    return hi;
}

// Row of the entry at absolute position pe, given a row i_cur with
// rowptr[i_cur] <= pe (each lane its own pe, i_cur wave-uniform): lane l
// holds rowptr[win + 1 + l] of a 64-row window, each lane counts the window
// values <= pe by a binary search over the lanes (shuffles), and the window
// moves on by 64 rows while some lane's entry lies beyond it (runs of empty
// rows).  Requires pe < rowptr[M].
__device__ inline int64_t row_in_window(const int32_t *rowptr, int64_t M,
                                        int64_t i_cur, int64_t pe, int lane,
                                        int64_t first_wv = -1)
{
    // first_wv: this lane's value of the first window, rowptr[min(i_cur + 1
    // + lane, M)], when the caller has loaded it ahead (-1: load it here)
    int64_t row = 0;
    bool done = false;
    for (int64_t win = i_cur; __ballot(!done) != 0; win += kWave) {
        const int64_t wi = win + 1 + lane;
        const int64_t wv = (win == i_cur && first_wv >= 0) ? first_wv
                                                           : (int64_t)rowptr[wi < M ? wi : M];
        int pos = 0;
#pragma unroll
        for (int st = kWave / 2; st > 0; st >>= 1)
            if (__shfl(wv, pos + st - 1) <= pe)
                pos += st;
        if (pos == kWave - 1 && __shfl(wv, kWave - 1) <= pe)
            pos = kWave;
        if (!done && pos < kWave) {
            row = win + pos;
            done = true;
        }
    }
    return row;
}

}  // namespace
}  // namespace sdl
