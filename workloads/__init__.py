"""Seeded synthetic CSR problems for CSR sparse x dense products.

This module only *draws inputs*: it holds none of the product's arithmetic
and imports neither the oracle nor the HIP binding, so both sides can take
their inputs from it.

The pages measure on collections that are not available here (the 72-test
matrix collection of [IntelMax], the unnamed SpMM datasets of [Sgap]); the
generators below stand in for them with the shapes, sizes, value
distributions and sparsity structure of the five workloads this library is
measured on:

  uniform_1k_n32      1024 x 1024, exactly 16 distinct uniform columns per
                      row, vals U(-1,1), B 1024 x 32 U(-1,1), fp32
  powerlaw_262k_n64   262144 x 262144, row length from the discrete power
                      law p(d) ~ d^-2.1 on {1..8192}, uniform distinct
                      columns, vals U(0,1), B 262144 x 64 N(0,1), fp32
  pruned_4k_n256_bf16 4096 x 4096, each entry kept with probability 0.1,
                      vals N(0, 0.02^2), B 4096 x 256 N(0,1); vals and B
                      rounded to bf16 (the fp32 twin keeps the same draws)
  banded_4m_n128      4194304 x 4194304, 32 per row: 24 distinct in
                      [i-4096, i+4096] and 8 uniform over [0, K), all
                      distinct, vals U(-1,1), B 4194304 x 128 U(-1,1), fp32
  skew_1m_n512_bf16   1048576 x 1048576, 1049 hub rows (0.1 %) with
                      U{20000..200000} entries, the rest U{1..8}, uniform
                      distinct columns, vals U(-1,1), B 1048576 x 512 N(0,1),
                      vals and B in bf16

Pages:
  [IntelMax] "Performance Optimization of Deep Learning Sparse Matrix Kernels
             on Intel Max Series GPU"
  [Sgap]     "Sgap: Towards Efficient Sparse Tensor Algebra Compilation for GPU"

Conventions: numpy's PCG64 ``default_rng(seed)``; column indices of a row are
distinct and ascending; fp32 values come from float64 draws rounded to
nearest; bf16 values are the fp32 values rounded to nearest-even bf16.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Rows of B and of fp32 value arrays are drawn in blocks of this many
# elements so that large problems do not need float64 temporaries of the
# full size.  Changing it changes the drawn numbers.
_BLOCK = 1 << 24


@dataclass
class CsrProblem:
    """One seeded problem: A (CSR, int32 indices) and dense B (row-major)."""
    name: str
    M: int
    K: int
    N: int
    rowptr: np.ndarray          # int32 [M+1]
    colind: np.ndarray          # int32 [nnz]
    vals: np.ndarray            # float32, or uint16 bf16 bits
    B: np.ndarray               # float32 or uint16, shape (K, N)
    dtype: str                  # "f32" or "bf16"
    meta: dict = field(default_factory=dict)

    @property
    def nnz(self) -> int:
        return int(self.rowptr[-1] - self.rowptr[0])

    def lengths(self) -> np.ndarray:
        return np.diff(self.rowptr.astype(np.int64))


# ---------------------------------------------------------------- helpers

def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even.

    Finite inputs only (the generators never produce NaN or Inf)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in = x.reshape(-1)
    flat_out = out.reshape(-1)
    for s in range(0, flat_in.shape[0], _BLOCK):
        u = flat_in[s:s + _BLOCK].view(np.uint32)
        bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
        flat_out[s:s + _BLOCK] = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    return out


def _uniform_f32(rng, n, lo, hi) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _BLOCK):
        e = min(n, s + _BLOCK)
        out[s:e] = rng.uniform(lo, hi, e - s)
    return out


def _normal_f32(rng, n, sigma=1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _BLOCK):
        e = min(n, s + _BLOCK)
        out[s:e] = rng.standard_normal(e - s) * sigma
    return out


def _distinct_sorted_fixed(rng, lo, hi, d) -> np.ndarray:
    """(M, d) int64: per row, d distinct integers from [lo[i], hi[i]), sorted.

    Draw, sort per row, redraw every entry equal to its left neighbour, repeat
    until no duplicates remain (each surviving set is a uniform d-subset)."""
    lo = np.asarray(lo, dtype=np.int64)
    hi = np.asarray(hi, dtype=np.int64)
    M = lo.shape[0]
    if d == 0:
        return np.zeros((M, 0), dtype=np.int64)
    if np.any(hi - lo < d):
        raise ValueError("a row's range is smaller than its length")
    cols = rng.integers(lo[:, None], hi[:, None], size=(M, d))
    while True:
        cols.sort(axis=1)
        dup = np.zeros(cols.shape, dtype=bool)
        dup[:, 1:] = cols[:, 1:] == cols[:, :-1]
        if not dup.any():
            return cols
        r, c = np.nonzero(dup)
        cols[r, c] = rng.integers(lo[r], hi[r])


def _distinct_sorted_variable(rng, lengths, K) -> np.ndarray:
    """Column indices (int64, CSR order) for rows of the given lengths: per
    row, lengths[i] distinct uniform integers from [0, K), ascending.

    Draws lengths[i] values per row, keeps the distinct ones, then draws only
    the shortfall of each row again until every row is full."""
    lengths = np.asarray(lengths, dtype=np.int64)
    M = lengths.shape[0]
    if np.any(lengths > K):
        raise ValueError("a row is longer than K")
    if not lengths.any():
        return np.zeros(0, dtype=np.int64)
    rows = np.repeat(np.arange(M, dtype=np.int64), lengths)
    keys = np.unique(rows * K + rng.integers(0, K, size=rows.shape[0]))
    while True:
        counts = np.bincount(keys // K, minlength=M)
        short = lengths - counts
        if not short.any():
            return keys % K
        rows = np.repeat(np.arange(M, dtype=np.int64), short)
        fresh = rows * K + rng.integers(0, K, size=rows.shape[0])
        keys = np.unique(np.concatenate([keys, fresh]))


def _distinct_sorted_one(rng, d, K) -> np.ndarray:
    """d distinct uniform integers from [0, K), ascending (one long row)."""
    got = np.unique(rng.integers(0, K, size=d))
    while got.shape[0] < d:
        got = np.unique(np.concatenate(
            [got, rng.integers(0, K, size=d - got.shape[0])]))
    return got


def _rowptr(lengths) -> np.ndarray:
    rp = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=rp[1:])
    if rp[-1] >= 2 ** 31:
        raise ValueError("nnz does not fit int32 offsets")
    return rp.astype(np.int32)


def _finish(name, M, K, N, lengths, cols, vals32, B32, dtype, meta) -> CsrProblem:
    rowptr = _rowptr(lengths)
    colind = np.ascontiguousarray(cols, dtype=np.int32).reshape(-1)
    if dtype == "bf16":
        vals = f32_to_bf16_bits(vals32)
        B = f32_to_bf16_bits(B32).reshape(K, N)
    elif dtype == "f32":
        vals = np.ascontiguousarray(vals32, dtype=np.float32)
        B = np.ascontiguousarray(B32, dtype=np.float32).reshape(K, N)
    else:
        raise ValueError(dtype)
    return CsrProblem(name, M, K, N, rowptr, colind, vals, B, dtype, meta)


# ------------------------------------------------------------- generators

def uniform_rows(M=1024, K=1024, N=32, per_row=16, seed=1, dtype="f32",
                 name="uniform_1k_n32") -> CsrProblem:
    """Exactly ``per_row`` distinct uniform columns per row; vals and B
    U(-1,1)."""
    rng = np.random.default_rng(seed)
    cols = _distinct_sorted_fixed(rng, np.zeros(M, np.int64),
                                  np.full(M, K, np.int64), per_row)
    lengths = np.full(M, per_row, dtype=np.int64)
    vals = _uniform_f32(rng, M * per_row, -1.0, 1.0)
    B = _uniform_f32(rng, K * N, -1.0, 1.0)
    return _finish(name, M, K, N, lengths, cols, vals, B, dtype,
                   {"per_row": per_row, "seed": seed})


def powerlaw_lengths(rng, M, alpha, dmin, dmax) -> np.ndarray:
    """Row lengths from the discrete law p(d) ~ d^-alpha on {dmin..dmax},
    by inverse transform on the exact cumulative sum."""
    d = np.arange(dmin, dmax + 1, dtype=np.float64)
    cdf = np.cumsum(d ** (-alpha))
    cdf /= cdf[-1]
    u = rng.random(M)
    idx = np.searchsorted(cdf, u, side="right")
    return np.minimum(idx, dmax - dmin).astype(np.int64) + dmin


def powerlaw_rows(M=262144, K=None, N=64, alpha=2.1, dmin=1, dmax=8192,
                  seed=2, dtype="f32", name="powerlaw_262k_n64") -> CsrProblem:
    """GNN-style power-law graph: lengths ~ d^-alpha on {dmin..dmax} (capped
    at K), uniform distinct columns, vals U(0,1), B N(0,1)."""
    K = M if K is None else K
    rng = np.random.default_rng(seed)
    lengths = powerlaw_lengths(rng, M, alpha, dmin, min(dmax, K))
    cols = _distinct_sorted_variable(rng, lengths, K)
    vals = _uniform_f32(rng, cols.shape[0], 0.0, 1.0)
    B = _normal_f32(rng, K * N)
    return _finish(name, M, K, N, lengths, cols, vals, B, dtype,
                   {"alpha": alpha, "dmin": dmin, "dmax": min(dmax, K),
                    "seed": seed})


def bernoulli_rows(M=4096, K=4096, N=256, p=0.1, sigma=0.02, seed=3,
                   dtype="bf16", name=None) -> CsrProblem:
    """Pruned DL weight: every entry kept independently with probability p,
    vals N(0, sigma^2), B N(0,1)."""
    name = name or f"pruned_4k_n256_{dtype}"
    rng = np.random.default_rng(seed)
    keep = rng.random((M, K)) < p
    rows, cols = np.nonzero(keep)
    del keep
    lengths = np.bincount(rows, minlength=M).astype(np.int64)
    vals = _normal_f32(rng, cols.shape[0], sigma)
    B = _normal_f32(rng, K * N)
    return _finish(name, M, K, N, lengths, cols, vals, B, dtype,
                   {"p": p, "sigma": sigma, "seed": seed})


def banded_rows(M=4194304, K=None, N=128, band_nnz=24, uniform_nnz=8,
                half_width=4096, seed=4, dtype="f32",
                name="banded_4m_n128") -> CsrProblem:
    """Banded-clustered rows: band_nnz distinct columns in
    [i-half_width, i+half_width] (clipped to [0,K)), plus uniform_nnz uniform
    over [0,K), every column of a row distinct; vals and B U(-1,1)."""
    K = M if K is None else K
    rng = np.random.default_rng(seed)
    i = np.arange(M, dtype=np.int64)
    lo = np.maximum(0, i - half_width)
    hi = np.minimum(K, i + half_width + 1)
    band = _distinct_sorted_fixed(rng, lo, hi, band_nnz)
    uni = rng.integers(0, K, size=(M, uniform_nnz))
    while True:
        both = np.concatenate([band, uni], axis=1)
        order = np.argsort(both, axis=1, kind="stable")
        srt = np.take_along_axis(both, order, axis=1)
        dup = np.zeros(srt.shape, dtype=bool)
        dup[:, 1:] = srt[:, 1:] == srt[:, :-1]
        if not dup.any():
            cols = srt
            break
        # band columns are distinct, and the stable sort puts a band column
        # before an equal uniform one, so each flagged entry is a uniform draw
        r, c = np.nonzero(dup)
        src = order[r, c] - band_nnz
        uni[r, src] = rng.integers(0, K, size=r.shape[0])
    in_band = (np.abs(cols - i[:, None]) <= half_width).mean()
    lengths = np.full(M, band_nnz + uniform_nnz, dtype=np.int64)
    vals = _uniform_f32(rng, M * (band_nnz + uniform_nnz), -1.0, 1.0)
    B = _uniform_f32(rng, K * N, -1.0, 1.0)
    return _finish(name, M, K, N, lengths, cols, vals, B, dtype,
                   {"half_width": half_width, "band_nnz": band_nnz,
                    "uniform_nnz": uniform_nnz, "in_band_share": float(in_band),
                    "seed": seed})


def skew_rows(M=1048576, K=None, N=512, hub_frac=0.001, hub_lo=20000,
              hub_hi=200000, short_lo=1, short_hi=8, seed=5, dtype="bf16",
              name="skew_1m_n512_bf16") -> CsrProblem:
    """Extreme skew: round(hub_frac*M) hub rows at seeded random positions
    with U{hub_lo..hub_hi} entries, the others U{short_lo..short_hi}; uniform
    distinct columns; vals U(-1,1); B N(0,1)."""
    K = M if K is None else K
    hub_hi = min(hub_hi, K)
    hub_lo = min(hub_lo, hub_hi)
    rng = np.random.default_rng(seed)
    n_hubs = int(round(hub_frac * M))
    hubs = np.sort(rng.permutation(M)[:n_hubs])
    lengths = rng.integers(short_lo, short_hi + 1, size=M).astype(np.int64)
    lengths[hubs] = rng.integers(hub_lo, hub_hi + 1, size=n_hubs)
    is_hub = np.zeros(M, dtype=bool)
    is_hub[hubs] = True
    small = lengths.copy()
    small[is_hub] = 0
    small_cols = _distinct_sorted_variable(rng, small, K)
    rowptr = _rowptr(lengths).astype(np.int64)
    cols = np.empty(int(rowptr[-1]), dtype=np.int64)
    cols[np.repeat(~is_hub, lengths)] = small_cols
    for h in hubs:
        cols[rowptr[h]:rowptr[h + 1]] = _distinct_sorted_one(rng, int(lengths[h]), K)
    vals = _uniform_f32(rng, cols.shape[0], -1.0, 1.0)
    B = _normal_f32(rng, K * N)
    return _finish(name, M, K, N, lengths, cols, vals, B, dtype,
                   {"hubs": hubs, "hub_range": (hub_lo, hub_hi),
                    "short_range": (short_lo, short_hi), "seed": seed})


# ------------------------------------------------------------- registry

#: The five measured workloads at full size (and the fp32 twin of the pruned
#: one).  Values are zero-argument builders.
WORKLOADS = {
    "uniform_1k_n32": lambda: uniform_rows(),
    "powerlaw_262k_n64": lambda: powerlaw_rows(),
    # secondary power-law case: the exponent that gives mean row length 16
    # on {1..8192}
    "powerlaw_262k_n64_mean16": lambda: powerlaw_rows(
        alpha=1.7694, seed=22, name="powerlaw_262k_n64_mean16"),
    "pruned_4k_n256_bf16": lambda: bernoulli_rows(dtype="bf16"),
    "pruned_4k_n256_f32": lambda: bernoulli_rows(dtype="f32"),
    "banded_4m_n128": lambda: banded_rows(),
    "skew_1m_n512_bf16": lambda: skew_rows(),
}


def make(name: str) -> CsrProblem:
    """Build one of the full-size workloads by name."""
    return WORKLOADS[name]()



def rows_with_lengths(lengths, K, N, seed=0, dtype="f32", name="lengths",
                      value_range=(-1.0, 1.0)) -> CsrProblem:
    """Edge-case problem with the given row lengths: uniform distinct sorted
    columns in [0, K), vals U(value_range), B U(-1,1)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    M = lengths.shape[0]
    rng = np.random.default_rng(seed)
    cols = _distinct_sorted_variable(rng, lengths, K)
    vals = _uniform_f32(rng, cols.shape[0], *value_range)
    B = _uniform_f32(rng, K * N, -1.0, 1.0)
    return _finish(name, M, K, N, lengths, cols, vals, B, dtype, {"seed": seed})
