"""Pins of the SpMM oracle: checks against values fixed by the mathematics.

Every pin takes ``ref``, a function with the signature of
``oracle.spmm_ref`` (rowptr, colind, vals, B, N, rows=None, with_bound=True)
-> (C, S), and raises AssertionError when ``ref`` is wrong.  The pins never
re-run the oracle's own formula: they compare with a dense brute-force
product in plain Python floats, with scipy.sparse, with exact integer
products, with a hand-derived worked example, and with algebraic invariants
(identity, permutation, empty rows, scaling, duplicates, the bound, row
sampling and row-block views).

Definition pinned ("Performance Optimization of Deep Learning Sparse Matrix
Kernels on Intel Max Series GPU", SpMM operation, Fig. 5 and Algorithm 2):
C[i, :] = sum over stored entries p of row i of vals[p] * B[colind[p], :],
and S[i, :] = sum of |vals[p]| * |B[colind[p], :]|.
"""
from __future__ import annotations

import json
import os
import struct

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------ helpers

def bf16_bits_to_float(bits: int) -> float:
    """Independent exact widening: the 16 bits are the top half of an IEEE
    binary32 word (big-endian bytes: bits, then two zero bytes)."""
    return struct.unpack(">f", struct.pack(">HH", bits & 0xFFFF, 0))[0]


def random_csr(rng, M, K, density, sorted_cols=True):
    """Small random CSR with distinct columns per row."""
    rows = []
    for _ in range(M):
        if K == 0:
            rows.append(np.zeros(0, dtype=np.int64))
            continue
        mask = rng.random(K) < density
        cols = np.nonzero(mask)[0]
        if not sorted_cols:
            cols = rng.permutation(cols)
        rows.append(cols)
    rowptr = np.zeros(M + 1, dtype=np.int32)
    rowptr[1:] = np.cumsum([len(r) for r in rows])
    colind = (np.concatenate(rows) if rows else np.zeros(0)).astype(np.int32)
    return rowptr, colind


def dense_of(rowptr, colind, vals_f64, M, K):
    A = [[0.0] * K for _ in range(M)]
    for i in range(M):
        for p in range(rowptr[i], rowptr[i + 1]):
            A[i][colind[p]] += vals_f64[p]
    return A


def brute_force(A, Bf, M, K, N):
    """C and S by the dense triple loop over every column k (ascending), in
    Python floats (IEEE double)."""
    C = [[0.0] * N for _ in range(M)]
    S = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for k in range(K):
            a = A[i][k]
            for n in range(N):
                b = Bf[k][n]
                C[i][n] = C[i][n] + a * b
                S[i][n] = S[i][n] + abs(a) * abs(b)
    return np.array(C).reshape(M, N), np.array(S).reshape(M, N)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even bf16 bits of float32 values (test-local)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


# --------------------------------------------------------------- pins

def pin_bruteforce_f32(ref):
    """Dense brute force, fp32 inputs: equal to the last bit (sorted rows add
    the same products in the same order; the extra zero products are exact)."""
    rng = np.random.default_rng(101)
    for case in range(40):
        M, K, N = (int(v) for v in rng.integers(0, 10, size=3))
        density = [0.0, 0.2, 0.5, 1.0][case % 4]
        rowptr, colind = random_csr(rng, M, K, density)
        vals = rng.uniform(-2, 2, colind.shape[0]).astype(np.float32)
        B = rng.uniform(-2, 2, (K, N)).astype(np.float32)
        C, S = ref(rowptr, colind, vals, B, N)
        A = dense_of(rowptr, colind, [float(v) for v in vals], M, K)
        Cb, Sb = brute_force(A, [[float(v) for v in r] for r in B], M, K, N)
        assert C.shape == (M, N) and S.shape == (M, N)
        assert np.array_equal(C, Cb), f"case {case}: C differs from brute force"
        assert np.array_equal(S, Sb), f"case {case}: S differs from brute force"


def pin_bruteforce_bf16(ref):
    """Dense brute force on bf16 bit patterns, widened independently."""
    rng = np.random.default_rng(202)
    for case in range(30):
        M, K, N = (int(v) for v in rng.integers(1, 9, size=3))
        rowptr, colind = random_csr(rng, M, K, 0.5)
        vals = f32_to_bf16(rng.uniform(-2, 2, colind.shape[0]))
        B = f32_to_bf16(rng.uniform(-2, 2, (K, N)))
        C, S = ref(rowptr, colind, vals, B, N)
        A = dense_of(rowptr, colind, [bf16_bits_to_float(int(v)) for v in vals], M, K)
        Bf = [[bf16_bits_to_float(int(v)) for v in r] for r in B]
        Cb, Sb = brute_force(A, Bf, M, K, N)
        assert np.array_equal(C, Cb), f"case {case}: bf16 C differs"
        assert np.array_equal(S, Sb), f"case {case}: bf16 S differs"


def pin_scipy(ref):
    """scipy.sparse CSR times dense, in float64, agrees within 1e-13 * S."""
    import scipy.sparse as sp
    rng = np.random.default_rng(303)
    for M, K, N, d in [(200, 150, 7, 0.05), (64, 300, 33, 0.2), (1, 500, 5, 0.9)]:
        rowptr, colind = random_csr(rng, M, K, d, sorted_cols=False)
        vals = rng.standard_normal(colind.shape[0]).astype(np.float32)
        B = rng.standard_normal((K, N)).astype(np.float32)
        C, S = ref(rowptr, colind, vals, B, N)
        A = sp.csr_matrix((vals.astype(np.float64), colind, rowptr), shape=(M, K))
        Cs = A @ B.astype(np.float64)
        assert np.all(np.abs(C - Cs) <= 1e-13 * S + 1e-300), "scipy disagrees"


def pin_worked_example(ref):
    """Hand-built Fig. 5 structure (tests/golden/worked_example_fig5.json):
    exact C and S, for fp32 and for bf16 inputs (all values are
    bf16-representable)."""
    with open(os.path.join(GOLDEN, "worked_example_fig5.json")) as f:
        g = json.load(f)
    rowptr = np.array(g["rowptr"], dtype=np.int32)
    colind = np.array(g["colind"], dtype=np.int32)
    vals = np.array(g["vals"], dtype=np.float32)
    B = np.array(g["B"], dtype=np.float32)
    for v, b in [(vals, B), (f32_to_bf16(vals), f32_to_bf16(B))]:
        C, S = ref(rowptr, colind, v, b, g["N"])
        assert np.array_equal(C, np.array(g["C"])), "worked example C"
        assert np.array_equal(S, np.array(g["S"])), "worked example S"


def pin_integer_exact(ref):
    """Small integers: every product and partial sum is an exact integer in
    double, so C must equal the int64 dense product exactly."""
    rng = np.random.default_rng(404)
    M, K, N = 40, 37, 6
    rowptr, colind = random_csr(rng, M, K, 0.4)
    vals_i = rng.integers(-9, 10, colind.shape[0])
    B_i = rng.integers(-9, 10, (K, N))
    A_i = np.zeros((M, K), dtype=np.int64)
    for i in range(M):
        for p in range(rowptr[i], rowptr[i + 1]):
            A_i[i, colind[p]] += vals_i[p]
    C, S = ref(rowptr, colind, vals_i.astype(np.float32), B_i.astype(np.float32), N)
    assert np.array_equal(C, (A_i @ B_i).astype(np.float64)), "integer product"
    assert np.array_equal(S, (np.abs(A_i) @ np.abs(B_i)).astype(np.float64)), "integer bound"


def pin_identity_and_permutation(ref):
    """A = I gives C = B; A = a permutation P gives C[i] = B[perm[i]]; both
    exactly, fp32 and bf16."""
    rng = np.random.default_rng(505)
    M, N = 50, 9
    B = rng.standard_normal((M, N)).astype(np.float32)
    ident_rp = np.arange(M + 1, dtype=np.int32)
    ident_ci = np.arange(M, dtype=np.int32)
    ones = np.ones(M, dtype=np.float32)
    C, _ = ref(ident_rp, ident_ci, ones, B, N)
    assert np.array_equal(C, B.astype(np.float64)), "identity"
    perm = rng.permutation(M).astype(np.int32)
    C, _ = ref(ident_rp, perm, ones, B, N)
    assert np.array_equal(C, B[perm].astype(np.float64)), "permutation"
    Bb = f32_to_bf16(B)
    C, _ = ref(ident_rp, perm, f32_to_bf16(ones), Bb, N)
    widened = np.array([[bf16_bits_to_float(int(v)) for v in r] for r in Bb])
    assert np.array_equal(C, widened[perm]), "bf16 permutation"


def pin_empty_rows_and_views(ref):
    """Empty rows are exact zeros; a block of rows passed as a view with
    rowptr[0] != 0 gives the same rows; a sampled row list gives the same
    rows as the full product."""
    rng = np.random.default_rng(606)
    M, K, N = 30, 20, 5
    rowptr, colind = random_csr(rng, M, K, 0.3)
    # empty out rows 0, 7 and the last one
    lens = np.diff(rowptr).astype(np.int64)
    keep = np.ones(colind.shape[0], dtype=bool)
    for r in (0, 7, M - 1):
        keep[rowptr[r]:rowptr[r + 1]] = False
        lens[r] = 0
    colind = colind[keep]
    rowptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    vals = rng.uniform(-1, 1, colind.shape[0]).astype(np.float32)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    C, S = ref(rowptr, colind, vals, B, N)
    for r in (0, 7, M - 1):
        assert np.all(C[r] == 0.0) and np.all(S[r] == 0.0), "empty row not zero"
    # view of rows 10..19: rowptr slice keeps absolute offsets
    Cv, Sv = ref(rowptr[10:21], colind, vals, B, N)
    assert np.array_equal(Cv, C[10:20]) and np.array_equal(Sv, S[10:20]), "row view"
    rows = np.array([19, 3, 3, 0, 25])
    Cs, Ss = ref(rowptr, colind, vals, B, N, rows=rows)
    assert np.array_equal(Cs, C[rows]) and np.array_equal(Ss, S[rows]), "row sample"


def pin_scaling_and_sign(ref):
    """C(2*vals) = 2*C(vals) and C(-vals) = -C(vals), exactly (binary
    scaling and negation commute with every rounding)."""
    rng = np.random.default_rng(707)
    M, K, N = 25, 30, 8
    rowptr, colind = random_csr(rng, M, K, 0.5)
    vals = rng.standard_normal(colind.shape[0]).astype(np.float32)
    B = rng.standard_normal((K, N)).astype(np.float32)
    C, S = ref(rowptr, colind, vals, B, N)
    C2, S2 = ref(rowptr, colind, 2 * vals, B, N)
    Cn, Sn = ref(rowptr, colind, -vals, B, N)
    assert np.array_equal(C2, 2 * C) and np.array_equal(S2, 2 * S), "scaling"
    assert np.array_equal(Cn, -C) and np.array_equal(Sn, S), "negation"


def pin_duplicates_add(ref):
    """Repeated (row, column) entries add up: entries (k, 0.75) and (k, 0.25)
    act like one entry (k, 1.0) (dyadic, so exact)."""
    B = np.array([[1.5, -2.0], [4.0, 0.125], [3.0, 8.0]], dtype=np.float32)
    rowptr = np.array([0, 3, 4], dtype=np.int32)
    colind = np.array([1, 2, 1, 2], dtype=np.int32)
    vals = np.array([0.75, 2.0, 0.25, 1.0], dtype=np.float32)
    C, _ = ref(rowptr, colind, vals, B, 2)
    expect = np.array([[4.0 + 6.0, 0.125 + 16.0], [3.0, 8.0]])
    assert np.array_equal(C, expect), "duplicates"


def pin_bound(ref):
    """S >= |C| everywhere; with non-negative inputs S equals C exactly."""
    rng = np.random.default_rng(808)
    M, K, N = 40, 40, 6
    rowptr, colind = random_csr(rng, M, K, 0.3)
    vals = rng.standard_normal(colind.shape[0]).astype(np.float32)
    B = rng.standard_normal((K, N)).astype(np.float32)
    C, S = ref(rowptr, colind, vals, B, N)
    assert np.all(S >= np.abs(C)), "S below |C|"
    C, S = ref(rowptr, colind, np.abs(vals), np.abs(B), N)
    assert np.array_equal(S, C), "S != C for non-negative inputs"


def pin_spmv(ref):
    """N = 1 is a sparse matrix-vector product: equal to the dense mat-vec
    (numpy float64) within 1e-14 * S."""
    rng = np.random.default_rng(909)
    M, K = 80, 120
    rowptr, colind = random_csr(rng, M, K, 0.25)
    vals = rng.standard_normal(colind.shape[0]).astype(np.float32)
    x = rng.standard_normal((K, 1)).astype(np.float32)
    C, S = ref(rowptr, colind, vals, x, 1)
    A = np.zeros((M, K))
    for i in range(M):
        for p in range(rowptr[i], rowptr[i + 1]):
            A[i, colind[p]] += float(vals[p])
    y = A @ x.astype(np.float64)
    assert np.all(np.abs(C - y) <= 1e-14 * S + 1e-300), "mat-vec"


ALL_PINS = [
    pin_bruteforce_f32,
    pin_bruteforce_bf16,
    pin_scipy,
    pin_worked_example,
    pin_integer_exact,
    pin_identity_and_permutation,
    pin_empty_rows_and_views,
    pin_scaling_and_sign,
    pin_duplicates_add,
    pin_bound,
    pin_spmv,
]
