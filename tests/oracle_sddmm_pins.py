"""Pins of the SDDMM and FusedMM oracles against what the mathematics fixes.

Every pin is a function ``pin(sddmm, fusedmm)`` taking two callables with
the signatures of ``oracle.sddmm_ref`` and ``oracle.fusedmm_ref`` (so the
mutant test can hand in oracles built from altered sources) and raising
AssertionError when they disagree with the fixed values.

Pages: [IntelMax] "Performance Optimization of Deep Learning Sparse Matrix
Kernels on Intel Max Series GPU", the SDDMM operation (Fig. 3, Algorithm 1)
and the FusedMM operation (Fig. 6, Algorithm 3).
"""
from __future__ import annotations

import json
import os
import struct

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand_pattern(rng, M, K, density):
    mask = rng.random((M, K)) < density
    rowptr = np.concatenate([[0], np.cumsum(mask.sum(axis=1))]).astype(np.int32)
    colind = np.nonzero(mask)[1].astype(np.int32)
    return rowptr, colind


def _bf16_bits(x: float) -> int:
    """Upper half of the binary32 word (x chosen bf16-exact by the caller)."""
    return struct.unpack("<I", struct.pack("<f", x))[0] >> 16


def _bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits << 16))[0]


def pin_worked_example(sddmm, fusedmm):
    """Hand-derived Fig. 3 / Fig. 6 instance: exact values."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example_fig3_fig6.json")))
    rp = np.array(g["rowptr"], np.int32)
    ci = np.array(g["colind"], np.int32)
    for kind in ("f32", "bf16"):
        def conv(x):
            a = np.array(x, np.float32)
            if kind == "f32":
                return a
            return (a.view(np.uint32) >> 16).astype(np.uint16)
        C, B, D = conv(g["C"]), conv(g["B"]), conv(g["D"])
        A, S = sddmm(rp, ci, C, B, g["N"])
        assert np.array_equal(A, np.array(g["A"])), (kind, A)
        assert np.array_equal(S, np.array(g["S"])), (kind, S)
        E, T = fusedmm(rp, ci, C, B, D, g["N"])
        assert np.array_equal(E, np.array(g["E"])), (kind, E)
        assert np.array_equal(T, np.array(g["T"])), (kind, T)


def pin_brute_force_python(sddmm, fusedmm):
    """Dense definition in Python floats, same summation order: bitwise."""
    rng = np.random.default_rng(11)
    for (M, K, N, dens) in [(5, 7, 3, 0.4), (9, 4, 17, 0.7), (1, 1, 1, 1.0), (6, 9, 8, 0.25)]:
        rp, ci = _rand_pattern(rng, M, K, dens)
        C = rng.uniform(-1, 1, (M, N)).astype(np.float32)
        B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
        D = rng.uniform(-1, 1, (K, N)).astype(np.float32)
        A, S = sddmm(rp, ci, C, B, N)
        E, T = fusedmm(rp, ci, C, B, D, N)
        for i in range(M):
            e = [0.0] * N
            t = [0.0] * N
            for p in range(rp[i], rp[i + 1]):
                j = int(ci[p])
                acc = 0.0
                s = 0.0
                for n in range(N):
                    c = float(C[i, n])
                    b = float(B[j, n])
                    acc = acc + c * b
                    s = s + abs(c) * abs(b)
                assert A[p] == acc and S[p] == s, (M, K, N, i, p)
                for n in range(N):
                    d = float(D[j, n])
                    e[n] = e[n] + acc * d
                    t[n] = t[n] + s * abs(d)
            assert list(E[i]) == e and list(T[i]) == t, (M, K, N, i)


def pin_dense_matmul(sddmm, fusedmm):
    """numpy in fp64: A = (C B^T) sampled on the pattern; E = A_dense D.
    The orders differ, so compare within a few ulps of the bound."""
    rng = np.random.default_rng(12)
    M, K, N = 40, 33, 24
    rp, ci = _rand_pattern(rng, M, K, 0.3)
    C = rng.standard_normal((M, N)).astype(np.float32)
    B = rng.standard_normal((K, N)).astype(np.float32)
    D = rng.standard_normal((K, N)).astype(np.float32)
    full = C.astype(np.float64) @ B.astype(np.float64).T
    rows = np.repeat(np.arange(M), np.diff(rp))
    A, S = sddmm(rp, ci, C, B, N)
    assert np.all(np.abs(A - full[rows, ci]) <= 1e-13 * S + 1e-300)
    Ad = np.zeros((M, K))
    Ad[rows, ci] = full[rows, ci]
    E, T = fusedmm(rp, ci, C, B, D, N)
    assert np.all(np.abs(E - Ad @ D.astype(np.float64)) <= 1e-12 * T + 1e-300)


def pin_transpose_symmetry(sddmm, fusedmm):
    """<C_i, B_j> = <B_j, C_i>: SDDMM of (C, B) on a pattern equals SDDMM of
    (B, C) on the transposed pattern, entry for entry, bitwise (the products
    commute exactly and both sums run over n upwards).  Uses K != M and
    N != K so that a swapped operand or index cannot pass."""
    rng = np.random.default_rng(13)
    M, K, N = 7, 11, 5
    rp, ci = _rand_pattern(rng, M, K, 0.45)
    C = rng.uniform(-2, 2, (M, N)).astype(np.float32)
    B = rng.uniform(-2, 2, (K, N)).astype(np.float32)
    A, _ = sddmm(rp, ci, C, B, N)
    rows = np.repeat(np.arange(M), np.diff(rp))
    order = np.lexsort((rows, ci))            # transposed pattern, CSR order
    rpt = np.concatenate([[0], np.cumsum(np.bincount(ci, minlength=K))]).astype(np.int32)
    At, _ = sddmm(rpt, rows[order].astype(np.int32), B, C, N)
    assert np.array_equal(At, A[order])


def pin_scaling_and_sign(sddmm, fusedmm):
    """Scaling C by 2 scales A and E by 2 exactly; negating B negates A
    and E, and negating D negates E, exactly."""
    rng = np.random.default_rng(14)
    M, K, N = 12, 10, 9
    rp, ci = _rand_pattern(rng, M, K, 0.5)
    C = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    D = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    A, S = sddmm(rp, ci, C, B, N)
    E, T = fusedmm(rp, ci, C, B, D, N)
    A2, S2 = sddmm(rp, ci, 2 * C, B, N)
    assert np.array_equal(A2, 2 * A) and np.array_equal(S2, 2 * S)
    An, Sn = sddmm(rp, ci, C, -B, N)
    assert np.array_equal(An, -A) and np.array_equal(Sn, S)
    En, Tn = fusedmm(rp, ci, C, -B, D, N)
    assert np.array_equal(En, -E) and np.array_equal(Tn, T)
    Ed, _ = fusedmm(rp, ci, C, B, -D, N)
    assert np.array_equal(Ed, -E)
    E2, _ = fusedmm(rp, ci, 2 * C, B, D, N)
    assert np.array_equal(E2, 2 * E)


def pin_identity_D(sddmm, fusedmm):
    """With K = N and D the identity, E_i[n] is the SDDMM value of the entry
    of row i at column n (0 if none): FusedMM scatters A back into a dense
    row, so it must use each entry's own column for D."""
    rng = np.random.default_rng(15)
    M, N = 9, 8
    rp, ci = _rand_pattern(rng, M, N, 0.5)
    C = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    B = rng.uniform(-1, 1, (N, N)).astype(np.float32)
    D = np.eye(N, dtype=np.float32)
    A, _ = sddmm(rp, ci, C, B, N)
    E, _ = fusedmm(rp, ci, C, B, D, N)
    want = np.zeros((M, N))
    rows = np.repeat(np.arange(M), np.diff(rp))
    want[rows, ci] = A
    assert np.array_equal(E, want)


def pin_integer_exact(sddmm, fusedmm):
    """Small integers: every product and sum is exact in any order, so the
    values equal exact integer arithmetic (numpy int64)."""
    rng = np.random.default_rng(16)
    M, K, N = 15, 13, 6
    rp, ci = _rand_pattern(rng, M, K, 0.4)
    Ci = rng.integers(-7, 8, (M, N))
    Bi = rng.integers(-7, 8, (K, N))
    Di = rng.integers(-7, 8, (K, N))
    A, _ = sddmm(rp, ci, Ci.astype(np.float32), Bi.astype(np.float32), N)
    rows = np.repeat(np.arange(M), np.diff(rp))
    Aint = (Ci[rows] * Bi[ci]).sum(axis=1)
    assert np.array_equal(A, Aint.astype(np.float64))
    E, _ = fusedmm(rp, ci, Ci.astype(np.float32), Bi.astype(np.float32),
                   Di.astype(np.float32), N)
    Eint = np.zeros((M, N), np.int64)
    np.add.at(Eint, rows, Aint[:, None] * Di[ci])
    assert np.array_equal(E, Eint.astype(np.float64))


def pin_empty_and_offsets(sddmm, fusedmm):
    """Empty rows give no SDDMM entries and zero FusedMM rows; rowptr[0] != 0
    (a view) and the row sample return the same values as the full call."""
    rng = np.random.default_rng(17)
    lens = np.array([0, 3, 0, 0, 5, 1, 0, 2])
    M, K, N = len(lens), 9, 4
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ci = np.concatenate([np.sort(rng.choice(K, l, replace=False)) for l in lens]).astype(np.int32)
    C = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    D = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    A, _ = sddmm(rp, ci, C, B, N)
    E, T = fusedmm(rp, ci, C, B, D, N)
    assert A.shape == (lens.sum(),)
    for i in np.nonzero(lens == 0)[0]:
        assert np.array_equal(E[i], np.zeros(N)) and np.array_equal(T[i], np.zeros(N))
    # view: entries start at position 4 of a longer colind
    ci_v = np.concatenate([np.zeros(4, np.int32), ci])
    A_v, _ = sddmm(rp + 4, ci_v, C, B, N)
    assert np.array_equal(A_v, A)
    rows = np.array([4, 1, 6, 4, 7])
    As, _ = sddmm(rp, ci, C, B, N, rows=rows)
    want = np.concatenate([A[rp[i]:rp[i + 1]] for i in rows])
    assert np.array_equal(As, want)
    Es, _ = fusedmm(rp, ci, C, B, D, N, rows=rows)
    assert np.array_equal(Es, E[rows])


def pin_bf16_widening(sddmm, fusedmm):
    """bf16 operands are widened exactly: known bit patterns."""
    vals = [1.0, -2.5, 0.15625, -0.0078125, 2.0 ** -126, 2.0 ** 127, 192.0]
    bits = np.array([_bf16_bits(v) for v in vals], np.uint16)
    for v, b in zip(vals, bits):
        assert _bf16_value(int(b)) == v      # the chosen values are bf16-exact
    # one entry per value: C_0 = [bits[k]] (N = 1) times B_0 = [1.0]
    one = np.array([_bf16_bits(1.0)], np.uint16)
    for b in bits:
        A, _ = sddmm(np.array([0, 1], np.int32), np.array([0], np.int32),
                     np.array([b], np.uint16), one, 1)
        assert A[0] == _bf16_value(int(b))


def pin_bounds(sddmm, fusedmm):
    """S >= |A| and T >= |E| always; for non-negative inputs the bound is
    the value itself, bitwise (same operations in the same order)."""
    rng = np.random.default_rng(18)
    M, K, N = 20, 17, 7
    rp, ci = _rand_pattern(rng, M, K, 0.35)
    C = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    D = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    A, S = sddmm(rp, ci, C, B, N)
    E, T = fusedmm(rp, ci, C, B, D, N)
    assert np.all(S >= np.abs(A)) and np.all(T >= np.abs(E))
    Ap, Sp = sddmm(rp, ci, np.abs(C), np.abs(B), N)
    assert np.array_equal(Ap, Sp)
    Ep, Tp = fusedmm(rp, ci, np.abs(C), np.abs(B), np.abs(D), N)
    assert np.array_equal(Ep, Tp)


ALL_PINS = [pin_worked_example, pin_brute_force_python, pin_dense_matmul,
            pin_transpose_symmetry, pin_scaling_and_sign, pin_identity_D,
            pin_integer_exact, pin_empty_and_offsets, pin_bf16_widening,
            pin_bounds]
