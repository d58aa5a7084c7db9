"""GPU parity of the SDDMM entry points against the fp64 oracle.

Page: [IntelMax] "Performance Optimization of Deep Learning Sparse Matrix
Kernels on Intel Max Series GPU", the SDDMM operation (Fig. 3, Algorithm 1).

Bar: |A_gpu - A_ref| <= tol(N) * S + 1e-6 per entry, S = sum_n |C_in| |B_jn|.
tol(N) = max(1e-5, N * 2^-23): an fp32 dot product of length N computed with
fused multiply-adds in any order is off by at most about N * 2^-24 * S, and
the GPU adds the lane partials in a different order than the oracle; bf16
operands are widened exactly, so the same bound holds for them.  Cases whose
result is exact in any order are compared bit for bit.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import sparse_dense_linear_amd as sdl
import workloads as W

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def tol(N):
    return max(1e-5, N * 2.0 ** -23)


def _dense(rng, rows, N, dtype):
    x = rng.uniform(-1, 1, (rows, N)).astype(np.float32)
    if dtype == "bf16":
        return W.f32_to_bf16_bits(x)
    return x


def _dev(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda()
    return torch.from_numpy(x).cuda()


def run_sddmm(rowptr, colind, C, B, M, K, N, fill=float("nan")):
    rp = torch.from_numpy(np.ascontiguousarray(rowptr, np.int32)).cuda()
    ci = torch.from_numpy(np.ascontiguousarray(colind, np.int32)).cuda()
    nnz = int(rowptr[-1]) - int(rowptr[0])
    A = torch.full((nnz,), fill, dtype=torch.float32, device="cuda")
    if C.dtype == np.float32:
        sdl.sddmm_csr_f32(rp, ci, _dev(C), _dev(B), A, M, K, N)
    else:
        sdl.sddmm_csr_bf16in_f32acc(rp, ci, _dev(C), _dev(B), A, M, K, N)
    torch.cuda.synchronize()
    return A.cpu().numpy()


def check(rowptr, colind, C, B, M, K, N, what="", margin=None):
    """A against the oracle within the bar; with `margin`, also the worst
    |A - Aref| / S over entries with S > 0 below margin * tol(N)."""
    A = run_sddmm(rowptr, colind, C, B, M, K, N)
    Aref, S = oracle.sddmm_ref(rowptr, colind, C, B, N)
    err = np.abs(A.astype(np.float64) - Aref)
    bad = ~(err <= tol(N) * S + 1e-6)
    if bad.any():
        p = int(np.argmax(bad))
        raise AssertionError(f"{what}: {int(bad.sum())} of {A.size} outside the bound; "
                             f"first p={p}: gpu={A[p]!r} ref={Aref[p]!r} S={S[p]!r}")
    if margin is not None:
        live = S > 0
        worst = float((err[live] / S[live]).max()) if live.any() else 0.0
        assert worst <= margin * tol(N), f"{what}: worst err/S {worst:.3e}"
    return A


def pattern(lengths, K, seed):
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, np.int64)
    rowptr = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    colind = np.concatenate([np.sort(rng.choice(K, int(l), replace=False))
                             if l else np.zeros(0, np.int64) for l in lengths]).astype(np.int32)
    return rowptr, colind


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_worked_example_bitwise(dtype):
    g = json.load(open(os.path.join(GOLDEN, "worked_example_fig3_fig6.json")))
    C = np.array(g["C"], np.float32)
    B = np.array(g["B"], np.float32)
    if dtype == "bf16":
        C, B = W.f32_to_bf16_bits(C), W.f32_to_bf16_bits(B)
    A = run_sddmm(np.array(g["rowptr"]), np.array(g["colind"]), C, B,
                  g["M"], g["K"], g["N"])
    assert np.array_equal(A, np.array(g["A"], np.float32))


EDGE = [0, 1, 2, 3, 5, 17, 63, 64, 65, 130, 700]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 3, 4, 8, 32, 64, 100, 128, 256, 512, 1000])
def test_edge_rows(N, dtype):
    rng = np.random.default_rng(N)
    M, K = 250, 900
    lengths = rng.choice(EDGE, size=M)
    lengths[:len(EDGE)] = EDGE
    rp, ci = pattern(lengths, K, seed=N)
    check(rp, ci, _dense(rng, M, N, dtype), _dense(rng, K, N, dtype), M, K, N,
          f"N={N} {dtype}")


def test_long_runs_of_empty_rows():
    """Batches whose 64 entries spread over more than 64 rows (runs of
    empty rows) move the row window on, possibly several times."""
    rng = np.random.default_rng(5)
    M, K, N = 5000, 300, 64
    lengths = np.zeros(M, np.int64)
    lengths[rng.choice(M, 90, replace=False)] = rng.integers(1, 4, 90)
    lengths[-1] = 2
    rp, ci = pattern(lengths, K, seed=5)
    check(rp, ci, _dense(rng, M, N, "f32"), _dense(rng, K, N, "f32"), M, K, N)


def test_view_rowptr_offset():
    """rowptr[0] != 0: values are written at p - rowptr[0]."""
    rng = np.random.default_rng(6)
    M, K, N = 300, 500, 32
    rp, ci = pattern(rng.integers(0, 40, M), K, seed=6)
    C, B = _dense(rng, M, N, "f32"), _dense(rng, K, N, "f32")
    A0 = run_sddmm(rp, ci, C, B, M, K, N)
    pad = 7
    A1 = run_sddmm(rp + pad, np.concatenate([np.zeros(pad, np.int32), ci]), C, B, M, K, N)
    assert np.array_equal(A1, A0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_transpose_symmetry_bitwise(dtype):
    """<C_i, B_j> on a pattern equals <B_j, C_i> on the transposed pattern,
    bit for bit (same N, so the same lanes and summation order)."""
    rng = np.random.default_rng(7)
    M, K, N = 700, 500, 64
    rp, ci = pattern(rng.integers(0, 30, M), K, seed=7)
    C, B = _dense(rng, M, N, dtype), _dense(rng, K, N, dtype)
    A = run_sddmm(rp, ci, C, B, M, K, N)
    rows = np.repeat(np.arange(M), np.diff(rp))
    order = np.lexsort((rows, ci))
    rpt = np.concatenate([[0], np.cumsum(np.bincount(ci, minlength=K))]).astype(np.int32)
    At = run_sddmm(rpt, rows[order].astype(np.int32), B, C, K, M, N)
    assert np.array_equal(At, A[order])


def test_repeatable_bitwise():
    rng = np.random.default_rng(8)
    M, K, N = 2000, 2000, 64
    rp, ci = pattern(rng.integers(0, 50, M), K, seed=8)
    C, B = _dense(rng, M, N, "f32"), _dense(rng, K, N, "f32")
    assert np.array_equal(run_sddmm(rp, ci, C, B, M, K, N),
                          run_sddmm(rp, ci, C, B, M, K, N, fill=0.0))


def test_degenerate():
    rng = np.random.default_rng(9)
    # nnz == 0: nothing is written, no launch
    rp = np.zeros(11, np.int32)
    assert run_sddmm(rp, np.zeros(0, np.int32), _dense(rng, 10, 4, "f32"),
                     _dense(rng, 5, 4, "f32"), 10, 5, 4).size == 0
    # one row, one entry, N = 1
    A = run_sddmm(np.array([0, 1], np.int32), np.array([2], np.int32),
                  np.array([[3.0]], np.float32), np.array([[1.0], [2.0], [-0.5]], np.float32),
                  1, 3, 1)
    assert A[0] == -1.5
    # N == 0 with stored entries is unsupported
    rpt = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    cit = torch.tensor([0], dtype=torch.int32, device="cuda")
    Ct = torch.zeros(0, dtype=torch.float32, device="cuda")
    At = torch.zeros(1, dtype=torch.float32, device="cuda")
    with pytest.raises(sdl.SpmmError) as e:
        sdl.sddmm_csr_f32(rpt, cit, Ct, Ct, At, 1, 1, 0)
    assert e.value.status == 4


@pytest.mark.parametrize("name,N", [("powerlaw_262k_n64", 64), ("pruned_4k_n256_f32", 256),
                                    ("pruned_4k_n256_bf16", 256)])
def test_workload_patterns(name, N):
    """SDDMM on the sparsity pattern of a full workload, dense operands drawn
    with the workload's value recipe, compared element by element."""
    p = W.make(name)
    rng = np.random.default_rng(10)
    C = _dense(rng, p.M, N, p.dtype)
    # measured worst err/S: 1e-7 or less, against the bar's 1e-5 (N = 64)
    # and 3e-5 (N = 256)
    check(p.rowptr, p.colind, C, p.B.reshape(p.K, p.N), p.M, p.K, N, name, margin=0.05)


def test_banded_pattern_sampled():
    """Banded 4M-row pattern at N = 128: every entry of a row sample."""
    p = W.make("banded_4m_n128")
    rng = np.random.default_rng(11)
    C = rng.uniform(-1, 1, (p.M, p.N)).astype(np.float32)
    B = p.B.reshape(p.K, p.N)
    A = run_sddmm(p.rowptr, p.colind, C, B, p.M, p.K, p.N)
    rows = np.sort(rng.choice(p.M, 4000, replace=False))
    Aref, S = oracle.sddmm_ref(p.rowptr, p.colind, C, B, p.N, rows=rows)
    got = np.concatenate([A[p.rowptr[i]:p.rowptr[i + 1]] for i in rows])
    assert np.all(np.abs(got.astype(np.float64) - Aref) <= tol(p.N) * S + 1e-6)
