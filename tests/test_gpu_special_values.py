"""Infinities and NaN in B go where IEEE arithmetic sends them, and nowhere
else: C[i, n] is NaN or +-Inf exactly when the fp64 oracle's is, with the
same sign, and every other element is within the usual bound.  This pins
the gather slots that carry no entry (rows shorter than a batch, the tails
of medium rows, chunks and hub chunks, element-balanced batches): such a
slot must leave the accumulator as it is, even when the row of B it would
otherwise touch holds an infinity, and must not move a non-finite value
into another column.  Both element types, short/medium/long/hub rows, the
row-split kernel and the element-balanced kernel; SDDMM values and FusedMM
rows (their bf16 dot products pair neighbouring columns) too."""
import numpy as np
import pytest
import torch

import oracle
import sparse_dense_linear_amd as sdl
import workloads as W
from gpu_helpers import ABS, TOL, dev_arrays

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

K = 2000
BF16_BITS = {"inf": 0x7F80, "-inf": 0xFF80, "nan": 0x7FC0}


def problem(dtype, N, seed, K=K, M=3000):
    rng = np.random.default_rng(seed)
    lengths = rng.choice([0, 1, 2, 3, 5, 7, 9, 12, 30, 100, 700, 1500], size=M,
                         p=[.05, .1, .1, .1, .1, .1, .1, .1, .1, .08, .05, .02])
    p = W.rows_with_lengths(lengths, K, N, seed=seed, dtype=dtype)
    # one special value in about 5 % of the rows of B, at a random column
    rows = rng.choice(K, K // 20, replace=False)
    cols = rng.integers(0, N, rows.size)
    kinds = rng.choice(list(BF16_BITS), rows.size)
    B = p.B.reshape(K, N)
    for r, c, kd in zip(rows, cols, kinds):
        if dtype == "bf16":
            B[r, c] = BF16_BITS[kd]
        else:
            B[r, c] = {"inf": np.inf, "-inf": -np.inf, "nan": np.nan}[kd]
    return p


def check(got, p, what):
    Cref, S = oracle.spmm_ref(p.rowptr, p.colind, p.vals, p.B, p.N)
    nan_ref, nan_got = np.isnan(Cref), np.isnan(got)
    assert nan_ref.any() and np.isinf(Cref).any(), "the case must hold specials"
    assert np.array_equal(nan_got, nan_ref), f"{what}: NaN pattern"
    inf_ref = np.isinf(Cref)
    assert np.array_equal(np.isinf(got), inf_ref), f"{what}: Inf pattern"
    assert np.array_equal(np.sign(got[inf_ref]), np.sign(Cref[inf_ref])), f"{what}: Inf sign"
    fin = np.isfinite(Cref)
    err = np.abs(got[fin].astype(np.float64) - Cref[fin])
    assert np.all(err <= TOL["f32"] * S[fin] + ABS), f"{what}: finite elements"


TUNINGS = [None,
           sdl.Tuning(short_max=8, medium_max=256, chunk_nnz=64),
           sdl.Tuning(short_max=4, medium_max=64, chunk_nnz=32, hub_min=600, slab_rows=128)]


@pytest.mark.parametrize("dtype,N", [("bf16", 256), ("bf16", 64), ("f32", 64)])
def test_special_values_stay_in_their_columns(dtype, N):
    p = problem(dtype, N, seed=91 + N)
    dt = sdl.DTYPE_F32 if dtype == "f32" else sdl.DTYPE_BF16
    args = dev_arrays(p)
    for tuning in TUNINGS:
        C = torch.full((p.M * p.N,), 7.0, dtype=torch.float32, device="cuda")
        sdl.spmm_csr_tuned(dt, *args, C, p.M, p.K, p.N, tuning)
        torch.cuda.synchronize()
        assert sdl.stream_faults() == 0
        check(C.cpu().numpy().reshape(p.M, p.N), p, f"{dtype} N={N} {tuning}")
    C = torch.full((p.M * p.N,), 7.0, dtype=torch.float32, device="cuda")
    sdl.spmm_csr_eb(dt, *args, C, p.M, p.K, p.N)
    torch.cuda.synchronize()
    assert sdl.stream_faults() == 0
    check(C.cpu().numpy().reshape(p.M, p.N), p, f"{dtype} N={N} element-balanced")


def test_special_values_pair_form():
    """B of 307 MB with rows of 512 bytes (bf16, N = 256): the PAIR form, two
    medium rows per item, one column half each."""
    p = problem("bf16", 256, seed=97, K=600_000, M=2000)
    args = dev_arrays(p)
    C = torch.full((p.M * p.N,), 7.0, dtype=torch.float32, device="cuda")
    sdl.spmm_csr_bf16in_f32acc(*args, C, p.M, p.K, p.N)
    torch.cuda.synchronize()
    assert sdl.stream_faults() == 0
    check(C.cpu().numpy().reshape(p.M, p.N), p, "bf16 N=256 PAIR form")


def check_values(got, ref, S, tol, what):
    """NaN and infinities where the fp64 oracle has them (with their signs),
    every finite value within tol * S + 1e-6."""
    assert np.isnan(ref).any() and np.isinf(ref).any(), "the case must hold specials"
    assert np.array_equal(np.isnan(got), np.isnan(ref)), f"{what}: NaN pattern"
    inf = np.isinf(ref)
    assert np.array_equal(np.isinf(got), inf), f"{what}: Inf pattern"
    assert np.array_equal(np.sign(got[inf]), np.sign(ref[inf])), f"{what}: Inf sign"
    fin = np.isfinite(ref)
    err = np.abs(got[fin].astype(np.float64) - ref[fin])
    assert np.all(err <= tol * S[fin] + ABS), f"{what}: finite values"


@pytest.mark.parametrize("dtype,N", [("bf16", 256), ("bf16", 12), ("f32", 64)])
def test_special_values_sddmm_fusedmm(dtype, N):
    """SDDMM values and FusedMM rows with infinities and NaN in B: each dot
    product (bf16: by dot-product instructions over column pairs) is
    non-finite exactly where IEEE arithmetic makes it so.  bf16 at N = 12
    takes FusedMM's widened fp32 copy."""
    p = problem(dtype, N, seed=131 + N, M=1500)
    rng = np.random.default_rng(131)
    x = rng.uniform(-1, 1, (p.M, p.N)).astype(np.float32)
    d = rng.uniform(-1, 1, (p.K, p.N)).astype(np.float32)
    if dtype == "bf16":
        x = W.f32_to_bf16_bits(x).reshape(p.M, p.N)
        d = W.f32_to_bf16_bits(d).reshape(p.K, p.N)
    def dev(a):
        a = np.ascontiguousarray(a).reshape(-1)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()
    rowptr, colind, _, B = dev_arrays(p)
    tol = max(1e-5, p.N * 2.0 ** -23)
    A = torch.full((p.nnz,), 7.0, dtype=torch.float32, device="cuda")
    fn = sdl.sddmm_csr_f32 if dtype == "f32" else sdl.sddmm_csr_bf16in_f32acc
    fn(rowptr, colind, dev(x), B, A, p.M, p.K, p.N)
    torch.cuda.synchronize()
    assert sdl.stream_faults() == 0
    Aref, S = oracle.sddmm_ref(p.rowptr, p.colind, x, p.B, p.N)
    check_values(A.cpu().numpy(), Aref, S, tol, f"sddmm {dtype} N={N}")
    E = torch.full((p.M * p.N,), 7.0, dtype=torch.float32, device="cuda")
    fn = sdl.fusedmm_csr_f32 if dtype == "f32" else sdl.fusedmm_csr_bf16in_f32acc
    fn(rowptr, colind, dev(x), B, dev(d), E, p.M, p.K, p.N, p.nnz)
    torch.cuda.synchronize()
    assert sdl.stream_faults() == 0
    Eref, T = oracle.fusedmm_ref(p.rowptr, p.colind, x, p.B, d, p.N)
    check_values(E.cpu().numpy().reshape(p.M, p.N), Eref, T, 2 * tol,
                 f"fusedmm {dtype} N={N}")
