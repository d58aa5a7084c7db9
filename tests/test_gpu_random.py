"""Seeded random sweep of the product (and of SDDMM and FusedMM on some of
the cases) against the fp64 oracle: random
shapes, row-length mixes, dense widths, element types, routing thresholds
(short, medium, long and hub rows in every proportion), column orders
(sorted, shuffled within rows, repeated columns) and row-block views
(rowptr[0] != 0).  Each case is checked element by element, with C
NaN-filled first, and with the fault count read after the call; the
element-balanced kernel and the no-allocation entry point are run on some
of the cases too.  The generator is seeded per case, so a failure names a
reproducible case."""
import numpy as np
import pytest
import torch

import oracle
import sparse_dense_linear_amd as sdl
import workloads as W
from gpu_helpers import assert_parity, dev_arrays

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

WIDTHS = [1, 2, 3, 4, 5, 7, 8, 12, 16, 24, 31, 32, 33, 48, 64, 100, 128, 200, 256,
          300, 512, 520, 1024]


def random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    N = int(rng.choice(WIDTHS))
    dtype = "bf16" if rng.random() < 0.35 else "f32"
    K = int(rng.integers(1, 6000))
    M = int(rng.integers(1, 2500))
    mix = rng.choice(["short", "mixed", "heavy"])
    if mix == "short":
        lengths = rng.integers(0, 9, M)
    elif mix == "mixed":
        lengths = rng.choice([0, 1, 3, 8, 20, 70, 300, 1500], size=M,
                             p=[.1, .3, .2, .15, .1, .08, .05, .02])
    else:
        lengths = rng.choice([0, 2, 40, 600, 4000], size=M, p=[.1, .4, .3, .15, .05])
    # keep the case small enough for the oracle: at most ~3e8 multiply-adds
    budget = max(1, int(3e8 // max(N, 1)))
    while lengths.sum() > budget and lengths.max() > 1:
        lengths = np.maximum(lengths // 2, np.minimum(lengths, 1))
    lengths = np.minimum(lengths, K)           # a row may hold every column
    order = rng.choice(["sorted", "shuffled", "repeats"], p=[.6, .25, .15])
    rows = []
    for n in lengths:
        c = rng.permutation(K)[:n]                 # distinct columns
        if order == "sorted":
            c = np.sort(c)
        elif order == "repeats" and n > 1:         # a few columns repeated
            k = max(1, n // 4)
            c[rng.integers(0, n, k)] = c[rng.integers(0, n, k)]
        rows.append(c)
    cols = np.concatenate(rows + [np.zeros(0, np.int64)])
    vals32 = rng.uniform(-1, 1, cols.size).astype(np.float32)
    B32 = rng.uniform(-1, 1, K * N).astype(np.float32)
    rowptr = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    if dtype == "bf16":
        vals, B = W.f32_to_bf16_bits(vals32), W.f32_to_bf16_bits(B32).reshape(K, N)
    else:
        vals, B = vals32, B32.reshape(K, N)
    p = W.CsrProblem(f"random{seed}", M, K, N, rowptr, cols.astype(np.int32), vals, B,
                     dtype)
    # routing thresholds: library defaults or a random valid set
    if rng.random() < 0.3:
        tuning = None
    else:
        short_max = int(rng.choice([0, 1, 2, 4, 8, 16]))
        medium_max = int(short_max + rng.choice([0, 1, 10, 64, 256, 2000]))
        chunk = int(rng.choice([1, 7, 32, 128, 512, 4096]))
        hub = int(rng.choice([-1, medium_max, medium_max + 100, 3000]))
        slab = int(rng.choice([1, 17, 256, 4096, 1 << 20]))
        tuning = sdl.Tuning(short_max, medium_max, chunk, hub_min=hub, slab_rows=slab)
        try:     # the tuning must be one the product accepts (short tile capacity)
            sdl.resolve_tuning(0 if dtype == "f32" else 1, N, tuning, K=K)
        except sdl.SpmmError:
            tuning = None
    view = rng.random() < 0.25 and M > 4
    what = (f"seed={seed} M={M} K={K} N={N} {dtype} {mix} {order} nnz={p.nnz} "
            f"tuning={tuning} view={view}")
    return p, tuning, view, what, rng


def run_tuned(p, tuning, fn, rows=None):
    dt = sdl.DTYPE_F32 if p.dtype == "f32" else sdl.DTYPE_BF16
    rowptr, colind, vals, B = dev_arrays(p)
    C = torch.full((p.M * p.N,), float("nan"), dtype=torch.float32, device="cuda")
    if rows is None:
        fn(dt, rowptr, colind, vals, B, C, p.M, p.K, p.N, tuning)
    else:
        r0, r1 = rows
        fn(dt, rowptr[r0:r1 + 1], colind, vals, B, C[r0 * p.N:r1 * p.N], r1 - r0, p.K, p.N,
           tuning)
    torch.cuda.synchronize()
    assert sdl.stream_faults() == 0
    return C.cpu().numpy().reshape(p.M, p.N)


def sddmm_tol(N):
    """The SDDMM bar of test_gpu_sddmm: an fp32 dot product of length N."""
    return max(1e-5, N * 2.0 ** -23)


def dense_like(p, rng, rows):
    """A dense rows x N operand in p's element type (as uploaded, and as the
    oracle reads it)."""
    x = rng.uniform(-1, 1, (rows, p.N)).astype(np.float32)
    return W.f32_to_bf16_bits(x).reshape(rows, p.N) if p.dtype == "bf16" else x


def to_dev(x):
    x = np.ascontiguousarray(x).reshape(-1)
    return torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).cuda()


def check_sddmm_fusedmm(p, rng, what, fused):
    rowptr, colind, _, B = dev_arrays(p)
    Cn = dense_like(p, rng, p.M)
    if not fused:
        A = torch.full((p.nnz,), float("nan"), dtype=torch.float32, device="cuda")
        fn = sdl.sddmm_csr_f32 if p.dtype == "f32" else sdl.sddmm_csr_bf16in_f32acc
        fn(rowptr, colind, to_dev(Cn), B, A, p.M, p.K, p.N)
        torch.cuda.synchronize()
        assert sdl.stream_faults() == 0
        Aref, S = oracle.sddmm_ref(p.rowptr, p.colind, Cn, p.B, p.N)
        err = np.abs(A.cpu().numpy().astype(np.float64) - Aref)
        assert np.all(err <= sddmm_tol(p.N) * S + 1e-6), what + " sddmm"
        return
    Dn = dense_like(p, rng, p.K)
    E = torch.full((p.M * p.N,), float("nan"), dtype=torch.float32, device="cuda")
    fn = sdl.fusedmm_csr_f32 if p.dtype == "f32" else sdl.fusedmm_csr_bf16in_f32acc
    fn(rowptr, colind, to_dev(Cn), B, to_dev(Dn), E, p.M, p.K, p.N, p.nnz)
    torch.cuda.synchronize()
    assert sdl.stream_faults() == 0
    Eref, T = oracle.fusedmm_ref(p.rowptr, p.colind, Cn, p.B, Dn, p.N)
    err = np.abs(E.cpu().numpy().reshape(p.M, p.N).astype(np.float64) - Eref)
    assert np.all(err <= 2 * sddmm_tol(p.N) * T + 1e-6), what + " fusedmm"


@pytest.mark.parametrize("seed", range(120))
def test_random_case(seed):
    p, tuning, view, what, rng = random_case(seed)
    Cref, Sref = oracle.spmm_ref(p.rowptr, p.colind, p.vals, p.B, p.N)
    if view:
        r0 = int(rng.integers(0, p.M // 2))
        r1 = int(rng.integers(r0 + 1, p.M + 1))
        got = run_tuned(p, tuning, sdl.spmm_csr_tuned, rows=(r0, r1))
        assert_parity(got[r0:r1], Cref[r0:r1], Sref[r0:r1], p.dtype, what)
    else:
        got = run_tuned(p, tuning, sdl.spmm_csr_tuned)
        assert_parity(got, Cref, Sref, p.dtype, what)
    if seed % 4 == 0 and p.M <= 300000:
        got = run_tuned(p, tuning, sdl.spmm_csr_tuned_noalloc)
        assert_parity(got, Cref, Sref, p.dtype, what + " no-alloc")
    if seed % 4 == 1:
        dt = sdl.DTYPE_F32 if p.dtype == "f32" else sdl.DTYPE_BF16
        rowptr, colind, vals, B = dev_arrays(p)
        C = torch.full((p.M * p.N,), float("nan"), dtype=torch.float32, device="cuda")
        sdl.spmm_csr_eb(dt, rowptr, colind, vals, B, C, p.M, p.K, p.N)
        torch.cuda.synchronize()
        assert sdl.stream_faults() == 0
        assert_parity(C.cpu().numpy().reshape(p.M, p.N), Cref, Sref, p.dtype, what + " eb")
    if seed % 4 in (2, 3) and p.nnz > 0:
        check_sddmm_fusedmm(p, rng, what, fused=seed % 4 == 3)
