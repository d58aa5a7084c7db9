"""GPU parity with B above 4 GiB, where the product kernels gather through
flat 64-bit addresses instead of 32-bit offsets into a buffer resource.

B (K x N fp32, K = 2^20 + 4096, N = 1024: 4.3 GB) is drawn on the GPU; the
pattern's columns are drawn so that many of them point past the 4 GiB
boundary (row 2^20 of B starts at byte 2^32), including the last row.  The
oracle gets the referenced rows of B only, with the columns renumbered into
that compact copy: every entry still multiplies the same value by the same
row, in the same order, so C and the bound S are unchanged.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_dense_linear_amd as sdl
from gpu_helpers import assert_parity

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

K = (1 << 20) + 4096
N = 1024
M = 2048


def _problem(seed, lo=0, hi=40):
    rng = np.random.default_rng(seed)
    lengths = rng.integers(lo, hi, M)
    lengths[:6] = [0, 1, 300, 700, 2000, 5]   # empty, short, medium and long rows
    rowptr = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    cols = []
    for n in lengths:
        # half of each row's columns beyond row 2^20 of B (past 4 GiB)
        hi = rng.choice(np.arange(1 << 20, K), size=n // 2, replace=False)
        lo = rng.choice(1 << 20, size=n - n // 2, replace=False)
        cols.append(np.sort(np.concatenate([lo, hi])))
    colind = np.concatenate(cols).astype(np.int32)
    colind[-1] = K - 1                          # the last row of B
    vals = rng.uniform(-1, 1, colind.size).astype(np.float32)
    return rowptr, colind, vals


@pytest.mark.parametrize("kernel", ["planned", "element_balanced"])
def test_B_above_4GiB(kernel):
    assert K * N * 4 > (1 << 32)
    rowptr, colind, vals = _problem(seed=11)
    g = torch.Generator(device="cuda")
    g.manual_seed(12)
    B = torch.randn(K * N, generator=g, device="cuda")
    C = torch.full((M * N,), float("nan"), device="cuda")
    rp = torch.from_numpy(rowptr).cuda()
    ci = torch.from_numpy(colind).cuda()
    v = torch.from_numpy(vals).cuda()
    if kernel == "planned":
        sdl.spmm_csr_f32(rp, ci, v, B, C, M, K, N)
    else:
        sdl.spmm_csr_eb(sdl.DTYPE_F32, rp, ci, v, B, C, M, K, N)
    torch.cuda.synchronize()
    assert sdl.stream_faults() == 0

    used, compact = np.unique(colind, return_inverse=True)
    B_used = B.view(K, N)[torch.from_numpy(used).cuda().long()].cpu().numpy()
    del B
    Cref, Sref = oracle.spmm_ref(rowptr, compact.astype(np.int32), vals, B_used, N)
    assert_parity(C.cpu().numpy().reshape(M, N), Cref, Sref, "f32", f"B > 4 GiB, {kernel}")


def test_fusedmm_B_above_4GiB():
    """FusedMM's one-launch form through flat addresses: B (and D, the same
    array here) above 4 GiB.  At N = 1024 the one launch is taken for rows
    of 32 entries or more on average, so the rows here are that long."""
    rowptr, colind, _ = _problem(seed=13, lo=30, hi=60)
    assert colind.size >= 32 * M
    g = torch.Generator(device="cuda")
    g.manual_seed(14)
    B = torch.randn(K * N, generator=g, device="cuda")
    Cd = torch.randn(M * N, generator=g, device="cuda")
    E = torch.full((M * N,), float("nan"), device="cuda")
    rp = torch.from_numpy(rowptr).cuda()
    ci = torch.from_numpy(colind).cuda()
    sdl.fusedmm_csr_f32(rp, ci, Cd, B, B, E, M, K, N, colind.size)
    torch.cuda.synchronize()
    assert sdl.stream_faults() == 0

    used, compact = np.unique(colind, return_inverse=True)
    B_used = B.view(K, N)[torch.from_numpy(used).cuda().long()].cpu().numpy()
    del B
    C_host = Cd.cpu().numpy().reshape(M, N)
    Eref, T = oracle.fusedmm_ref(rowptr, compact.astype(np.int32), C_host, B_used, B_used, N)
    got = E.cpu().numpy().reshape(M, N).astype(np.float64)
    tol = 2 * max(1e-5, N * 2.0 ** -23)   # the FusedMM bound of test_gpu_fusedmm
    bad = ~(np.abs(got - Eref) <= tol * T + 1e-6)
    assert not bad.any(), f"{int(bad.sum())} of {got.size} outside the bound"
