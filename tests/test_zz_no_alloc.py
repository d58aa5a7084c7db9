"""The no-allocation entry point (spmm_csr_tuned_noalloc): its plan scratch
is the library's fixed per-GPU array.  Called through the C ABI and compared
with spmm_csr_tuned on the same inputs, and both with the fp64 oracle, on two
calls in a row, the second with a smaller input (the array keeps the first
call's words, which must not be taken for the second's).  Rows handled by one
wavefront (every row up to the long-row threshold) are summed in a fixed
order, so there the two entry points agree bit for bit; long rows are added
with atomics in any order and agree within the bound."""
import numpy as np
import pytest
import torch

import oracle
import sparse_dense_linear_amd as sdl
import workloads as W
from gpu_helpers import assert_parity, dev_arrays

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _both(p, dt):
    rowptr, colind, vals, B = dev_arrays(p)
    C_ref = torch.full((p.M * p.N,), float("nan"), dtype=torch.float32, device="cuda")
    C_fix = torch.full_like(C_ref, float("nan"))
    sdl.spmm_csr_tuned(dt, rowptr, colind, vals, B, C_ref, p.M, p.K, p.N)
    sdl.spmm_csr_tuned_noalloc(dt, rowptr, colind, vals, B, C_fix, p.M, p.K, p.N)
    torch.cuda.synchronize()
    assert sdl.stream_faults() == 0
    return (C_ref.cpu().numpy().reshape(p.M, p.N),
            C_fix.cpu().numpy().reshape(p.M, p.N))


def _check(p, dt):
    got_ref, got_fix = _both(p, dt)
    Cref, Sref = oracle.spmm_ref(p.rowptr, p.colind, p.vals, p.B, p.N)
    assert_parity(got_ref, Cref, Sref, p.dtype, f"{p.name} spmm_csr_tuned")
    assert_parity(got_fix, Cref, Sref, p.dtype, f"{p.name} no-alloc")
    t = sdl.resolve_tuning(dt, p.N)
    single = p.lengths() <= t.medium_max
    assert np.array_equal(got_ref[single], got_fix[single]), \
        "rows summed by one wavefront differ between the two entry points"


def test_noalloc_two_calls_second_smaller():
    big = W.powerlaw_rows(M=250000, N=64, seed=121)
    small = W.skew_rows(M=20000, N=512, hub_lo=2000, hub_hi=9000, seed=122)
    _check(big, sdl.DTYPE_F32)
    _check(small, sdl.DTYPE_BF16)


def test_noalloc_repeated_calls_and_views():
    """Many calls in a row with shrinking and growing M, including a view of
    a block of rows (rowptr + r0, C + r0 * N)."""
    p = W.powerlaw_rows(M=60000, N=32, seed=123)
    rowptr, colind, vals, B = dev_arrays(p)
    Cref, Sref = oracle.spmm_ref(p.rowptr, p.colind, p.vals, p.B, p.N)
    C = torch.full((p.M * p.N,), float("nan"), dtype=torch.float32, device="cuda")
    for r0, r1 in ((0, 60000), (1000, 1500), (0, 60000), (30000, 59999), (7, 8)):
        C.fill_(float("nan"))
        sdl.spmm_csr_tuned_noalloc(sdl.DTYPE_F32, rowptr[r0:r1 + 1], colind, vals, B,
                                   C[r0 * p.N:r1 * p.N], r1 - r0, p.K, p.N)
        torch.cuda.synchronize()
        got = C.cpu().numpy().reshape(p.M, p.N)[r0:r1]
        assert_parity(got, Cref[r0:r1], Sref[r0:r1], "f32", f"rows {r0}..{r1}")


def test_noalloc_rejects_too_many_rows():
    """Beyond the fixed array: a clear error before any work is enqueued."""
    M = 400000
    rowptr = torch.zeros(M + 1, dtype=torch.int32, device="cuda")
    empty_i = torch.zeros(0, dtype=torch.int32, device="cuda")
    empty_f = torch.zeros(0, dtype=torch.float32, device="cuda")
    B = torch.zeros(8, dtype=torch.float32, device="cuda")
    C = torch.zeros(M * 8, dtype=torch.float32, device="cuda")
    with pytest.raises(sdl.SpmmError) as e:
        sdl.spmm_csr_tuned_noalloc(sdl.DTYPE_F32, rowptr, empty_i, empty_f, B, C, M, 1, 8)
    assert e.value.status == 4  # SPMM_ERROR_UNSUPPORTED
    assert "at most" in str(e.value)
