"""The give-up path of the product's bounded plan waits, forced from the
host: with the wait bound set to 0 polls every item that needs a plan entry
(medium rows, long-row chunks, hub chunks) is left undone and counted,
while every kernel still runs to its end; the count reaches the caller
through spmm_stream_faults, and the calls after the bound is restored are
exact again (their queue counters were cleared as usual).  Short rows need
no plan entry, so they are still exact in the call that gave up."""
import numpy as np
import pytest
import torch

import sparse_dense_linear_amd as sdl
import workloads as W
from gpu_helpers import assert_parity, dev_arrays, reference

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def mixed_problem():
    """Short, medium, long and hub rows (with the tuning below)."""
    rng = np.random.default_rng(61)
    lengths = rng.choice([0, 1, 5, 9, 40, 200, 1500], size=6000)
    lengths[[17, 2500, 5999]] = [5000, 7000, 6500]
    return W.rows_with_lengths(lengths, 8000, 64, seed=61)


TUNING = sdl.Tuning(short_max=8, medium_max=256, chunk_nnz=256, hub_min=4000,
                    slab_rows=1000)


def short_rows(p, tuning):
    t = sdl.resolve_tuning(sdl.DTYPE_F32, p.N, tuning, K=p.K)
    return np.nonzero(np.diff(p.rowptr) <= t.short_max)[0]


@pytest.mark.parametrize("entry", ["tuned", "noalloc"])
def test_waits_that_give_up_are_counted_then_calls_are_exact(entry):
    p = mixed_problem()
    args = dev_arrays(p)
    fn = sdl.spmm_csr_tuned if entry == "tuned" else sdl.spmm_csr_tuned_noalloc
    Cref, Sref = reference(p)
    assert sdl.stream_faults() == 0           # and the count starts from zero
    C = torch.full((p.M * p.N,), float("nan"), device="cuda")
    try:
        sdl.debug_set_wait_polls(0)
        fn(sdl.DTYPE_F32, *args, C, p.M, p.K, p.N, TUNING)
    finally:
        sdl.debug_set_wait_polls(-1)
    torch.cuda.synchronize()
    assert sdl.stream_faults() > 0
    assert sdl.stream_faults() == 0           # reading resets it
    rows = short_rows(p, TUNING)
    got = C.cpu().numpy().reshape(p.M, p.N)
    assert_parity(got[rows], Cref[rows], Sref[rows], "f32", f"{entry}: short rows")
    # the next calls, with the default bound, are exact and fault-free
    for _ in range(2):
        C.fill_(float("nan"))
        fn(sdl.DTYPE_F32, *args, C, p.M, p.K, p.N, TUNING)
        torch.cuda.synchronize()
        assert sdl.stream_faults() == 0
        assert_parity(C.cpu().numpy().reshape(p.M, p.N), Cref, Sref, "f32", entry)


def test_fault_count_survives_scratch_growth():
    """Items counted in a stream's scratch block are still reported after a
    larger call has replaced the block (the count moves to the new one)."""
    p = mixed_problem()
    args = dev_arrays(p)
    s = torch.cuda.Stream()
    C = torch.full((p.M * p.N,), float("nan"), device="cuda")
    with torch.cuda.stream(s):
        sdl.stream_release(s)                  # a fresh, small block
        try:
            sdl.debug_set_wait_polls(0)
            sdl.spmm_csr_tuned(sdl.DTYPE_F32, *args, C, p.M, p.K, p.N, TUNING, stream=s)
        finally:
            sdl.debug_set_wait_polls(-1)
        # a call with 40 x the rows needs a larger block
        big = W.rows_with_lengths(np.full(40 * p.M, 3), 100, 8, seed=62)
        bargs = dev_arrays(big)
        Cb = torch.full((big.M * big.N,), float("nan"), device="cuda")
        sdl.spmm_csr_f32(*bargs, Cb, big.M, big.K, big.N, stream=s)
    s.synchronize()
    assert sdl.stream_faults(s) > 0
    assert sdl.stream_faults(s) == 0
    Cref, Sref = reference(big)
    assert_parity(Cb.cpu().numpy().reshape(big.M, big.N), Cref, Sref, "f32", "after growth")
    sdl.stream_release(s)
