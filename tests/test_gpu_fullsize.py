"""Full-size workloads on the GPU, in the launch configuration the benchmark
times (the plain entry points with default thresholds), compared with the
fp64 oracle on every element.  The two large workloads are compared in
blocks of consecutive rows (the oracle computes one block at a time, so the
reference never needs to hold all of C in fp64), every hub row of the
skewed matrix included.  Their plans are compared bit for bit with the plan
oracle as well."""
import sys
import time

import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import assert_parity, compare_plan, reference, run_gpu

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def log(msg):
    print(f"[fullsize] {msg}", file=sys.stderr, flush=True)


@pytest.mark.parametrize("name", ["uniform_1k_n32", "powerlaw_262k_n64",
                                  "powerlaw_262k_n64_mean16",
                                  "pruned_4k_n256_bf16", "pruned_4k_n256_f32"])
def test_full_compare(name):
    t = time.time()
    p = W.make(name)
    log(f"{name}: generated nnz={p.nnz} in {time.time() - t:.1f}s")
    C = run_gpu(p)
    Cref, Sref = reference(p)
    worst = assert_parity(C, Cref, Sref, p.dtype, name)
    log(f"{name}: all {C.size} elements within bound, worst err/S {worst:.2e}")


# Rows per oracle block: about 2^25 elements of C (two fp64 arrays of
# 256 MiB for the reference and its bound).
BLOCK_ELEMS = 1 << 25


@pytest.mark.parametrize("name", ["banded_4m_n128", "skew_1m_n512_bf16"])
def test_full_streamed(name):
    """The plan of the full matrix (default thresholds) equals the plan
    oracle bit for bit, and every element of C matches the oracle, compared
    one block of consecutive rows at a time."""
    t = time.time()
    p = W.make(name)
    log(f"{name}: generated nnz={p.nnz} in {time.time() - t:.1f}s")

    got = compare_plan(p)
    log(f"{name}: plan equal ({got['n_medium']} medium, {got['n_long']} long, "
        f"{got['n_chunks']} chunks, {got['n_hub']} hubs, {got['n_hub_chunks']} hub chunks)")
    del got

    C = run_gpu(p, fill=float("nan"))
    rows_per_block = max(1, BLOCK_ELEMS // p.N)
    worst = 0.0
    t = time.time()
    for r0 in range(0, p.M, rows_per_block):
        rows = np.arange(r0, min(p.M, r0 + rows_per_block), dtype=np.int64)
        Cref, Sref = reference(p, rows=rows)
        w = assert_parity(C[rows[0]:rows[-1] + 1], Cref, Sref, p.dtype,
                          f"{name} rows {rows[0]}..{rows[-1]}")
        worst = max(worst, w)
        del Cref, Sref
    log(f"{name}: all {p.M} rows ({C.size} elements) within bound in "
        f"{time.time() - t:.1f}s, worst err/S {worst:.2e}")
