"""Full-size workloads on the GPU, in the launch configuration the benchmark
times (the plain entry points with default thresholds).  Small workloads are
compared element by element; the two large ones on sampled rows that the
oracle computes one by one (every hub row of the skewed matrix is too
expensive; a sample of hubs is included)."""
import sys
import time

import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import assert_parity, reference, run_gpu

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


@pytest.mark.parametrize("name", ["banded_4m_n128", "skew_1m_n512_bf16"])
def test_full_sampled(name):
    t = time.time()
    p = W.make(name)
    log(f"{name}: generated nnz={p.nnz} in {time.time() - t:.1f}s")
    C = run_gpu(p, fill=float("nan"))
    # every element must have been written
    assert not np.isnan(C).any(), "unwritten (NaN) elements in C"
    rng = np.random.default_rng(0)
    rows = np.concatenate([np.arange(64), np.arange(p.M - 64, p.M),
                           rng.choice(p.M, 4096, replace=False)])
    if "hubs" in p.meta:
        rows = np.concatenate([rows, rng.choice(p.meta["hubs"], 12, replace=False)])
    rows = np.unique(rows)
    Cref, Sref = reference(p, rows=rows)
    worst = assert_parity(C[rows], Cref, Sref, p.dtype, name)
    log(f"{name}: {rows.size} sampled rows within bound, worst err/S {worst:.2e}")
