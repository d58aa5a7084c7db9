"""GPU parity of the element-balanced product (spmm_csr_eb) against the
fp64 oracle.

Page: [Sgap] "Sgap: Towards Efficient Sparse Tensor Algebra Compilation for
GPU", element-balanced atomic parallelism with grouped segmented reduction.
Same bar as the planned product: |C - C_ref| <= tol S + 1e-6 (tol 1e-5 for
fp32 inputs, 1e-2 for bf16 inputs); this kernel sums every row in a fixed
order, so two runs must agree bit for bit.
"""
import json
import os

import numpy as np
import pytest
import torch

import sparse_dense_linear_amd as sdl
import workloads as W
from gpu_helpers import assert_parity, dev_arrays, reference
from test_gpu_parity import GOLDEN, edge_problem

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def run_eb(p, fill=float("nan"), rowptr=None, colind=None):
    rp, ci, vals, B = dev_arrays(p)
    if rowptr is not None:
        rp = torch.from_numpy(rowptr).cuda()
        ci = torch.from_numpy(colind).cuda()
        pad = int(rowptr[0])
        vals = torch.cat([torch.zeros(pad, dtype=vals.dtype, device="cuda"), vals])
    C = torch.full((p.M * p.N,), fill, dtype=torch.float32, device="cuda")
    dt = sdl.DTYPE_F32 if p.dtype == "f32" else sdl.DTYPE_BF16
    sdl.spmm_csr_eb(dt, rp, ci, vals, B, C, p.M, p.K, p.N)
    torch.cuda.synchronize()
    return C.cpu().numpy().reshape(p.M, p.N)


def check(p, what=""):
    C = run_eb(p)
    Cref, Sref = reference(p)
    assert_parity(C, Cref, Sref, p.dtype, what or p.name)
    return C


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_worked_example_bitwise(dtype):
    g = json.load(open(os.path.join(GOLDEN, "worked_example_fig5.json")))
    vals = np.array(g["vals"], np.float32)
    B = np.array(g["B"], np.float32)
    if dtype == "bf16":
        vals, B = W.f32_to_bf16_bits(vals), W.f32_to_bf16_bits(B)
    p = W.CsrProblem("fig5", g["M"], g["K"], g["N"], np.array(g["rowptr"], np.int32),
                     np.array(g["colind"], np.int32), vals, B, dtype)
    assert np.array_equal(run_eb(p), np.array(g["C"], np.float32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 3, 4, 8, 32, 33, 64, 100, 128, 256, 512, 1000,
                               1025, 2304])
def test_edge_rows(N, dtype):
    check(edge_problem(N, dtype), f"N={N} {dtype}")


def test_empty_rows_everywhere():
    """Leading, trailing and long runs of empty rows (more than 64 in a row,
    so a batch's row window moves on), and rows at span boundaries."""
    rng = np.random.default_rng(9)
    M = 20000
    lengths = np.zeros(M, np.int64)
    idx = rng.choice(np.arange(100, M - 100), 300, replace=False)
    lengths[idx] = rng.integers(1, 40, 300)
    check(W.rows_with_lengths(lengths, 500, 64, seed=9))


def test_no_entries():
    p = W.rows_with_lengths(np.zeros(3000, np.int64), 10, 16, seed=1)
    assert np.array_equal(run_eb(p), np.zeros((3000, 16), np.float32))


def test_one_row_spanning_every_wave():
    """A single very long row crosses every span: its partials travel
    through a long run of carry slots."""
    p = W.rows_with_lengths([0, 600000, 0, 3], 700000, 64, seed=2)
    check(p, "one long row")


def test_view_rowptr_offset():
    p = edge_problem(64, "f32", M=300, seed=3)
    C0 = run_eb(p)
    pad = 9
    rp = (p.rowptr + pad).astype(np.int32)
    ci = np.concatenate([np.zeros(pad, np.int32), p.colind])
    C1 = run_eb(p, rowptr=rp, colind=ci)
    assert np.array_equal(C0, C1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_repeatable_bitwise(dtype):
    p = W.powerlaw_rows(M=32768, N=64, seed=7, dtype=dtype)
    assert np.array_equal(run_eb(p), run_eb(p, fill=0.0))


@pytest.mark.parametrize("name", ["powerlaw_262k_n64", "pruned_4k_n256_bf16",
                                  "pruned_4k_n256_f32", "uniform_1k_n32"])
def test_full_workloads(name):
    check(W.make(name))


def test_skew_scaled():
    check(W.skew_rows(M=60000, N=512, hub_lo=2000, hub_hi=30000), "skew")
