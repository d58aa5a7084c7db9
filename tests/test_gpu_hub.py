"""Hub rows: rows above the hub threshold are cut at column-slab
boundaries, and each XCD works through its own range of slabs for all hub
rows.  The plan (hub rows, and the bounds of every hub chunk as the product
computes them) is compared bit for bit with the plan oracle, and C with the
fp64 oracle, on the edge cases of the slab cut: empty slabs, a row whose
entries all fall in one slab, one slab for all of B, one row of B per slab,
a slab count not divisible by the 8 XCDs, fewer hub chunks than queues, and
rows whose columns do not ascend (there the chunks must still tile the row,
which the oracle's bound on C checks)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_dense_linear_amd as sdl
import workloads as W
from gpu_helpers import assert_parity, compare_plan, dev_arrays, reference, run_gpu

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def hub_problem(lengths, K, N, dtype="f32", seed=0, clustered=None):
    """rows_with_lengths, optionally with one row's columns all inside
    [lo, hi) (clustered = (row, lo, hi))."""
    p = W.rows_with_lengths(lengths, K, N, seed=seed, dtype=dtype)
    if clustered is not None:
        row, lo, hi = clustered
        s, e = int(p.rowptr[row]), int(p.rowptr[row + 1])
        rng = np.random.default_rng(seed + 1)
        p.colind[s:e] = np.sort(rng.choice(np.arange(lo, hi), e - s, replace=False))
    return p


CASES = [
    # name, lengths, K, N, dtype, tuning, clustered
    ("default-skew-bf16", None, None, None, "bf16", None, None),
    ("slab-1", [0, 3, 900, 5, 1200, 0, 700], 2000, 64, "f32",
     sdl.Tuning(hub_min=600, slab_rows=1), None),
    ("one-slab", [1000, 2, 1500, 1, 3000], 5000, 32, "f32",
     sdl.Tuning(hub_min=500, slab_rows=5000), None),
    ("ragged-slabs-13", [4000, 7, 2500, 0, 9000, 33, 5000], 13000, 128, "f32",
     sdl.Tuning(hub_min=1000, slab_rows=1000), None),
    ("one-slab-holds-row", [3000, 4, 400, 8], 20000, 64, "f32",
     sdl.Tuning(hub_min=100, slab_rows=512), (2, 7168, 7680)),
    ("empty-and-edge-slabs", [600, 1, 700], 100000, 16, "f32",
     sdl.Tuning(hub_min=64, slab_rows=777), None),
    ("bf16-n512", [20000, 3, 9000, 1, 15000, 2], 30000, 512, "bf16",
     sdl.Tuning(hub_min=4000, slab_rows=2048), None),
    ("wide-n1500", [3000, 2, 2500], 6000, 1500, "f32",
     sdl.Tuning(hub_min=100, slab_rows=700), None),
]


def make_case(lengths, K, N, dtype, clustered, seed):
    if lengths is None:   # default thresholds; a 293 MiB B: hubs on by default
        return W.skew_rows(M=65536, K=300000, N=512, hub_lo=2000, hub_hi=30000, seed=seed)
    return hub_problem(lengths, K, N, dtype, seed=seed, clustered=clustered)


@pytest.mark.parametrize("name,lengths,K,N,dtype,tuning,clustered", CASES,
                         ids=[c[0] for c in CASES])
def test_hub_plan_and_product(name, lengths, K, N, dtype, tuning, clustered):
    p = make_case(lengths, K, N, dtype, clustered, seed=sum(map(ord, name)))
    got = compare_plan(p, tuning)
    assert got["n_hub"] > 0, "the case must have hub rows"
    C = run_gpu(p, tuning=tuning)
    Cref, Sref = reference(p)
    assert_parity(C, Cref, Sref, p.dtype, name)


def test_hub_unsorted_columns():
    """Hub rows whose columns are in random order: the device's slab bounds
    are a search over unsorted data, which must still tile every row (each
    entry added exactly once)."""
    p = hub_problem([5000, 3, 8000, 0, 6000], 20000, 64, seed=9)
    rng = np.random.default_rng(10)
    perm = np.arange(p.nnz)
    for i in range(p.M):
        seg = perm[p.rowptr[i]:p.rowptr[i + 1]]
        rng.shuffle(seg)
    q = W.CsrProblem(p.name, p.M, p.K, p.N, p.rowptr, np.ascontiguousarray(p.colind[perm]),
                     np.ascontiguousarray(p.vals[perm]), p.B, p.dtype)
    t = sdl.Tuning(hub_min=100, slab_rows=300)
    tr = sdl.resolve_tuning(0, q.N, t, K=q.K)
    got = sdl.plan_export(torch.from_numpy(q.rowptr).cuda(), tr,
                          colind=torch.from_numpy(q.colind).cuda(), K=q.K)
    n_hub, hc = got["n_hub"], got["hub_chunks"]
    assert n_hub == 3
    n_slabs = hc.shape[0] // n_hub
    for h, row in enumerate(got["hub_rows"]):
        mine = hc[np.arange(n_slabs) * n_hub + h]
        assert mine[0, 1] == q.rowptr[row] and mine[-1, 2] == q.rowptr[row + 1]
        assert np.all(mine[1:, 1] == mine[:-1, 2])       # tiles the row in order
    Cref, Sref = reference(q)
    assert_parity(run_gpu(q, tuning=t), Cref, Sref, "f32", "unsorted hubs")


def test_hub_rows_view_with_offset():
    """A view of a block of rows (rowptr + r0, absolute offsets) whose hub
    rows sit at its start and end."""
    p = hub_problem([7000, 1, 2, 9000, 4, 6000, 3, 8000], 30000, 64, seed=21)
    rowptr, colind, vals, B = dev_arrays(p)
    t = sdl.Tuning(hub_min=500, slab_rows=1024)
    r0, r1 = 3, 8
    C = torch.full(((r1 - r0) * p.N,), float("nan"), device="cuda")
    sdl.spmm_csr_tuned(sdl.DTYPE_F32, rowptr[r0:r1 + 1], colind, vals, B, C,
                       r1 - r0, p.K, p.N, t)
    torch.cuda.synchronize()
    Cref, Sref = reference(p)
    assert_parity(C.cpu().numpy().reshape(r1 - r0, p.N), Cref[r0:r1], Sref[r0:r1],
                  "f32", "view")


def test_hub_fusedmm_and_repeat():
    """The FusedMM form takes the same hub chunks; and a product repeated on
    the same stream (epochs advance) gives the same answer each time."""
    # B of 1,100,000 x 64 fp32 (269 MiB): hub rows by default (FusedMM
    # takes no tuning)
    p = hub_problem([4000, 2, 6000, 1, 5000], 1100000, 64, seed=31)
    rng = np.random.default_rng(32)
    Cd = rng.standard_normal((p.M, p.N)).astype(np.float32)
    Dd = rng.standard_normal((p.K, p.N), dtype=np.float32)
    rowptr, colind, _, B = dev_arrays(p)
    E = torch.full((p.M * p.N,), float("nan"), device="cuda")
    sdl.fusedmm_csr_f32(rowptr, colind, torch.from_numpy(Cd).cuda(), B,
                        torch.from_numpy(Dd).cuda(), E, p.M, p.K, p.N, p.nnz)
    torch.cuda.synchronize()
    Eref, T = oracle.fusedmm_ref(p.rowptr, p.colind, Cd, p.B, Dd, p.N)
    tol = 2 * max(1e-5, p.N * 2.0 ** -23)
    assert np.all(np.abs(E.cpu().numpy().reshape(p.M, p.N) - Eref) <= tol * T + 1e-6)
    t = sdl.Tuning(hub_min=100, slab_rows=400)
    Cref, Sref = reference(p)
    for _ in range(3):
        assert_parity(run_gpu(p, tuning=t), Cref, Sref, "f32", "repeat")
