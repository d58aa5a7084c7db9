"""GPU parity: the HIP library through its C ABI against the fp64 oracle.

Bar: |C_gpu - C_ref| <= tol * S + 1e-6 per element with S = |A||B|
(tol 1e-5 for fp32 inputs, 1e-2 for bf16 inputs with fp32 accumulation);
the row plan is compared bit for bit with the plan oracle; cases whose
result is exact in any summation order are compared bit for bit.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import sparse_dense_linear_amd as sdl
import workloads as W
from gpu_helpers import assert_parity, call, compare_plan, dev_arrays, reference, run_gpu

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Row lengths around every routing boundary of the default thresholds, and
# long rows spanning many chunks; K must exceed the longest row.
EDGE_LENGTHS = [0, 1, 2, 3, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65,
                127, 128, 129, 255, 256, 257, 511, 512, 513, 1000, 1023, 1024,
                1025, 2047, 2048, 2049, 5000]


def edge_problem(N, dtype, M=300, K=6000, seed=0):
    rng = np.random.default_rng(seed)
    lengths = rng.choice(EDGE_LENGTHS, size=M)
    lengths[:len(EDGE_LENGTHS)] = EDGE_LENGTHS
    return W.rows_with_lengths(lengths, K, N, seed=seed, dtype=dtype)


def test_worked_example_bitwise():
    """Fig. 5 structure with dyadic values: exact in every order."""
    with open(os.path.join(GOLDEN, "worked_example_fig5.json")) as f:
        g = json.load(f)
    vals = np.array(g["vals"], dtype=np.float32)
    B = np.array(g["B"], dtype=np.float32)
    for dtype in ("f32", "bf16"):
        v = vals if dtype == "f32" else W.f32_to_bf16_bits(vals)
        b = B if dtype == "f32" else W.f32_to_bf16_bits(B)
        p = W.CsrProblem("fig5", g["M"], g["K"], g["N"],
                         np.array(g["rowptr"], dtype=np.int32),
                         np.array(g["colind"], dtype=np.int32), v, b, dtype)
        C = run_gpu(p)
        assert np.array_equal(C, np.array(g["C"], dtype=np.float32)), dtype


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 3, 4, 8, 32, 33, 64, 100, 128, 256, 512, 1000,
                               1025, 1500, 2304])
def test_edge_rows_all_paths(N, dtype):
    """Rows of every length class (empty, short, medium, long with many
    chunks) for many N, including N that are not multiples of the lane
    vector and N that take several column passes (1025: 5 passes of 256
    single-element columns in fp32; 1500 and 2304: 2-3 passes of 16-byte
    vectors, the last one partial)."""
    p = edge_problem(N, dtype, seed=N)
    C = run_gpu(p)
    Cref, Sref = reference(p)
    assert_parity(C, Cref, Sref, dtype, f"N={N} {dtype}")


@pytest.mark.parametrize("tuning", [
    sdl.Tuning(0, 0, 1),        # every non-empty row long, one entry per chunk
    sdl.Tuning(1, 4, 3),        # tiny bins, many chunks
    sdl.Tuning(5000, 5000, 4096),  # everything short
    sdl.Tuning(0, 100000, 64),  # everything medium
    sdl.Tuning(16, 64, 7),      # odd chunk size
])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forced_thresholds(tuning, dtype):
    p = edge_problem(64, dtype, M=150, seed=7)
    C = run_gpu(p, tuning=tuning)
    Cref, Sref = reference(p)
    assert_parity(C, Cref, Sref, dtype, f"{tuning} {dtype}")


def test_chunk_table_overflow():
    """More chunks than the chunk table holds (M + 4096): the worker
    recomputes descriptors past the table from the long-row list."""
    p = W.rows_with_lengths([9000, 0, 12000, 3, 7000], K=20000, N=32, seed=3)
    t = sdl.Tuning(2, 8, 3)   # ~9300 chunks for 5 rows
    C = run_gpu(p, tuning=t)
    Cref, Sref = reference(p)
    assert_parity(C, Cref, Sref, "f32", "chunk table overflow")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_misaligned_operands(dtype):
    """B and C offset by one element from a 16-byte boundary: the library
    falls back to narrower lane vectors with the same results."""
    p = edge_problem(64, dtype, M=120, seed=11)
    rowptr, colind, vals, B = dev_arrays(p)
    Bbuf = torch.zeros(B.numel() + 1, dtype=B.dtype, device="cuda")
    Bbuf[1:] = B
    Cbuf = torch.full((p.M * p.N + 1,), float("nan"), device="cuda")
    call(p, rowptr, colind, vals, Bbuf[1:], Cbuf[1:])
    torch.cuda.synchronize()
    C = Cbuf[1:].cpu().numpy().reshape(p.M, p.N)
    Cref, Sref = reference(p)
    assert_parity(C, Cref, Sref, dtype, "misaligned")


def test_row_block_view():
    """rowptr + r0 with absolute offsets and C + r0*N: the rows of a block
    equal the same rows of the full product."""
    p = edge_problem(32, "f32", M=200, seed=5)
    full = run_gpu(p)
    rowptr, colind, vals, B = dev_arrays(p)
    r0, r1 = 37, 151
    C = torch.full(((r1 - r0) * p.N,), float("nan"), device="cuda")
    call(p, rowptr[r0:r1 + 1], colind, vals, B, C, M=r1 - r0)
    torch.cuda.synchronize()
    Cv = C.cpu().numpy().reshape(r1 - r0, p.N)
    # rows in one wavefront are computed the same way in both calls
    lens = np.diff(p.rowptr)[r0:r1]
    t = sdl.resolve_tuning(0, p.N)
    det = lens <= t.medium_max
    assert np.array_equal(Cv[det], full[r0:r1][det])
    Cref, Sref = reference(p)
    assert_parity(Cv, Cref[r0:r1], Sref[r0:r1], "f32", "view")


def test_degenerate_shapes():
    # K == 0 (no entries at all): C must be overwritten with zeros
    p = W.rows_with_lengths(np.zeros(70, dtype=np.int64), K=0, N=16)
    C = run_gpu(p)
    assert np.array_equal(C, np.zeros((70, 16), dtype=np.float32))
    # all rows empty with K > 0
    p = W.rows_with_lengths(np.zeros(1000, dtype=np.int64), K=50, N=8)
    assert np.array_equal(run_gpu(p), np.zeros((1000, 8), dtype=np.float32))
    # M == 0 and N == 0 are no-ops that succeed
    e = torch.zeros(1, dtype=torch.int32, device="cuda")
    f = torch.zeros(0, dtype=torch.float32, device="cuda")
    sdl.spmm_csr_f32(e, e[:0], f, torch.zeros(4, device="cuda"), f, 0, 2, 2)
    p = W.rows_with_lengths([1, 2], K=5, N=0)
    rowptr, colind, vals, B = dev_arrays(p)
    sdl.spmm_csr_f32(rowptr, colind, vals, B, f, 2, 5, 0)
    # a single dense row (every column once) and a single row overall
    p = W.rows_with_lengths([4096], K=4096, N=64, seed=2)
    Cref, Sref = reference(p)
    assert_parity(run_gpu(p), Cref, Sref, "f32", "dense row")
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identity_bitwise(dtype):
    """A = I: C equals B exactly (bf16: B widened exactly)."""
    M, N = 3000, 128
    rng = np.random.default_rng(1)
    B32 = rng.standard_normal((M, N)).astype(np.float32)
    ones = np.ones(M, dtype=np.float32)
    if dtype == "bf16":
        B = W.f32_to_bf16_bits(B32)
        v = W.f32_to_bf16_bits(ones)
        expect = oracle.widen_bf16(B).astype(np.float32)
    else:
        B, v, expect = B32, ones, B32
    p = W.CsrProblem("identity", M, M, N, np.arange(M + 1, dtype=np.int32),
                     np.arange(M, dtype=np.int32), v, B, dtype)
    assert np.array_equal(run_gpu(p), expect)


def test_scaling_and_repeatability_bitwise():
    """Rows computed inside one wavefront (no atomics): two runs agree to the
    bit, and doubling every value doubles C exactly."""
    p = edge_problem(64, "f32", M=400, seed=9)
    t = sdl.resolve_tuning(0, 64)
    det = np.diff(p.rowptr) <= t.medium_max
    C1 = run_gpu(p)
    C2 = run_gpu(p)
    assert np.array_equal(C1[det], C2[det])
    q = W.CsrProblem(p.name, p.M, p.K, p.N, p.rowptr, p.colind, p.vals * 2, p.B, "f32")
    Cq = run_gpu(q)
    assert np.array_equal(Cq[det], 2 * C1[det])
    Cn = run_gpu(W.CsrProblem(p.name, p.M, p.K, p.N, p.rowptr, p.colind, -p.vals, p.B, "f32"))
    assert np.array_equal(Cn[det], -C1[det])


def test_nonneg_equals_bound():
    """Non-negative inputs: C equals the bound S (up to fp32 rounding)."""
    p = edge_problem(32, "f32", M=200, seed=4)
    p = W.CsrProblem(p.name, p.M, p.K, p.N, p.rowptr, p.colind, np.abs(p.vals),
                     np.abs(p.B), "f32")
    C = run_gpu(p)
    _, Sref = reference(p)
    assert np.all(np.abs(C - Sref) <= 1e-5 * Sref + 1e-6)


def _with_vals(p, vals):
    return W.CsrProblem(p.name, p.M, p.K, p.N, p.rowptr, p.colind,
                        np.ascontiguousarray(vals), p.B, p.dtype)


def _single_wave_rows(p):
    """Rows computed by one wavefront (not split into chunks): their results
    do not depend on the order of atomic adds."""
    t = sdl.resolve_tuning(0 if p.dtype == "f32" else 1, p.N)
    return np.diff(p.rowptr.astype(np.int64)) <= t.medium_max


@pytest.mark.parametrize("N", [4, 64, 256])
def test_row_locality_bitwise(N):
    """Changing the values of some rows leaves every other row bit for bit
    unchanged (rows are independent; no state leaks between work items)."""
    p = edge_problem(N, "f32", M=400, seed=6)
    C1 = run_gpu(p)
    rng = np.random.default_rng(1)
    changed = rng.random(p.M) < 0.3
    mask = np.repeat(changed, np.diff(p.rowptr.astype(np.int64)))
    v2 = p.vals.copy()
    v2[mask] = rng.uniform(-1, 1, mask.sum()).astype(np.float32)
    C2 = run_gpu(_with_vals(p, v2))
    keep = ~changed & _single_wave_rows(p)
    assert keep.sum() > 100
    assert np.array_equal(C1[keep], C2[keep])
    Cref, Sref = reference(_with_vals(p, v2))
    assert_parity(C2, Cref, Sref, "f32", "changed rows")


def test_additivity():
    """C(v1 + v2) = C(v1) + C(v2) within the sum of the bounds."""
    p = edge_problem(64, "f32", M=300, seed=7)
    rng = np.random.default_rng(2)
    v1 = p.vals
    v2 = rng.uniform(-1, 1, p.vals.shape[0]).astype(np.float32)
    v12 = (v1.astype(np.float64) + v2).astype(np.float32)
    C1, C2, C12 = (run_gpu(_with_vals(p, v)) for v in (v1, v2, v12))
    _, S1 = reference(_with_vals(p, v1))
    _, S2 = reference(_with_vals(p, v2))
    _, S12 = reference(_with_vals(p, v12))
    err = np.abs(C12.astype(np.float64) - C1 - C2)
    # rounding v1 + v2 to fp32 moves each product by at most 2^-24 of it
    lim = 1e-5 * (S1 + S2 + S12) + 2.0 ** -24 * S12 + 3e-6
    assert np.all(err <= lim)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_permuted_entries_within_bound(dtype):
    """Shuffling the stored entries inside each row (unsorted colind) gives
    the same product within the bound."""
    p = edge_problem(64, dtype, M=300, seed=8)
    rng = np.random.default_rng(3)
    rp = p.rowptr.astype(np.int64)
    perm = np.arange(p.nnz)
    for i in range(p.M):
        seg = perm[rp[i]:rp[i + 1]]
        rng.shuffle(seg)
    q = W.CsrProblem(p.name, p.M, p.K, p.N, p.rowptr,
                     np.ascontiguousarray(p.colind[perm]),
                     np.ascontiguousarray(p.vals[perm]), p.B, p.dtype)
    Cref, Sref = reference(p)
    assert_parity(run_gpu(q), Cref, Sref, dtype, "permuted")


# ------------------------------------------------------------------ plan

PLAN_CASES = [
    ("edge-defaults", lambda: edge_problem(64, "f32", M=3000, seed=1), None),
    ("edge-tiny", lambda: edge_problem(64, "f32", M=3000, seed=2), sdl.Tuning(1, 4, 3)),
    ("edge-everything-long", lambda: edge_problem(8, "f32", M=500, seed=3), sdl.Tuning(0, 0, 5)),
    ("powerlaw-64k", lambda: W.powerlaw_rows(M=65536, N=64), None),
    ("skew-60k", lambda: W.skew_rows(M=60000, N=512, hub_lo=2000, hub_hi=30000), None),
]


def _lengths_rowptr(M, seed, dmax=8192, alpha=2.1, base=0):
    """rowptr only, power-law row lengths (the plan reads nothing else)."""
    rng = np.random.default_rng(seed)
    d = np.arange(1, dmax + 1, dtype=np.float64)
    cdf = np.cumsum(d ** -alpha)
    lens = np.searchsorted(cdf / cdf[-1], rng.random(M)) + 1
    lens[rng.random(M) < 0.05] = 0
    return np.concatenate([[base], base + np.cumsum(lens)]).astype(np.int32)


# M chosen so that plan tiles hold one round (262144), several rounds with
# a ragged tail (600001), and a last plan block with a single tile (262145).
PLAN_ROWPTR_CASES = [(262144, 0, None), (600001, 7, None), (262145, 0, sdl.Tuning(4, 40, 17))]


@pytest.mark.parametrize("M,base,tuning", PLAN_ROWPTR_CASES,
                         ids=[f"M{c[0]}" for c in PLAN_ROWPTR_CASES])
def test_plan_bit_exact_many_blocks(M, base, tuning):
    rp = _lengths_rowptr(M, seed=M % 97, base=base)
    t = sdl.resolve_tuning(0, 64, tuning)
    got = sdl.plan_export(torch.from_numpy(rp).cuda(), t)
    want = oracle.plan_ref(rp, t.short_max, t.medium_max, t.chunk_nnz)
    for k in ("n_short", "n_medium", "n_long", "n_chunks"):
        assert got[k] == want[k], k
    assert np.array_equal(got["medium_rows"], want["medium_rows"])
    assert np.array_equal(got["long_rows"], want["long_rows"])
    assert np.array_equal(got["chunks"], want["chunks"])


@pytest.mark.parametrize("name,make,tuning", PLAN_CASES, ids=[c[0] for c in PLAN_CASES])
def test_plan_bit_exact(name, make, tuning):
    compare_plan(make(), tuning)


def test_plan_bit_exact_offset_rowptr():
    """rowptr[0] != 0 and a chunk count beyond the chunk table."""
    p = W.rows_with_lengths([9000, 0, 12000, 3, 7000], K=20000, N=32, seed=3)
    rp = np.concatenate([[5], 5 + p.rowptr[1:]]).astype(np.int32)
    t = sdl.Tuning(2, 8, 3, hub_min=2 ** 31 - 1, slab_rows=1)   # resolved, no hubs
    got = sdl.plan_export(torch.from_numpy(rp).cuda(), t)
    want = oracle.plan_ref(rp, 2, 8, 3)
    assert got["n_chunks"] == want["n_chunks"] > 4096 + 5
    assert np.array_equal(got["chunks"], want["chunks"])
    assert np.array_equal(got["long_rows"], want["long_rows"])


def test_plan_bit_exact_offset_rowptr_hubs():
    """rowptr[0] != 0 with a hub row between two long rows: hub chunk bounds
    are absolute positions too."""
    p = W.rows_with_lengths([9000, 0, 12000, 3, 7000], K=20000, N=32, seed=4)
    rp = np.concatenate([[5], 5 + p.rowptr[1:]]).astype(np.int32)
    ci = np.concatenate([np.zeros(5, np.int32), p.colind]).astype(np.int32)
    t = sdl.Tuning(2, 8, 300, hub_min=10000, slab_rows=1000)
    got = sdl.plan_export(torch.from_numpy(rp).cuda(), t, colind=torch.from_numpy(ci).cuda(),
                          K=p.K)
    want = oracle.plan_ref(rp, 2, 8, 300, hub_min=10000, slab_rows=1000, K=p.K, colind=ci)
    assert got["n_hub"] == want["n_hub"] == 1 and got["n_long"] == 2
    for k in ("long_rows", "chunks", "hub_rows", "hub_chunks"):
        assert np.array_equal(got[k], want[k]), k


# ------------------------------------------------- scaled-down workloads

SCALED = [
    ("uniform", lambda: W.uniform_rows(M=4096, K=4096, N=32)),
    ("powerlaw", lambda: W.powerlaw_rows(M=32768, N=64)),
    ("pruned-bf16", lambda: W.bernoulli_rows(M=1024, K=2048, N=256, dtype="bf16")),
    ("pruned-f32", lambda: W.bernoulli_rows(M=1024, K=2048, N=256, dtype="f32")),
    ("banded", lambda: W.banded_rows(M=65536, N=128, half_width=4096)),
    ("skew", lambda: W.skew_rows(M=65536, N=512, hub_lo=2000, hub_hi=20000)),
]


@pytest.mark.parametrize("name,make", SCALED, ids=[s[0] for s in SCALED])
def test_scaled_workloads(name, make):
    p = make()
    C = run_gpu(p)
    Cref, Sref = reference(p)
    assert_parity(C, Cref, Sref, p.dtype, name)


@pytest.mark.parametrize("N", [1, 2, 4, 6, 8, 12, 16])
def test_small_n_powerlaw(N):
    """Small N (groups of 1 or 2 lanes, 64 or 32 rows per wavefront) on a
    scaled power-law pattern, every element."""
    p = W.powerlaw_rows(M=32768, N=N, seed=40 + N)
    Cref, Sref = reference(p)
    assert_parity(run_gpu(p), Cref, Sref, "f32", f"N={N}")


def test_small_job_many_rows():
    """A call that gathers only a few MB but has many rows: workgroups past
    the first 64 product workgroups leave at once, and the rest (with the
    plan's) must still cover every short tile, medium row and chunk."""
    rng = np.random.default_rng(51)
    M = 300000
    lens = np.zeros(M, dtype=np.int64)
    busy = rng.choice(M, 3000, replace=False)
    lens[busy] = rng.choice([1, 3, 17, 40, 100], size=busy.size)
    lens[busy[:4]] = 900                       # long rows: chunks
    p = W.rows_with_lengths(lens, K=1000, N=16, seed=52)
    assert p.nnz * p.N * 4 < (16 << 20)
    C = run_gpu(p)
    Cref, Sref = reference(p)
    assert_parity(C, Cref, Sref, "f32", "small job, many rows")
