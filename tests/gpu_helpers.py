"""Shared helpers of the GPU parity tests: upload a problem, run the HIP
library through the binding, compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import sparse_dense_linear_amd as sdl

#: Per-element bound |C_gpu - C_ref| <= TOL * S + 1e-6 (S = |A||B|): the
#: stated tolerance for fp32 inputs, and "1e-2 relative on the same bound"
#: for bf16 inputs with fp32 accumulation.
TOL = {"f32": 1e-5, "bf16": 1e-2}
ABS = 1e-6
#: bf16 inputs are widened exactly to fp32 and accumulated in fp32, so the
#: fp32 bound holds for them as well; asserting it too is what tells fp32
#: accumulation from a bf16 accumulator (relative error about 2^-8), which
#: the 1e-2 bound alone would let pass.
ACC_TOL = 1e-5


def dev_arrays(p, device="cuda"):
    rowptr = torch.from_numpy(p.rowptr).to(device)
    colind = torch.from_numpy(p.colind).to(device)
    if p.dtype == "f32":
        vals = torch.from_numpy(p.vals).to(device)
        B = torch.from_numpy(np.ascontiguousarray(p.B).reshape(-1)).to(device)
    else:
        vals = torch.from_numpy(p.vals.view(np.int16)).to(device)
        B = torch.from_numpy(np.ascontiguousarray(p.B).reshape(-1).view(np.int16)).to(device)
    return rowptr, colind, vals, B


def call(p, rowptr, colind, vals, B, C, M=None, tuning=None):
    M = p.M if M is None else M
    if tuning is not None:
        dt = sdl.DTYPE_F32 if p.dtype == "f32" else sdl.DTYPE_BF16
        sdl.spmm_csr_tuned(dt, rowptr, colind, vals, B, C, M, p.K, p.N, tuning)
    elif p.dtype == "f32":
        sdl.spmm_csr_f32(rowptr, colind, vals, B, C, M, p.K, p.N)
    else:
        sdl.spmm_csr_bf16in_f32acc(rowptr, colind, vals, B, C, M, p.K, p.N)


def run_gpu(p, tuning=None, fill=float("nan")):
    """C from the HIP library; C starts filled with `fill` (NaN by default),
    so any element the library fails to write is caught."""
    rowptr, colind, vals, B = dev_arrays(p)
    C = torch.full((p.M * p.N,), fill, dtype=torch.float32, device="cuda")
    call(p, rowptr, colind, vals, B, C, tuning=tuning)
    torch.cuda.synchronize()
    assert sdl.stream_faults() == 0, "a product wavefront gave up waiting for the plan"
    return C.cpu().numpy().reshape(p.M, p.N)


def reference(p, rows=None):
    return oracle.spmm_ref(p.rowptr, p.colind, p.vals, p.B, p.N, rows=rows)


def assert_parity(C, Cref, Sref, dtype, what=""):
    C = np.asarray(C, dtype=np.float64)
    err = np.abs(C - Cref)
    tols = [TOL[dtype]] + ([ACC_TOL] if dtype == "bf16" else [])
    for tol in tols:
        lim = tol * Sref + ABS
        bad = ~(err <= lim)          # NaN counts as a failure
        if bad.any():
            idx = np.argwhere(bad)
            i, n = idx[0]
            raise AssertionError(
                f"{what}: {int(bad.sum())} of {bad.size} elements outside the "
                f"bound {tol:g}*S + {ABS:g}; first at ({i},{n}): gpu={C[i, n]!r} "
                f"ref={Cref[i, n]!r} S={Sref[i, n]!r}")
    return float((err / np.maximum(Sref, 1e-30)).max()) if err.size else 0.0


def compare_plan(p, tuning=None):
    """The plan of problem p as the product call resolves it (its K, N and
    tuning) exported from the device, against the plan oracle: bit-exact
    lists, chunks, hub rows and hub chunks (the columns of p's rows ascend).
    Returns the device plan."""
    dt = sdl.DTYPE_F32 if p.dtype == "f32" else sdl.DTYPE_BF16
    t = sdl.resolve_tuning(dt, p.N, tuning, K=p.K)
    got = sdl.plan_export(torch.from_numpy(p.rowptr).cuda(), t,
                          colind=torch.from_numpy(p.colind).cuda(), K=p.K)
    want = oracle.plan_ref(p.rowptr, t.short_max, t.medium_max, t.chunk_nnz,
                           hub_min=t.hub_min, slab_rows=t.slab_rows, K=p.K,
                           colind=p.colind)
    for k in ("n_short", "n_medium", "n_long", "n_chunks", "n_hub"):
        assert got[k] == want[k], k
    assert got["n_hub_chunks"] == want["hub_chunks"].shape[0]
    assert np.array_equal(got["medium_rows"], want["medium_rows"])
    assert np.array_equal(got["long_rows"], want["long_rows"])
    assert np.array_equal(got["chunks"], want["chunks"])
    assert np.array_equal(got["hub_rows"], want["hub_rows"])
    assert np.array_equal(got["hub_chunks"], want["hub_chunks"])
    return got
