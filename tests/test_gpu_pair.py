"""The PAIR form of the product: with B larger than the Infinity Cache and
rows of B of 512 bytes (fp32 N = 128, bf16 N = 256), medium rows are taken
four at a time (one 16-lane group each), one column half per item, each
half on its own four XCDs.  These cases use such a B (600,000 rows,
307 MB) with few rows of A, so the oracle stays quick: 1, 2, 3 and 5
medium rows (items with fewer than four rows), rows of very different
lengths in one item, medium rows between short, long and hub rows (items
of rows that are not neighbours), empty rows, columns in any order, a
row-block view, and a banded matrix (the case the form is for).  Every
element against the oracle, C NaN-filled, fault count read."""
import numpy as np
import pytest
import torch

import oracle
import sparse_dense_linear_amd as sdl
import workloads as W
from gpu_helpers import assert_parity, compare_plan, dev_arrays, reference, run_gpu

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

K_BIG = 600_000
WIDTH = {"f32": 128, "bf16": 256}


def mixed(dtype, seed, M=3001, shuffle=False):
    rng = np.random.default_rng(seed)
    lengths = rng.choice([0, 1, 5, 17, 33, 64, 100, 200, 500, 3000], size=M,
                         p=[.05, .1, .1, .2, .15, .15, .1, .1, .04, .01])
    p = W.rows_with_lengths(lengths, K_BIG, WIDTH[dtype], seed=seed, dtype=dtype)
    if shuffle:
        for i in range(M):
            s, e = int(p.rowptr[i]), int(p.rowptr[i + 1])
            rng.shuffle(p.colind[s:e])
    return p


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_pair_form_mixed_rows(dtype):
    p = mixed(dtype, seed=81 if dtype == "f32" else 82)
    t = sdl.resolve_tuning(sdl.DTYPE_F32 if dtype == "f32" else sdl.DTYPE_BF16, p.N, K=p.K)
    assert compare_plan(p)["n_medium"] > 2
    Cref, Sref = reference(p)
    assert_parity(run_gpu(p), Cref, Sref, dtype, f"pair {dtype} defaults {t}")
    # every non-empty row medium, then medium rows between long and hub rows
    for tuning in (sdl.Tuning(0, 4096, 512), sdl.Tuning(16, 40, 50, hub_min=300,
                                                      slab_rows=70000)):
        assert_parity(run_gpu(p, tuning=tuning), Cref, Sref, dtype, f"pair {dtype} {tuning}")


def test_pair_form_odd_and_shuffled():
    """Columns in no order within rows, and 1, 2, 3 or 5 medium rows (items
    with fewer than four rows)."""
    p = mixed("f32", seed=83, M=1500, shuffle=True)
    Cref, Sref = reference(p)
    assert_parity(run_gpu(p), Cref, Sref, "f32", "pair shuffled")
    for n_medium in (1, 2, 3, 5):
        lengths = np.zeros(40, np.int64)
        lengths[[7, 8, 20, 21, 33][:n_medium]] = [50, 300, 90, 41, 200][:n_medium]
        q = W.rows_with_lengths(lengths, K_BIG, 128, seed=84 + n_medium)
        assert compare_plan(q)["n_medium"] == n_medium
        Cref, Sref = reference(q)
        assert_parity(run_gpu(q), Cref, Sref, "f32", f"{n_medium} medium rows")


def test_pair_form_banded_view():
    """A banded matrix over the large B, whole and as a block of rows."""
    p = W.banded_rows(M=K_BIG, N=128, half_width=4096, seed=85)
    rows = np.random.default_rng(85).choice(p.M, 4096, replace=False)
    rows = np.unique(np.concatenate([rows, [0, 1, p.M - 2, p.M - 1]]))
    Cref, Sref = reference(p, rows=rows)
    got = run_gpu(p)
    assert_parity(got[rows], Cref, Sref, "f32", "pair banded")
    r0, r1 = 12345, 20001                 # an odd number of rows, rowptr[0] != 0
    rowptr, colind, vals, B = dev_arrays(p)
    C = torch.full((p.M * p.N,), float("nan"), dtype=torch.float32, device="cuda")
    sdl.spmm_csr_f32(rowptr[r0:r1 + 1], colind, vals, B, C[r0 * p.N:r1 * p.N], r1 - r0,
                     p.K, p.N)
    torch.cuda.synchronize()
    assert sdl.stream_faults() == 0
    sub = np.arange(r0, r1)
    Cref, Sref = reference(p, rows=sub)
    assert_parity(C.cpu().numpy().reshape(p.M, p.N)[r0:r1], Cref, Sref, "f32",
                  "pair banded view")


@pytest.mark.parametrize("seed", range(6))
def test_pair_form_random(seed):
    """Seeded random cases of the form: M from 1 to 2500, medium rows of
    any length in any share (items of rows of very different lengths, a
    last item of one to four rows), short, long and empty rows among them,
    both element types, default or random thresholds."""
    rng = np.random.default_rng(700 + seed)
    dtype = "bf16" if seed % 2 else "f32"
    M = int(rng.integers(1, 2500))
    lengths = rng.choice([0, 3, 17, 40, 130, 512, 900], size=M,
                         p=[.05, .15, .3, .2, .2, .05, .05])
    p = W.rows_with_lengths(lengths, K_BIG, WIDTH[dtype], seed=700 + seed, dtype=dtype)
    tuning = None
    if seed >= 3:
        short_max = int(rng.choice([0, 4, 16]))
        tuning = sdl.Tuning(short_max, short_max + int(rng.choice([30, 200, 1000])),
                            int(rng.choice([64, 512])))
    plan = compare_plan(p, tuning)
    Cref, Sref = reference(p)
    what = f"seed={seed} M={M} {dtype} tuning={tuning} medium={plan['n_medium']}"
    assert_parity(run_gpu(p, tuning=tuning), Cref, Sref, dtype, what)
