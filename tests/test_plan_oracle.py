"""The row-plan oracle (oracle.plan_ref) against a hand-derived example and
against the invariants that define a plan (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_plan_golden_example():
    with open(os.path.join(GOLDEN, "plan_example.json")) as f:
        g = json.load(f)
    p = oracle.plan_ref(np.array(g["rowptr"]), g["short_max"], g["medium_max"],
                        g["chunk_nnz"])
    assert p["n_short"] == g["n_short"]
    assert p["medium_rows"].tolist() == g["medium_rows"]
    assert p["long_rows"].tolist() == g["long_rows"]
    assert p["chunks"].tolist() == g["chunks"]
    assert p["n_chunks"] == len(g["chunks"]) and p["n_long"] == len(g["long_rows"])


def check_plan_invariants(rowptr, short_max, medium_max, chunk, p):
    """What any correct plan satisfies, stated without its formula."""
    rp = np.asarray(rowptr, dtype=np.int64)
    lens = np.diff(rp)
    M = lens.shape[0]
    # the three bins partition the rows, by length
    assert p["n_short"] + p["n_medium"] + p["n_long"] == M
    med = p["medium_rows"]
    assert np.all(np.diff(med) > 0)
    assert np.all((lens[med] > short_max) & (lens[med] <= medium_max))
    lr = p["long_rows"]
    assert np.all(np.diff(lr[:, 0]) > 0) if len(lr) else True
    assert np.all(lens[lr[:, 0]] > medium_max) if len(lr) else True
    assert p["n_short"] == int((lens <= short_max).sum())
    assert p["n_medium"] == int(((lens > short_max) & (lens <= medium_max)).sum())
    # chunks tile every long row exactly, in order, each non-empty and at
    # most `chunk` entries, sizes within one of each other, and as few as
    # the size limit allows
    ch = p["chunks"]
    assert p["n_chunks"] == ch.shape[0]
    pos = 0
    for li, (row, first, n) in enumerate(lr):
        assert first == pos
        assert n == -(-lens[row] // chunk)
        cs = ch[first:first + n]
        assert np.all(cs[:, 0] == row) and np.all(cs[:, 3] == li)
        assert cs[0, 1] == rp[row] and cs[-1, 2] == rp[row + 1]
        assert np.all(cs[1:, 1] == cs[:-1, 2])
        sizes = cs[:, 2] - cs[:, 1]
        assert np.all(sizes >= 1) and np.all(sizes <= chunk)
        assert sizes.max() - sizes.min() <= 1
        pos += n
    assert pos == p["n_chunks"]


@pytest.mark.parametrize("seed", range(6))
def test_plan_invariants_random(seed):
    rng = np.random.default_rng(seed)
    M = int(rng.integers(1, 400))
    lens = rng.choice([0, 1, 2, 5, 31, 32, 33, 64, 255, 256, 257, 1000, 5000], size=M)
    rowptr = np.concatenate([[7], 7 + np.cumsum(lens)])   # rowptr[0] != 0
    short_max, medium_max, chunk = [(32, 256, 256), (0, 0, 1), (5, 300, 97),
                                    (16, 16, 8), (1000, 1000, 4096), (2, 64, 3)][seed]
    p = oracle.plan_ref(rowptr, short_max, medium_max, chunk)
    check_plan_invariants(rowptr, short_max, medium_max, chunk, p)


def test_plan_hub_golden_example():
    """Hand-derived plan with a long row at the hub threshold, two hub rows,
    a column exactly at a slab boundary and an empty hub chunk."""
    with open(os.path.join(GOLDEN, "plan_hub_example.json")) as f:
        g = json.load(f)
    p = oracle.plan_ref(np.array(g["rowptr"]), g["short_max"], g["medium_max"],
                        g["chunk_nnz"], hub_min=g["hub_min"], slab_rows=g["slab_rows"],
                        K=g["K"], colind=np.array(g["colind"]))
    assert p["n_short"] == g["n_short"]
    assert p["medium_rows"].tolist() == g["medium_rows"]
    assert p["long_rows"].tolist() == g["long_rows"]
    assert p["chunks"].tolist() == g["chunks"]
    assert p["hub_rows"].tolist() == g["hub_rows"]
    assert p["n_slabs"] == g["n_slabs"]
    assert p["hub_chunks"].tolist() == g["hub_chunks"]
    assert p["n_hub"] == len(g["hub_rows"])


def check_hub_invariants(rowptr, colind, medium_max, hub_min, slab_rows, K, p):
    """Hub rows and their chunks, stated without the plan's formula: the hub
    rows are exactly the rows above the threshold; for each, the chunks
    of slab s (found at index s * n_hub + h) tile the row in slab order,
    and (columns ascending) hold exactly the entries whose column is in
    slab s."""
    rp = np.asarray(rowptr, dtype=np.int64)
    lens = np.diff(rp)
    top = max(hub_min, medium_max)
    hubs = p["hub_rows"]
    assert hubs.tolist() == np.nonzero(lens > top)[0].tolist()
    n_slabs = p["n_slabs"]
    assert n_slabs * slab_rows >= K > (n_slabs - 1) * slab_rows
    hc = p["hub_chunks"]
    assert hc.shape == (hubs.size * n_slabs, 4)
    for h, row in enumerate(hubs):
        mine = hc[np.arange(n_slabs) * hubs.size + h]
        assert np.all(mine[:, 0] == row) and np.all(mine[:, 3] == h)
        assert mine[0, 1] == rp[row] and mine[-1, 2] == rp[row + 1]
        assert np.all(mine[1:, 1] == mine[:-1, 2])
        for s, (_, p0, p1, _) in enumerate(mine):
            cols = np.asarray(colind[p0:p1])
            assert np.all((cols >= s * slab_rows) & (cols < (s + 1) * slab_rows))
        # long and medium bins leave the hub rows out
    assert p["n_short"] + p["n_medium"] + p["n_long"] + p["n_hub"] == lens.size


@pytest.mark.parametrize("seed", range(5))
def test_plan_hub_invariants_random(seed):
    rng = np.random.default_rng(100 + seed)
    K = int(rng.integers(1, 3000))
    M = int(rng.integers(1, 200))
    lens = rng.choice([0, 1, 3, 40, 41, 100, 700, 2000], size=M)
    lens = np.minimum(lens, K)
    rowptr = np.concatenate([[3], 3 + np.cumsum(lens)])
    colind = np.concatenate([[0, 0, 0]] + [np.sort(rng.choice(K, int(n), replace=False))
                                           for n in lens]).astype(np.int32)
    short_max, medium_max, chunk, hub_min, slab = [(1, 40, 16, 40, 7), (3, 3, 2, 100, 1),
                                                   (0, 10, 5, 0, 1000), (2, 50, 9, 699, 64),
                                                   (1, 1, 1, 1, 3000)][seed]
    p = oracle.plan_ref(rowptr, short_max, medium_max, chunk, hub_min=hub_min,
                        slab_rows=slab, K=K, colind=colind)
    check_hub_invariants(rowptr, colind, medium_max, hub_min, slab, K, p)
    # the position chunks of the long rows are unchanged by the hub class
    lr = p["long_rows"]
    lens64 = np.diff(rowptr.astype(np.int64))
    assert np.all(lens64[lr[:, 0]] <= max(hub_min, medium_max)) if len(lr) else True


def test_plan_hub_brute_force_small():
    """Every (hub, slab) chunk of small random rows against a direct scan:
    the positions of the row whose column falls in the slab."""
    rng = np.random.default_rng(7)
    for _ in range(30):
        K = int(rng.integers(1, 60))
        slab = int(rng.integers(1, 20))
        lens = rng.integers(0, K + 1, size=int(rng.integers(1, 8)))
        rowptr = np.concatenate([[0], np.cumsum(lens)])
        colind = np.concatenate([np.sort(rng.choice(K, int(n), replace=False))
                                 for n in lens] + [np.zeros(0, np.int64)]).astype(np.int32)
        p = oracle.plan_ref(rowptr, 0, 0, 1, hub_min=0, slab_rows=slab, K=K, colind=colind)
        n_slabs = p["n_slabs"]
        for h, row in enumerate(p["hub_rows"]):
            for s in range(n_slabs):
                _, p0, p1, _ = p["hub_chunks"][s * p["n_hub"] + h]
                want = [q for q in range(rowptr[row], rowptr[row + 1])
                        if s * slab <= colind[q] < (s + 1) * slab]
                assert list(range(p0, p1)) == want


def test_plan_rejects_bad_thresholds():
    with pytest.raises(ValueError):
        oracle.plan_ref(np.array([0, 1]), 5, 4, 3)
    with pytest.raises(ValueError):
        oracle.plan_ref(np.array([0, 1]), 1, 4, 0)
    with pytest.raises(ValueError):   # hub rows need the slab width, K and colind
        oracle.plan_ref(np.array([0, 1]), 0, 0, 1, hub_min=0)
