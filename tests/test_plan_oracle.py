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


def test_plan_rejects_bad_thresholds():
    with pytest.raises(ValueError):
        oracle.plan_ref(np.array([0, 1]), 5, 4, 3)
    with pytest.raises(ValueError):
        oracle.plan_ref(np.array([0, 1]), 1, 4, 0)
