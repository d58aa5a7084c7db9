"""Seeded generators: structure, statistics and reproducibility (CPU only).
Small instances of every generator; the full sizes are built on the GPU machine
by the benchmark and the full-size tests."""
import numpy as np
import pytest
import torch

import workloads as W


def check_csr(p):
    rp = p.rowptr.astype(np.int64)
    assert p.rowptr.dtype == np.int32 and p.colind.dtype == np.int32
    assert rp[0] == 0 and np.all(np.diff(rp) >= 0) and rp[-1] == p.colind.shape[0]
    assert p.vals.shape[0] == p.colind.shape[0]
    assert p.B.shape == (p.K, p.N)
    assert np.all(p.colind >= 0) and np.all(p.colind < p.K)
    # columns distinct and ascending within each row
    d = np.diff(p.colind.astype(np.int64))
    row_starts = rp[1:-1]
    inner = np.ones(d.shape[0], dtype=bool)
    inner[row_starts[(row_starts > 0) & (row_starts <= d.shape[0])] - 1] = False
    assert np.all(d[inner] > 0)


def test_uniform():
    p = W.uniform_rows(M=512, K=300, N=8, per_row=16)
    check_csr(p)
    assert np.all(p.lengths() == 16)
    assert p.vals.dtype == np.float32 and np.all(np.abs(p.vals) < 1)


def test_powerlaw_law():
    p = W.powerlaw_rows(M=200000, K=20000, N=4)
    check_csr(p)
    L = p.lengths()
    assert L.min() >= 1 and L.max() <= 8192
    d = np.arange(1, 8193, dtype=np.float64)
    pmf = d ** -2.1 / (d ** -2.1).sum()
    # P(d = 1), P(d = 2) and the mean against the exact law (5 sigma)
    for k in (1, 2):
        se = np.sqrt(pmf[k - 1] * (1 - pmf[k - 1]) / L.shape[0])
        assert abs((L == k).mean() - pmf[k - 1]) < 5 * se
    mean = (d * pmf).sum()
    assert abs(mean - 4.18) < 0.01
    assert abs(L.mean() - mean) < 0.2
    assert np.all(p.vals >= 0) and np.all(p.vals < 1)


def test_bernoulli():
    p = W.bernoulli_rows(M=512, K=512, N=8, dtype="f32")
    check_csr(p)
    frac = p.nnz / (512 * 512)
    assert abs(frac - 0.1) < 5 * np.sqrt(0.1 * 0.9 / 512 ** 2)
    assert abs(p.vals.std() - 0.02) < 0.002
    q = W.bernoulli_rows(M=512, K=512, N=8, dtype="bf16")
    assert np.array_equal(q.colind, p.colind)
    assert np.array_equal(q.vals, W.f32_to_bf16_bits(p.vals))
    assert np.array_equal(q.B, W.f32_to_bf16_bits(p.B))


def test_banded():
    p = W.banded_rows(M=20000, N=4, half_width=512)
    check_csr(p)
    assert np.all(p.lengths() == 32)
    rows = np.repeat(np.arange(p.M), 32)
    in_band = np.abs(p.colind.astype(np.int64) - rows) <= 512
    # exactly 24 band draws per row; uniform draws land in the band rarely
    per_row = in_band.reshape(p.M, 32).sum(axis=1)
    assert np.all(per_row >= 24)
    # expected share: 24/32 plus the 8 uniform draws landing in the band
    i = np.arange(p.M)
    width = np.minimum(p.K, i + 513) - np.maximum(0, i - 512)
    expect = (24 + 8 * (width / p.K).mean()) / 32
    assert abs(in_band.mean() - expect) < 0.002


def test_skew():
    p = W.skew_rows(M=50000, N=4, hub_lo=2000, hub_hi=20000)
    check_csr(p)
    L = p.lengths()
    hubs = p.meta["hubs"]
    assert hubs.shape[0] == 50
    assert np.all((L[hubs] >= 2000) & (L[hubs] <= 20000))
    other = np.ones(p.M, dtype=bool)
    other[hubs] = False
    assert L[other].min() == 1 and L[other].max() == 8
    assert p.dtype == "bf16" and p.vals.dtype == np.uint16


def test_seed_reproducible():
    a = W.powerlaw_rows(M=5000, N=4, seed=9)
    b = W.powerlaw_rows(M=5000, N=4, seed=9)
    c = W.powerlaw_rows(M=5000, N=4, seed=10)
    assert np.array_equal(a.colind, b.colind) and np.array_equal(a.B, b.B)
    assert not np.array_equal(a.rowptr, c.rowptr)


def test_bf16_rounding_matches_torch():
    """Round-to-nearest-even against torch's float32 -> bfloat16 cast."""
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8,
                                  0.0, -0.0, 3.0e38], dtype=np.float32)])
    ours = W.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_registry_names():
    assert set(W.WORKLOADS) == {"uniform_1k_n32", "powerlaw_262k_n64",
                                "powerlaw_262k_n64_mean16",
                                "pruned_4k_n256_bf16", "pruned_4k_n256_f32",
                                "banded_4m_n128", "skew_1m_n512_bf16"}
    p = W.make("uniform_1k_n32")
    assert (p.M, p.K, p.N, p.nnz) == (1024, 1024, 32, 16384)


def test_powerlaw_mean16_exponent():
    """The secondary power-law case: exponent 1.7694 on {1..8192} has mean
    row length 16 (the law's mean, computed exactly)."""
    d = np.arange(1, 8193, dtype=np.float64)
    w = d ** -1.7694
    assert abs((d * w).sum() / w.sum() - 16.0) < 0.01
