"""GPU parity of the FusedMM entry point against the fp64 oracle.

Page: [IntelMax] "Performance Optimization of Deep Learning Sparse Matrix
Kernels on Intel Max Series GPU", the FusedMM operation (Fig. 6,
Algorithm 3).

Two routes: one launch that forms each value where it is used (fp32, N a
multiple of 4 up to 1024, operands 16-byte aligned, and N <= 64 or a mean
row of 32 entries or more), and otherwise SDDMM into a value array followed
by the product.  Both are checked here.

Bar: |E_gpu - E_ref| <= 2 tol(N) T + 1e-6 per element, with the bound
T[i,n] = sum_p S_p |D_jn| and tol(N) = max(1e-5, N 2^-23): each SDDMM value
is off by at most ~N 2^-24 S_p before it weights D_j (its rounding to fp32
adds 2^-24 |a_p|), and the sum over the row adds the product's own fp32
rounding, bounded the same way as the product's tests bound it.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import sparse_dense_linear_amd as sdl
import workloads as W

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def tol(N):
    return 2 * max(1e-5, N * 2.0 ** -23)


def _dev(x, shift=0):
    """x on the GPU; shift > 0 places it `shift` floats past a 16-byte
    boundary (a view into a larger buffer)."""
    flat = torch.from_numpy(np.ascontiguousarray(x).reshape(-1))
    if not shift:
        return flat.cuda()
    buf = torch.zeros(flat.numel() + shift, dtype=torch.float32, device="cuda")
    buf[shift:] = flat.cuda()
    return buf[shift:]


def run_fused(rowptr, colind, C, B, D, M, K, N, fill=float("nan"), shift=0):
    rp = torch.from_numpy(np.ascontiguousarray(rowptr, np.int32)).cuda()
    ci = torch.from_numpy(np.ascontiguousarray(colind, np.int32)).cuda()
    E = torch.full((M * N,), fill, dtype=torch.float32, device="cuda")
    nnz = int(rowptr[-1]) - int(rowptr[0])
    sdl.fusedmm_csr_f32(rp, ci, _dev(C, shift), _dev(B, shift), torch.from_numpy(D).cuda(),
                        E, M, K, N, nnz)
    torch.cuda.synchronize()
    assert sdl.stream_faults() == 0
    return E.cpu().numpy().reshape(M, N)


def check(rowptr, colind, C, B, D, M, K, N, what="", shift=0, margin=None):
    """E against the oracle within the bar; with `margin`, also the worst
    |E - Eref| / T over elements with T > 0 below margin * tol(N)."""
    E = run_fused(rowptr, colind, C, B, D, M, K, N, shift=shift)
    Eref, T = oracle.fusedmm_ref(rowptr, colind, C, B, D, N)
    err = np.abs(E.astype(np.float64) - Eref)
    bad = ~(err <= tol(N) * T + 1e-6)
    if bad.any():
        i, n = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {E.size} outside the bound; "
                             f"first ({i},{n}): gpu={E[i, n]!r} ref={Eref[i, n]!r} T={T[i, n]!r}")
    if margin is not None:
        live = T > 0
        worst = float((err[live] / T[live]).max()) if live.any() else 0.0
        assert worst <= margin * tol(N), f"{what}: worst err/T {worst:.3e}"
    return E


def pattern(lengths, K, seed):
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, np.int64)
    rowptr = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    colind = np.concatenate([np.sort(rng.choice(K, int(l), replace=False))
                             if l else np.zeros(0, np.int64) for l in lengths]).astype(np.int32)
    return rowptr, colind


def dense(rng, rows, N):
    return rng.uniform(-1, 1, (rows, N)).astype(np.float32)


def test_worked_example_bitwise():
    g = json.load(open(os.path.join(GOLDEN, "worked_example_fig3_fig6.json")))
    f = lambda k: np.array(g[k], np.float32)
    E = run_fused(np.array(g["rowptr"]), np.array(g["colind"]), f("C"), f("B"), f("D"),
                  g["M"], g["K"], g["N"])
    assert np.array_equal(E, f("E"))


EDGE = [0, 1, 2, 3, 9, 16, 17, 64, 200, 257, 1100, 3000]


@pytest.mark.parametrize("N", [1, 3, 4, 6, 8, 32, 64, 128, 256, 512, 1024, 1100])
def test_edge_rows(N):
    """Rows of every kind the product routes (empty, short, medium, long
    rows cut into chunks)."""
    rng = np.random.default_rng(N + 100)
    M, K = 200, 4000
    lengths = rng.choice(EDGE, size=M)
    lengths[:len(EDGE)] = EDGE
    rp, ci = pattern(lengths, K, seed=N)
    check(rp, ci, dense(rng, M, N), dense(rng, K, N), dense(rng, K, N), M, K, N, f"N={N}")


@pytest.mark.parametrize("N", [68, 96, 256, 512, 1024])
def test_wide_rows_of_few_entries(N):
    """N above 64 with a mean row of fewer than 32 entries takes the
    two-launch route (one launch pays only for long rows there); rows of
    every length class, against the oracle."""
    rng = np.random.default_rng(N + 300)
    M, K = 400, 3000
    lengths = rng.choice([0, 1, 2, 3, 9, 16, 17, 40], size=M)
    lengths[:3] = [300, 700, 0]          # a medium and a long row
    assert lengths.sum() < 32 * M
    rp, ci = pattern(lengths, K, seed=N + 300)
    check(rp, ci, dense(rng, M, N), dense(rng, K, N), dense(rng, K, N), M, K, N,
          f"N={N} few entries")


def test_two_launch_route_refuses_a_short_nnz():
    """nnz below rowptr[M] - rowptr[0] (a broken precondition) on the
    two-launch route: the SDDMM writes only nnz values, and the product,
    which would read the missing ones past the value array, is refused on
    the device and counted as a fault; the next call with the right nnz is
    exact."""
    rng = np.random.default_rng(71)
    M, K, N = 400, 3000, 128                   # N > 64, short rows: two launches
    lengths = rng.choice([0, 1, 2, 3, 9, 16, 17, 40], size=M)
    rp, ci = pattern(lengths, K, seed=71)
    stored = int(rp[-1])
    assert stored < 32 * M
    C, B, D = dense(rng, M, N), dense(rng, K, N), dense(rng, K, N)
    args = (torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda(), _dev(C), _dev(B),
            _dev(D))
    E = torch.full((M * N,), float("nan"), dtype=torch.float32, device="cuda")
    assert sdl.stream_faults() == 0
    sdl.fusedmm_csr_f32(*args, E, M, K, N, stored // 2)
    torch.cuda.synchronize()
    assert sdl.stream_faults() > 0
    check(rp, ci, C, B, D, M, K, N, "right nnz after a short one")


@pytest.mark.parametrize("N", [8, 64, 256])
def test_unaligned_operands(N):
    """C and B one float past a 16-byte boundary take the two-launch route
    (whose SDDMM then reads single elements, another summation order); both
    routes are held to the same bound."""
    rng = np.random.default_rng(N + 7)
    M, K = 300, 900
    rp, ci = pattern(rng.integers(0, 50, M), K, seed=N + 7)
    C, B, D = dense(rng, M, N), dense(rng, K, N), dense(rng, K, N)
    check(rp, ci, C, B, D, M, K, N, f"N={N} unaligned", shift=1)
    check(rp, ci, C, B, D, M, K, N, f"N={N} aligned")


def test_view_and_empty():
    rng = np.random.default_rng(3)
    M, K, N = 300, 700, 64
    lengths = rng.integers(0, 30, M)
    lengths[::7] = 0
    rp, ci = pattern(lengths, K, seed=3)
    C, B, D = dense(rng, M, N), dense(rng, K, N), dense(rng, K, N)
    E0 = check(rp, ci, C, B, D, M, K, N)
    assert np.array_equal(E0[lengths == 0], np.zeros(((lengths == 0).sum(), N), np.float32))
    pad = 5
    E1 = run_fused(rp + pad, np.concatenate([np.zeros(pad, np.int32), ci]), C, B, D, M, K, N)
    assert np.array_equal(E1[lengths <= 64], E0[lengths <= 64])


def test_no_entries():
    rng = np.random.default_rng(4)
    M, K, N = 50, 10, 16
    E = run_fused(np.zeros(M + 1, np.int32), np.zeros(0, np.int32), dense(rng, M, N),
                  dense(rng, K, N), dense(rng, K, N), M, K, N)
    assert np.array_equal(E, np.zeros((M, N), np.float32))


def test_equals_sddmm_then_spmm():
    """The one-launch call equals, bit for bit, SDDMM into an array followed
    by the product with those values, on rows that are not split: at N = 64
    both use 16-lane groups, so the fused worker forms each value in the
    SDDMM kernel's order and accumulates it as the product does."""
    rng = np.random.default_rng(5)
    M, K, N = 1500, 1200, 64
    rp, ci = pattern(rng.integers(0, 40, M), K, seed=5)
    C, B, D = dense(rng, M, N), dense(rng, K, N), dense(rng, K, N)
    E = run_fused(rp, ci, C, B, D, M, K, N)
    rpt, cit = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    A = torch.empty(ci.size, dtype=torch.float32, device="cuda")
    sdl.sddmm_csr_f32(rpt, cit, torch.from_numpy(C).cuda(), torch.from_numpy(B).cuda(),
                      A, M, K, N)
    E2 = torch.empty(M * N, dtype=torch.float32, device="cuda")
    sdl.spmm_csr_f32(rpt, cit, A, torch.from_numpy(D).cuda(), E2, M, K, N)
    torch.cuda.synchronize()
    single = np.diff(rp) <= sdl.resolve_tuning(0, N).medium_max
    assert np.array_equal(E[single], E2.cpu().numpy().reshape(M, N)[single])


def test_powerlaw_pattern():
    """FusedMM on the power-law workload's pattern (N = 64), every element."""
    p = W.make("powerlaw_262k_n64")
    rng = np.random.default_rng(6)
    C = rng.standard_normal((p.M, p.N)).astype(np.float32)
    D = rng.standard_normal((p.K, p.N)).astype(np.float32)
    # measured worst err/T: 1.1e-7 against the bar's 2e-5
    check(p.rowptr, p.colind, C, p.B.reshape(p.K, p.N), D, p.M, p.K, p.N, "powerlaw",
          margin=0.05)


# ---- bf16 inputs (one launch only) -------------------------------------

def bf16(x):
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even."""
    return W.f32_to_bf16_bits(np.ascontiguousarray(x, np.float32))


def widen(bits):
    """bf16 bit patterns -> the fp32 values they stand for (exact)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _dev16(bits, shift=0):
    flat = torch.from_numpy(np.ascontiguousarray(bits).reshape(-1).view(np.int16))
    if not shift:
        return flat.cuda()
    buf = torch.zeros(flat.numel() + shift, dtype=torch.int16, device="cuda")
    buf[shift:] = flat.cuda()
    return buf[shift:]


def run_fused_bf16(rowptr, colind, C, B, D, M, K, N, shift=0):
    rp = torch.from_numpy(np.ascontiguousarray(rowptr, np.int32)).cuda()
    ci = torch.from_numpy(np.ascontiguousarray(colind, np.int32)).cuda()
    E = torch.full((M * N,), float("nan"), dtype=torch.float32, device="cuda")
    nnz = int(rowptr[-1]) - int(rowptr[0])
    sdl.fusedmm_csr_bf16in_f32acc(rp, ci, _dev16(C, shift), _dev16(B, shift), _dev16(D),
                                  E, M, K, N, nnz)
    torch.cuda.synchronize()
    assert sdl.stream_faults() == 0
    return E.cpu().numpy().reshape(M, N)


def check_bf16(rowptr, colind, C, B, D, M, K, N, what="", shift=0):
    """C, B, D are bf16 bits; the oracle gets the values they stand for, so
    the fp32 bound applies unchanged (widening is exact)."""
    E = run_fused_bf16(rowptr, colind, C, B, D, M, K, N, shift=shift)
    Eref, T = oracle.fusedmm_ref(rowptr, colind, widen(C), widen(B), widen(D), N)
    bad = ~(np.abs(E.astype(np.float64) - Eref) <= tol(N) * T + 1e-6)
    if bad.any():
        i, n = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {E.size} outside the bound; "
                             f"first ({i},{n}): gpu={E[i, n]!r} ref={Eref[i, n]!r} T={T[i, n]!r}")
    return E


def test_bf16_worked_example_bitwise():
    """The worked example's values are exact in bf16 and every sum in it is
    exact.  Padded with zero columns to N = 8 (the bf16 form needs N a
    multiple of 8; zeros add nothing to a dot product), the bf16 call gives
    the golden E in the first columns and zeros in the rest, bit for bit."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example_fig3_fig6.json")))
    f = lambda k: np.array(g[k], np.float32)
    N0, N = g["N"], 8
    pad = lambda x: np.pad(x, ((0, 0), (0, N - N0)))
    C, B, D = (pad(f(k)) for k in ("C", "B", "D"))
    for x in (C, B, D):
        assert np.array_equal(widen(bf16(x)), x)
    E = run_fused_bf16(np.array(g["rowptr"]), np.array(g["colind"]), bf16(C),
                       bf16(B), bf16(D), g["M"], g["K"], N)
    assert np.array_equal(E[:, :N0], f("E"))
    assert np.array_equal(E[:, N0:], np.zeros((g["M"], N - N0), np.float32))


@pytest.mark.parametrize("N", [8, 16, 64, 128, 256, 512, 1024])
def test_bf16_edge_rows(N):
    rng = np.random.default_rng(N + 300)
    M, K = 200, 4000
    lengths = rng.choice(EDGE, size=M)
    lengths[:len(EDGE)] = EDGE
    rp, ci = pattern(lengths, K, seed=N + 300)
    check_bf16(rp, ci, bf16(dense(rng, M, N)), bf16(dense(rng, K, N)),
               bf16(dense(rng, K, N)), M, K, N, f"bf16 N={N}")


def test_bf16_powerlaw_pattern():
    p = W.make("powerlaw_262k_n64")
    rng = np.random.default_rng(16)
    C = bf16(rng.standard_normal((p.M, p.N)))
    B = bf16(p.B.reshape(p.K, p.N))
    D = bf16(rng.standard_normal((p.K, p.N)))
    check_bf16(p.rowptr, p.colind, C, B, D, p.M, p.K, p.N, "bf16 powerlaw")


def test_bf16_empty_and_widened_shapes():
    """nnz == 0 gives E = 0.  Shapes outside the one-launch form (N not a
    multiple of 8, N above 1024, C and B off 16-byte alignment) run on an
    exact fp32 copy of C, B and D: within the bound of the oracle, and, in
    the rows that are not split across wavefronts (split rows meet in fp32
    atomic adds, in no fixed order), bit for bit what fusedmm_csr_f32 gives
    on the widened values; a row view of the same rows gives the same."""
    rng = np.random.default_rng(17)
    M, K = 40, 30
    E = run_fused_bf16(np.zeros(M + 1, np.int32), np.zeros(0, np.int32),
                       bf16(dense(rng, M, 16)), bf16(dense(rng, K, 16)),
                       bf16(dense(rng, K, 16)), M, K, 16)
    assert np.array_equal(E, np.zeros((M, 16), np.float32))
    M, K = 200, 4000
    lengths = rng.choice(EDGE, size=M)
    lengths[:len(EDGE)] = EDGE
    rp, ci = pattern(lengths, K, seed=17)
    for N, shift in [(1, 0), (12, 0), (100, 0), (1032, 0), (64, 1), (13, 1)]:
        C, B, D = (bf16(dense(rng, r, N)) for r in (M, K, K))
        E = check_bf16(rp, ci, C, B, D, M, K, N, f"bf16 widened N={N} shift={shift}",
                       shift=shift)
        E32 = run_fused(rp, ci, widen(C), widen(B), widen(D), M, K, N)
        whole = np.diff(rp) <= sdl.resolve_tuning(sdl.DTYPE_F32, N, K=K).medium_max
        assert whole.sum() > M // 2
        assert np.array_equal(E[whole], E32[whole]), (N, shift)
        if N == 12:
            # a row view (rowptr[0] = 5): the same rows, bit for bit
            Ev = run_fused_bf16(rp + 5, np.concatenate([np.zeros(5, np.int32), ci]),
                                C, B, D, M, K, N)
            assert np.array_equal(Ev[whole], E[whole])


