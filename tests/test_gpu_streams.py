"""Calls on several streams.  Each stream has its own scratch (plan words,
queue counters, epochs) and its own FusedMM / element-balanced work buffer,
so calls on two streams may run at the same time; calls on one stream reuse
its scratch, call after call.  Every result is checked against the oracle.
Streams are created with torch's default priority."""
import numpy as np
import pytest
import torch

import oracle
import sparse_dense_linear_amd as sdl
import workloads as W
from gpu_helpers import assert_parity

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _dev(p):
    return (torch.from_numpy(p.rowptr).cuda(), torch.from_numpy(p.colind).cuda(),
            torch.from_numpy(p.vals).cuda(),
            torch.from_numpy(np.ascontiguousarray(p.B).reshape(-1)).cuda())


def test_two_streams_concurrently():
    """Two problems of different shapes, product and element-balanced kernel,
    issued alternately on two streams several times (so the streams' calls
    overlap and each stream's epochs and queue sets advance), then checked."""
    p1 = W.powerlaw_rows(M=50000, N=64, seed=31)
    p2 = W.rows_with_lengths(np.random.default_rng(32).integers(0, 300, 3000), 5000, 128,
                             seed=32)
    a1, a2 = _dev(p1), _dev(p2)
    C1 = torch.full((p1.M * p1.N,), float("nan"), device="cuda")
    C2 = torch.full((p2.M * p2.N,), float("nan"), device="cuda")
    E1 = torch.full_like(C1, float("nan"))
    E2 = torch.full_like(C2, float("nan"))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(5):
        with torch.cuda.stream(s1):
            sdl.spmm_csr_f32(*a1, C1, p1.M, p1.K, p1.N, stream=s1)
            sdl.spmm_csr_eb(sdl.DTYPE_F32, *a1, E1, p1.M, p1.K, p1.N, stream=s1)
        with torch.cuda.stream(s2):
            sdl.spmm_csr_f32(*a2, C2, p2.M, p2.K, p2.N, stream=s2)
            sdl.spmm_csr_eb(sdl.DTYPE_F32, *a2, E2, p2.M, p2.K, p2.N, stream=s2)
    torch.cuda.synchronize()
    assert sdl.stream_faults(s1) == 0 and sdl.stream_faults(s2) == 0
    for p, C, E, what in ((p1, C1, E1, "stream 1"), (p2, C2, E2, "stream 2")):
        Cref, Sref = oracle.spmm_ref(p.rowptr, p.colind, p.vals, p.B, p.N)
        assert_parity(C.cpu().numpy().reshape(p.M, p.N), Cref, Sref, "f32", what)
        assert_parity(E.cpu().numpy().reshape(p.M, p.N), Cref, Sref, "f32", what + " eb")


def test_fusedmm_on_two_streams():
    """The two-launch FusedMM route keeps its value array per stream: two
    calls in flight on two streams must not share it."""
    rng = np.random.default_rng(33)
    M, K, N = 4000, 3000, 6            # N = 6: the two-launch route
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    cases = []
    for s in streams:
        p = W.rows_with_lengths(rng.integers(0, 60, M), K, N, seed=int(rng.integers(1 << 30)))
        Cd = rng.uniform(-1, 1, (M, N)).astype(np.float32)
        D = rng.uniform(-1, 1, (K, N)).astype(np.float32)
        E = torch.full((M * N,), float("nan"), device="cuda")
        cases.append((p, Cd, D, E, s))
    torch.cuda.synchronize()
    for _ in range(3):
        for p, Cd, D, E, s in cases:
            with torch.cuda.stream(s):
                sdl.fusedmm_csr_f32(torch.from_numpy(p.rowptr).cuda(),
                                    torch.from_numpy(p.colind).cuda(),
                                    torch.from_numpy(Cd).cuda(),
                                    torch.from_numpy(p.B.reshape(K, N)).cuda(),
                                    torch.from_numpy(D).cuda(), E, M, K, N, p.nnz, stream=s)
    torch.cuda.synchronize()
    for p, Cd, D, E, s in cases:
        assert sdl.stream_faults(s) == 0
        Eref, T = oracle.fusedmm_ref(p.rowptr, p.colind, Cd, p.B.reshape(K, N), D, N)
        got = E.cpu().numpy().reshape(M, N).astype(np.float64)
        bad = ~(np.abs(got - Eref) <= 2 * max(1e-5, N * 2.0 ** -23) * T + 1e-6)
        assert not bad.any(), f"{int(bad.sum())} of {got.size} outside the bound"


def test_growing_and_shrinking_calls_on_one_stream():
    """Calls of increasing then decreasing size on one stream: the stream's
    scratch grows when a call needs more, and later smaller calls reuse it."""
    s = torch.cuda.Stream()
    for M in (1000, 120000, 3000, 60000):
        p = W.powerlaw_rows(M=M, N=32, seed=M)
        a = _dev(p)
        C = torch.full((p.M * p.N,), float("nan"), device="cuda")
        with torch.cuda.stream(s):
            sdl.spmm_csr_f32(*a, C, p.M, p.K, p.N, stream=s)
        s.synchronize()
        assert sdl.stream_faults(s) == 0
        rows = np.random.default_rng(M).choice(p.M, 500, replace=False)
        Cref, Sref = oracle.spmm_ref(p.rowptr, p.colind, p.vals, p.B, p.N, rows=rows)
        assert_parity(C.cpu().numpy().reshape(p.M, p.N)[rows], Cref, Sref, "f32", f"M={M}")


def test_every_kind_of_call_interleaved_on_one_stream():
    """Product, element-balanced product, FusedMM (one launch and two
    launches), SDDMM and a product of another width, one after another on
    one stream, twice: each call takes the stream's next epoch and reuses its
    scratch and work buffer; every result must still match the oracle."""
    rng = np.random.default_rng(41)
    s = torch.cuda.Stream()
    p = W.powerlaw_rows(M=30000, N=64, seed=41)
    q = W.rows_with_lengths(rng.integers(0, 200, 2500), 4000, 6, seed=42)   # N = 6
    rp, ci, v, B = _dev(p)
    rq, cq, vq, Bq = _dev(q)
    Cf = rng.uniform(-1, 1, (p.M, p.N)).astype(np.float32)
    Df = rng.uniform(-1, 1, (p.K, p.N)).astype(np.float32)
    Cq = rng.uniform(-1, 1, (q.M, q.N)).astype(np.float32)
    Dq = rng.uniform(-1, 1, (q.K, q.N)).astype(np.float32)
    Cf_d, Df_d = torch.from_numpy(Cf).cuda(), torch.from_numpy(Df).cuda()
    Cq_d, Dq_d = torch.from_numpy(Cq).cuda(), torch.from_numpy(Dq).cuda()
    nan = lambda n: torch.full((n,), float("nan"), device="cuda")
    outs = {k: nan(n) for k, n in [("spmm", p.M * p.N), ("eb", p.M * p.N),
                                   ("fused1", p.M * p.N), ("fused2", q.M * q.N),
                                   ("sddmm", p.nnz), ("spmm_q", q.M * q.N)]}
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for _ in range(2):
            sdl.spmm_csr_f32(rp, ci, v, B, outs["spmm"], p.M, p.K, p.N, stream=s)
            sdl.spmm_csr_eb(sdl.DTYPE_F32, rp, ci, v, B, outs["eb"], p.M, p.K, p.N, stream=s)
            sdl.fusedmm_csr_f32(rp, ci, Cf_d, B, Df_d, outs["fused1"], p.M, p.K, p.N,
                                p.nnz, stream=s)
            sdl.fusedmm_csr_f32(rq, cq, Cq_d, Bq, Dq_d, outs["fused2"], q.M, q.K, q.N,
                                q.nnz, stream=s)
            sdl.sddmm_csr_f32(rp, ci, Cf_d, B, outs["sddmm"], p.M, p.K, p.N, stream=s)
            sdl.spmm_csr_f32(rq, cq, vq, Bq, outs["spmm_q"], q.M, q.K, q.N, stream=s)
    torch.cuda.synchronize()
    assert sdl.stream_faults(s) == 0
    got = {k: t.cpu().numpy() for k, t in outs.items()}
    Cref, Sref = oracle.spmm_ref(p.rowptr, p.colind, p.vals, p.B, p.N)
    assert_parity(got["spmm"].reshape(p.M, p.N), Cref, Sref, "f32", "spmm")
    assert_parity(got["eb"].reshape(p.M, p.N), Cref, Sref, "f32", "eb")
    Cqr, Sqr = oracle.spmm_ref(q.rowptr, q.colind, q.vals, q.B, q.N)
    assert_parity(got["spmm_q"].reshape(q.M, q.N), Cqr, Sqr, "f32", "spmm N=6")
    tol = lambda n: 2 * max(1e-5, n * 2.0 ** -23)
    for key, r, Cx, Dx in (("fused1", p, Cf, Df), ("fused2", q, Cq, Dq)):
        Eref, T = oracle.fusedmm_ref(r.rowptr, r.colind, Cx, r.B.reshape(r.K, r.N), Dx, r.N)
        e = got[key].reshape(r.M, r.N).astype(np.float64)
        assert np.all(np.abs(e - Eref) <= tol(r.N) * T + 1e-6), key
    Aref, S = oracle.sddmm_ref(p.rowptr, p.colind, Cf, p.B.reshape(p.K, p.N), p.N)
    assert np.all(np.abs(got["sddmm"].astype(np.float64) - Aref) <=
                  max(1e-5, p.N * 2.0 ** -23) * S + 1e-6), "sddmm"


def test_host_threads_on_their_own_streams():
    """Four host threads, each with its own stream, call the library at the
    same time (the binding releases Python's lock during a call), so the
    per-stream tables of scratch and work buffers are created and looked up
    concurrently."""
    import threading

    problems = [W.powerlaw_rows(M=20000, N=64, seed=50 + t) for t in range(4)]
    results, errors = {}, []

    def work(t):
        try:
            p = problems[t]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                a = _dev(p)
                C = torch.full((p.M * p.N,), float("nan"), device="cuda")
                E = torch.full((p.M * p.N,), float("nan"), device="cuda")
                for _ in range(10):
                    sdl.spmm_csr_f32(*a, C, p.M, p.K, p.N, stream=s)
                    sdl.spmm_csr_eb(sdl.DTYPE_F32, *a, E, p.M, p.K, p.N, stream=s)
            s.synchronize()
            results[t] = (C.cpu().numpy(), E.cpu().numpy(), sdl.stream_faults(s))
        except Exception as exc:           # reported by the main thread
            errors.append(exc)

    threads = [threading.Thread(target=work, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not errors, errors
    for t, p in enumerate(problems):
        C, E, faults = results[t]
        assert faults == 0
        Cref, Sref = oracle.spmm_ref(p.rowptr, p.colind, p.vals, p.B, p.N)
        assert_parity(C.reshape(p.M, p.N), Cref, Sref, "f32", f"thread {t}")
        assert_parity(E.reshape(p.M, p.N), Cref, Sref, "f32", f"thread {t} eb")


def test_host_threads_on_one_stream():
    """Four host threads share ONE stream.  Each issues products of growing
    M (so the stream's scratch block is replaced by larger ones while other
    threads' calls that use the old block are already enqueued), each
    followed by an element-balanced call (which takes an epoch and clears
    the next queue set).  The library holds the stream's lock from a call's
    choice of epoch and block until its launch is enqueued, so epochs reach
    the stream in order; every result is checked against the oracle."""
    import threading

    sizes = [(3000, 15000, 60000), (5000, 25000, 45000),
             (2000, 35000, 70000), (8000, 12000, 80000)]
    problems = [[W.powerlaw_rows(M=m, N=64, seed=70 + 10 * t + k)
                 for k, m in enumerate(sizes[t])] for t in range(4)]
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    outs, errors = {}, []
    start = threading.Barrier(4)

    def work(t):
        try:
            with torch.cuda.stream(s):
                bufs = []
                for p in problems[t]:
                    a = _dev(p)
                    C = torch.full((p.M * p.N,), float("nan"), device="cuda")
                    E = torch.full((p.M * p.N,), float("nan"), device="cuda")
                    bufs.append((p, a, C, E))
                s.synchronize()
                start.wait(timeout=60)
                for _ in range(3):
                    for p, a, C, E in bufs:
                        sdl.spmm_csr_f32(*a, C, p.M, p.K, p.N, stream=s)
                        sdl.spmm_csr_eb(sdl.DTYPE_F32, *a, E, p.M, p.K, p.N, stream=s)
            outs[t] = bufs
        except Exception as exc:           # reported by the main thread
            errors.append(exc)

    threads = [threading.Thread(target=work, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not errors, errors
    s.synchronize()
    assert sdl.stream_faults(s) == 0
    for t in range(4):
        for p, _, C, E in outs[t]:
            Cref, Sref = oracle.spmm_ref(p.rowptr, p.colind, p.vals, p.B, p.N)
            assert_parity(C.cpu().numpy().reshape(p.M, p.N), Cref, Sref, "f32",
                          f"thread {t} M={p.M}")
            assert_parity(E.cpu().numpy().reshape(p.M, p.N), Cref, Sref, "f32",
                          f"thread {t} M={p.M} eb")
    sdl.stream_release(s)


def test_stream_release_then_reuse():
    """After spmm_stream_release the stream's blocks are gone; the next call
    on the same stream allocates fresh ones and is still correct."""
    p = W.powerlaw_rows(M=30000, N=64, seed=91)
    a = _dev(p)
    s = torch.cuda.Stream()
    C = torch.full((p.M * p.N,), float("nan"), device="cuda")
    Cref, Sref = oracle.spmm_ref(p.rowptr, p.colind, p.vals, p.B, p.N)
    for _ in range(2):
        with torch.cuda.stream(s):
            sdl.spmm_csr_f32(*a, C, p.M, p.K, p.N, stream=s)
            sdl.spmm_csr_eb(sdl.DTYPE_F32, *a, C, p.M, p.K, p.N, stream=s)
        sdl.stream_release(s)        # waits for the stream
        assert_parity(C.cpu().numpy().reshape(p.M, p.N), Cref, Sref, "f32", "release")
        C.fill_(float("nan"))
    sdl.stream_release(s)            # nothing held: a no-op
