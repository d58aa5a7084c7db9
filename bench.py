"""Benchmark of the CSR sparse x dense product C = A*B on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one call of the library's entry point -- the planning pass and
the worker kernel -- on the same resident inputs.  W untimed steps, then K
timed steps bracketed by device synchronisation; rank 0 prints one JSON line.

Metric: GFLOP/s = 2*nnz*N / time per step, with the effective bandwidth
min_bytes / time, where min_bytes is the minimum HBM traffic of one product
(rowptr, colind and vals read once, B read once, C written once).

Besides the headline, the line carries
  roofline      the worker kernel's algorithmic bytes (min_bytes) over its
                mean duration, timed with HIP events that the library
                records on the call's stream during the timed steps, against
                the 8 TB/s HBM peak; `traffic` is the HBM bytes per launch
                measured by rocprofv3 counters (FETCH_SIZE + WRITE_SIZE,
                scaled by a copy kernel of known size) when the committed
                profile matches the current kernel sources, else null;
                `cold_achieved` / `cold_frac`: the same for the median of
                the cold calls;
  cold          median and best of 20 calls, each after a 1 GiB write that
                evicts L2 and the Infinity Cache, each launch timed by the
                library's events;
  cpu_baseline  the fp64 oracle timed on this host's cores on the same
                matrix, and on one core, with the CPU model (a reported
                baseline, not a target).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("SpMM GFLOP/s (2·nnz·N) and effective HBM GB/s as % of peak, "
          "1 MI355X")
HBM_PEAK_GBPS = 8000.0
# Vector fp32 peak of the part: 256 CUs x 4 SIMDs x 16 lanes x 2 flops per
# FMA x 2 (packed fp32) x 2.4 GHz = 157.3 TFLOP/s (78.6 without packed math,
# which this build does not use).
VECTOR_FP32_PEAK_TFLOPS = 157.3


def roofline_bound(op_flops: float, op_bytes: float) -> str:
    """'alu' when the work's arithmetic intensity (flops per algorithmic
    byte) is above the part's balance point (vector fp32 peak over HBM
    peak, 19.7 flops per byte), else 'hbm'."""
    balance = VECTOR_FP32_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    return "alu" if op_flops / op_bytes > balance else "hbm"
DEFAULT_WORKLOAD = "powerlaw_262k_n64"
KERNEL_SOURCES = ["sparse_dense_linear_amd/csrc/worker.hip",
                  "sparse_dense_linear_amd/csrc/worker_impl.h",
                  "sparse_dense_linear_amd/csrc/worker_f32_buf.hip",
                  "sparse_dense_linear_amd/csrc/worker_f32_flat.hip",
                  "sparse_dense_linear_amd/csrc/worker_bf16_buf.hip",
                  "sparse_dense_linear_amd/csrc/worker_bf16_flat.hip",
                  "sparse_dense_linear_amd/csrc/worker_fused_buf.hip",
                  "sparse_dense_linear_amd/csrc/worker_fused_flat.hip",
                  "sparse_dense_linear_amd/csrc/eb.hip",
                  "sparse_dense_linear_amd/csrc/gather.h",
                  "sparse_dense_linear_amd/csrc/span.h",
                  "sparse_dense_linear_amd/csrc/sddmm.hip",
                  "sparse_dense_linear_amd/csrc/plan_device.h",
                  "sparse_dense_linear_amd/csrc/plan.hip",
                  "sparse_dense_linear_amd/csrc/internal.h",
                  "sparse_dense_linear_amd/csrc/api.hip"]
COUNTER_FILE = os.path.join(ROOT, "profiles", "counters_{workload}.md")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def min_bytes(p) -> int:
    """rowptr (M+1 int32) + colind and vals (nnz each) + B once + C (fp32)."""
    s_val = p.vals.dtype.itemsize
    s_b = p.B.dtype.itemsize
    return 4 * (p.M + 1) + p.nnz * (4 + s_val) + p.K * p.N * s_b + 4 * p.M * p.N


def sddmm_min_bytes(p) -> int:
    """rowptr + colind (nnz) + C (M x N) and B (K x N) once + A written."""
    s_d = p.B.dtype.itemsize
    return 4 * (p.M + 1) + 4 * p.nnz + (p.M + p.K) * p.N * s_d + 4 * p.nnz


def flops(p) -> int:
    return 2 * p.nnz * p.N


def measured_traffic(workload: str, op: str = "spmm"):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources."""
    path = COUNTER_FILE.format(workload=workload if op == "spmm" else f"{op}_{workload}")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_src = re.search(r"source_hash:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_b or m_src.group(1) != kernel_source_hash():
        return None
    return float(m_b.group(1))


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(p, budget_s: float = 10.0, op: str = "spmm", dense=None) -> dict:
    """The fp64 oracle on this host: on all cores (the reported value) and on
    one core, each repeated for about budget_s seconds on the whole
    matrix (at least once)."""
    import oracle

    def leg(threads):
        oracle.set_num_threads(threads)
        reps = 0
        t0 = time.perf_counter()
        while True:
            if op in ("spmm", "eb"):
                oracle.spmm_ref(p.rowptr, p.colind, p.vals, p.B, p.N, with_bound=False)
            elif op == "sddmm":
                oracle.sddmm_ref(p.rowptr, p.colind, dense, p.B, p.N)
            else:
                oracle.fusedmm_ref(p.rowptr, p.colind, dense, p.B, p.B, p.N)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or reps >= 1_000_000:
                return reps, el

    op_flops = flops(p) * (2 if op == "fusedmm" else 1)
    what = {"spmm": "C only, no bound", "eb": "C only, no bound",
            "sddmm": "SDDMM values and bound", "fusedmm": "FusedMM rows and bound"}[op]
    cores = oracle.num_threads()  # OpenMP's default: the host's threads
    reps, el = leg(cores)
    reps1, el1 = leg(1)
    oracle.set_num_threads(cores)
    return {"value": round(op_flops * reps / el / 1e9, 4), "unit": "GFLOP/s",
            "cores": cores, "kind": "oracle",
            "sample": f"the whole {p.name} matrix ({what}), {reps} repetitions "
                      f"in {el:.1f} s on {cores} threads",
            "one_core": {"value": round(op_flops * reps1 / el1 / 1e9, 4),
                         "unit": "GFLOP/s", "cores": 1,
                         "sample": f"{reps1} repetitions in {el1:.1f} s"},
            "cpu_model": cpu_model()}


def gather_ceiling(torch, dev) -> dict:
    """Bandwidth of the bare access pattern: output row i = sum of D random
    rows of B (D gathers of N fp32 + one row store per output row), for
    256-byte rows (N = 64) from a B the size of the power-law workload's
    (67 MB, fits the Infinity Cache) and one 16x larger (1 GiB, does not);
    for 1 KB rows (N = 256: the pruned and skewed workloads' row size) from
    a B of 4 MB (fits each XCD's L2) and of 1 GiB; and of a 1 GiB device
    copy.  Bytes counted: gathers + index reads + C writes (copy: read +
    write)."""
    import ctypes
    from sparse_dense_linear_amd import build as B_
    lib = ctypes.CDLL(B_.CEILING_PATH)
    lib.sdl_gather_ceiling.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_void_p]
    lib.sdl_gather_ceiling.restype = ctypes.c_int
    stream = torch.cuda.current_stream(dev)
    reps = 20

    def timed(fn):
        for _ in range(3):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    out = {"kernel": "gather_rows (ceiling.hip)", "reps": reps, "runs": []}
    for N, M, K, Ds in ((64, 262144, 262144, (1, 2, 4, 8)),
                        (64, 262144, 4194304, (1, 2, 4, 8)),
                        (256, 65536, 4096, (4, 8, 16)),
                        (256, 65536, 1048576, (4, 8, 16))):
        Bm = torch.randn(K * N, dtype=torch.float32, device=dev)
        for D in Ds:
            idx = torch.randint(0, K, (M * D,), dtype=torch.int32, device=dev)
            C = torch.empty(M * N, dtype=torch.float32, device=dev)

            def run():
                rc = lib.sdl_gather_ceiling(Bm.data_ptr(), idx.data_ptr(), C.data_ptr(),
                                            M, N, D, stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"sdl_gather_ceiling returned {rc}")
            t = timed(run)
            nbytes = M * D * N * 4 + M * D * 4 + M * N * 4
            out["runs"].append({"N": N, "M": M, "B_bytes": K * N * 4, "D": D,
                                "us": round(t * 1e6, 2), "GBps": round(nbytes / t / 1e9, 1)})
        del Bm
    a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    t = timed(lambda: b.copy_(a))
    out["copy_1GiB_GBps"] = round(2 * a.numel() * 4 / t / 1e9, 1)
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cold-reps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for counter scaling)")
    ap.add_argument("--gather-ceiling", action="store_true",
                    help="only time the bare row-gather kernel and a device copy")
    ap.add_argument("--n", type=int, default=None,
                    help="spmm only: dense width N in place of the workload's "
                         "(B drawn N(0,1) fp32 on the same pattern)")
    ap.add_argument("--op", default="spmm", choices=["spmm", "eb", "sddmm", "fusedmm"],
                    help="spmm: C = A*B (the headline); eb: the same product by the "
                         "element-balanced kernel; sddmm: A = (C B^T) sampled "
                         "on the workload's pattern, C drawn like B; fusedmm: "
                         "E = sum_p <C_i,B_j> D_j on the pattern (fp32 workloads)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import sparse_dense_linear_amd as sdl
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = 1 << 28  # 256 Mi floats = 1 GiB
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n,
                          "launches": 5}))
        return 0

    if args.gather_ceiling:
        print(json.dumps(gather_ceiling(torch, dev)), flush=True)
        return 0

    p = W.make(args.workload)
    if args.n is not None and args.n != p.N:
        if args.op != "spmm" or p.dtype != "f32":
            raise SystemExit("--n applies to the fp32 product only")
        rng = np.random.default_rng(args.n)
        p = W.CsrProblem(f"{p.name}_as_n{args.n}", p.M, p.K, args.n, p.rowptr, p.colind,
                         p.vals, rng.standard_normal((p.K, args.n)).astype(np.float32),
                         p.dtype, {**p.meta, "n_override": args.n})
    rowptr = torch.from_numpy(p.rowptr).to(dev)
    colind = torch.from_numpy(p.colind).to(dev)
    if p.dtype == "f32":
        vals = torch.from_numpy(p.vals).to(dev)
        B = torch.from_numpy(p.B.reshape(-1)).to(dev)
        fn = sdl.spmm_csr_f32
    else:
        vals = torch.from_numpy(p.vals.view(np.int16)).to(dev)
        B = torch.from_numpy(p.B.reshape(-1).view(np.int16)).to(dev)
        fn = sdl.spmm_csr_bf16in_f32acc
    stream = torch.cuda.current_stream(dev)
    if args.op in ("spmm", "eb"):
        C = torch.empty(p.M * p.N, dtype=torch.float32, device=dev)
        if args.op == "spmm":
            def step():
                fn(rowptr, colind, vals, B, C, p.M, p.K, p.N, stream)
        else:
            dt = sdl.DTYPE_F32 if p.dtype == "f32" else sdl.DTYPE_BF16

            def step():
                sdl.spmm_csr_eb(dt, rowptr, colind, vals, B, C, p.M, p.K, p.N, stream)
        op_flops, op_bytes = flops(p), min_bytes(p)
    else:
        # dense left operand: M x N, same element type and recipe as B
        Cd = torch.randn(p.M * p.N, dtype=torch.float32, device=dev,
                         generator=torch.Generator(device=dev).manual_seed(7))
        if p.dtype != "f32":
            Cd = Cd.to(torch.bfloat16).view(torch.int16)
        A = torch.empty(p.nnz, dtype=torch.float32, device=dev)
        sfn = sdl.sddmm_csr_f32 if p.dtype == "f32" else sdl.sddmm_csr_bf16in_f32acc

        def step():
            sfn(rowptr, colind, Cd, B, A, p.M, p.K, p.N, stream)
        op_flops, op_bytes = flops(p), sddmm_min_bytes(p)
        if args.op == "fusedmm":
            if p.dtype != "f32":
                raise SystemExit("fusedmm runs on fp32 workloads")
            Dd = torch.randn(p.K * p.N, dtype=torch.float32, device=dev,
                             generator=torch.Generator(device=dev).manual_seed(8))
            E = torch.empty(p.M * p.N, dtype=torch.float32, device=dev)

            def step():  # noqa: F811
                sdl.fusedmm_csr_f32(rowptr, colind, Cd, B, Dd, E, p.M, p.K, p.N,
                                    p.nnz, stream)
            op_flops = 2 * flops(p)
            op_bytes = sddmm_min_bytes(p) - 4 * p.nnz + (p.K + p.M) * p.N * 4
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K back-to-back steps on the host clock, no timing events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # kernel duration: the same steps again with HIP events attached to the
    # start and the end of each call's launch (on the call's stream)
    sdl.timing_enable(True)
    sdl.timing_read()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    sdl.timing_enable(False)
    plan_ms, worker_ms, ncalls = sdl.timing_read()
    faults = sdl.stream_faults(stream)
    if faults:
        raise RuntimeError(f"{faults} items were left undone (plan entries never visible)")

    ms_per_step = elapsed * 1e3 / args.steps
    gflops = op_flops / (ms_per_step * 1e-3) / 1e9
    mb = op_bytes
    eff = mb / (ms_per_step * 1e-3) / 1e9
    worker_avg_ms = worker_ms / max(ncalls, 1)
    achieved = mb / (worker_avg_ms * 1e-3) / 1e9 if worker_avg_ms > 0 else None

    # cold calls: evict L2 and the Infinity Cache (a 1 GiB write on the same
    # stream) before each call; each call's launch is timed by the events
    # the library attaches to it
    evict = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(args.cold_reps):
        evict.fill_(1.0)
        sdl.timing_enable(True)
        step()
        sdl.timing_enable(False)
        _, ms, n = sdl.timing_read()
        if n != 1:
            raise RuntimeError(f"expected one timed launch per cold call, got {n}")
        cold.append(ms)
    del evict
    if sdl.stream_faults(stream):
        raise RuntimeError("items were left undone in the cold calls")
    cold_med = float(np.median(cold)) if cold else None
    cold_best = min(cold) if cold else None
    cold_ach = None if not cold_med else mb / (cold_med * 1e-3) / 1e9

    traffic = measured_traffic(p.name, args.op)
    if roofline_bound(op_flops, mb) == "hbm":
        roofline = {
            "bound": "hbm",
            "achieved": None if achieved is None else round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": None if achieved is None else round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            # the same launch after a 1 GiB eviction of L2 and the Infinity
            # Cache (median of the cold calls below)
            "cold_achieved": None if cold_ach is None else round(cold_ach, 2),
            "cold_frac": None if cold_ach is None else round(cold_ach / HBM_PEAK_GBPS, 4),
        }
    else:
        # arithmetic intensity above the balance point: the vector fp32 ALU
        # roofline, flops per launch over the launch's duration
        tf = None if worker_avg_ms <= 0 else op_flops / (worker_avg_ms * 1e-3) / 1e12
        cold_tf = None if not cold_med else op_flops / (cold_med * 1e-3) / 1e12
        roofline = {
            "bound": "alu",
            "achieved": None if tf is None else round(tf, 3),
            "peak": VECTOR_FP32_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": None if tf is None else round(tf / VECTOR_FP32_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "cold_achieved": None if cold_tf is None else round(cold_tf, 3),
            "cold_frac": None if cold_tf is None else round(cold_tf / VECTOR_FP32_PEAK_TFLOPS, 4),
            "flops_per_byte": round(op_flops / mb, 2),
            "hbm_achieved": None if achieved is None else round(achieved, 2),
        }

    out = {
        "metric": METRIC if args.op in ("spmm", "eb") else METRIC.replace(
            "SpMM", {"sddmm": "SDDMM", "fusedmm": "FusedMM"}[args.op]).replace(
            "2·nnz·N", "2·nnz·N" if args.op == "sddmm" else "4·nnz·N"),
        "value": round(gflops, 3),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if p.dtype == "f32" else "bf16-in/f32-acc",
        "data": "synthetic",
        "config": {"workload": p.name, "op": args.op, "M": p.M, "K": p.K, "N": p.N,
                   "nnz": p.nnz, **{k: v for k, v in p.meta.items()
                                    if k not in ("hubs",)}},
        "eff_GBps": round(eff, 2),
        "hbm_frac": round(eff / HBM_PEAK_GBPS, 4),
        "min_bytes": mb,
        "flops_per_step": op_flops,
        "kernel_ms": {"call": round(worker_avg_ms, 6)},
        "roofline": roofline,
        "cold": {"median_ms": cold_med, "best_ms": cold_best,
                 "reps": len(cold),
                 "eff_GBps_median": None if not cold_med else round(mb / (cold_med * 1e-3) / 1e9, 2),
                 "gflops_median": None if not cold_med else round(op_flops / (cold_med * 1e-3) / 1e9, 3)},
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu:
        dense = None
        if args.op in ("sddmm", "fusedmm"):
            dense = Cd.cpu().numpy()
            dense = dense.view(np.uint16) if p.dtype != "f32" else dense
        out["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds, args.op, dense)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
