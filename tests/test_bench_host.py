"""Host-side logic of bench.py, without a GPU: the one-GPU contract, the
algorithmic byte counts behind the roofline fraction, and when measured
traffic is reported."""
import importlib.util
import os
import subprocess
import sys

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


def test_more_than_one_gpu_is_refused():
    """--gpus N > 1 ends with a message and no JSON line, before any GPU
    call."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_min_bytes_reads_every_input_once_and_writes_C_once():
    """rowptr, colind, vals and B read once, C (fp32) written once: the sum of
    the arrays' own sizes, for fp32 and bf16 inputs."""
    for name in ("uniform_1k_n32", "pruned_4k_n256_bf16"):
        p = W.make(name)
        expect = (p.rowptr.nbytes + p.colind.nbytes + p.vals.nbytes + p.B.nbytes +
                  4 * p.M * p.N)
        assert bench.min_bytes(p) == expect, name


def test_sddmm_min_bytes():
    """rowptr and colind read, C (M x N) and B (K x N) read once, one fp32
    value written per stored entry."""
    p = W.make("uniform_1k_n32")
    expect = (p.rowptr.nbytes + p.colind.nbytes + p.M * p.N * p.B.itemsize +
              p.B.nbytes + 4 * p.nnz)
    assert bench.sddmm_min_bytes(p) == expect


def test_flops_are_two_per_entry_and_column():
    p = W.make("uniform_1k_n32")
    assert bench.flops(p) == 2 * p.nnz * p.N


def test_traffic_reported_only_for_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "COUNTER_FILE", str(tmp_path / "counters_{workload}.md"))
    current = bench.kernel_source_hash()
    (tmp_path / "counters_w.md").write_text(
        f"source_hash: {current}\nhbm_bytes_per_launch: 123456\n")
    assert bench.measured_traffic("w") == 123456.0
    (tmp_path / "counters_sddmm_w.md").write_text(
        f"source_hash: {current}\nhbm_bytes_per_launch: 789\n")
    assert bench.measured_traffic("w", "sddmm") == 789.0
    (tmp_path / "counters_w.md").write_text(
        "source_hash: 0000000000000000\nhbm_bytes_per_launch: 123456\n")
    assert bench.measured_traffic("w") is None
    assert bench.measured_traffic("absent") is None


def test_source_hash_covers_every_kernel_source():
    """Every HIP source and header the library is built from is hashed (the
    measurement-only gather probe aside)."""
    csrc = os.path.join(ROOT, "sparse_dense_linear_amd", "csrc")
    files = {f"sparse_dense_linear_amd/csrc/{f}" for f in os.listdir(csrc)
             if f.endswith((".hip", ".h")) and f != "ceiling.hip"}
    assert files == set(bench.KERNEL_SOURCES)


def test_roofline_bound_follows_arithmetic_intensity():
    """Work above the balance point (157.3 TFLOP/s over 8 TB/s, 19.7 flops
    per algorithmic byte) is measured against the vector ALU peak: the
    pruned (about 39-52 flops per byte) and skewed (about 31) products, not
    the uniform (2.6), power-law (1.0) or banded (6.4) ones."""
    for name, expect in (("uniform_1k_n32", "hbm"), ("pruned_4k_n256_f32", "alu"),
                         ("pruned_4k_n256_bf16", "alu")):
        p = W.make(name)
        assert bench.roofline_bound(bench.flops(p), bench.min_bytes(p)) == expect, name
    # the skewed, banded and power-law intensities, from their sizes
    assert bench.roofline_bound(123.0e9, 3.946e9) == "alu"
    assert bench.roofline_bound(34.36e9, 5.385e9) == "hbm"
    assert bench.roofline_bound(140.3e6, 144.0e6) == "hbm"
