"""The C-ABI library without a GPU: it loads, exports every function the
header declares, resolves thresholds, and rejects bad arguments on the host
before any HIP call."""
import ctypes
import os
import re

import pytest
import torch

import sparse_dense_linear_amd as sdl
from sparse_dense_linear_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spmm.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    # every function declaration: a return type, a name, an opening paren
    names = re.findall(r"^\s*(?:spmm_status_t|const\s+char\s*\*)\s*(\w+)\s*\(",
                       text, re.M)
    return sorted(set(names))


def test_header_declares_entry_points():
    names = header_functions()
    for must in ("spmm_csr_f32", "spmm_csr_bf16in_f32acc", "spmm_csr_tuned",
                 "spmm_resolve_tuning", "spmm_plan_export", "spmm_status_string",
                 "spmm_last_error", "spmm_timing_enable", "spmm_timing_read",
                 "spmm_stream_faults", "spmm_stream_release", "spmm_csr_tuned_noalloc",
                 "spmm_debug_set_wait_polls",
                 "sddmm_csr_f32", "sddmm_csr_bf16in_f32acc",
                 "fusedmm_csr_f32", "fusedmm_csr_bf16in_f32acc"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(sdl.lib_path())
    missing = [n for n in header_functions() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"


def test_status_strings():
    assert sdl.status_string(0) == "SPMM_SUCCESS"
    assert sdl.status_string(1) == "SPMM_ERROR_INVALID_VALUE"
    assert sdl.status_string(2) == "SPMM_ERROR_HIP"
    assert sdl.status_string(3) == "SPMM_ERROR_OUT_OF_MEMORY"
    assert sdl.status_string(4) == "SPMM_ERROR_UNSUPPORTED"
    assert sdl.status_string(99) == "SPMM_ERROR_UNKNOWN"


@pytest.mark.parametrize("dtype,N", [(0, 32), (0, 64), (0, 128), (0, 1), (0, 1000),
                                     (1, 256), (1, 512), (1, 3)])
def test_resolve_defaults_are_consistent(dtype, N):
    t = sdl.resolve_tuning(dtype, N)
    assert 0 <= t.short_max <= t.medium_max
    assert 128 <= t.chunk_nnz <= 4096
    assert t.medium_max == t.chunk_nnz
    # explicit values win over defaults
    u = sdl.resolve_tuning(dtype, N, sdl.Tuning(3, 77, 11))
    assert (u.short_max, u.medium_max, u.chunk_nnz) == (3, 77, 11)


def test_resolve_rejects_bad_input():
    with pytest.raises(sdl.SpmmError) as e:
        sdl.resolve_tuning(0, 64, sdl.Tuning(10, 5, 4))
    assert e.value.status == 1
    with pytest.raises(sdl.SpmmError):
        sdl.resolve_tuning(7, 64)
    with pytest.raises(sdl.SpmmError):
        sdl.resolve_tuning(0, -1)


def raw_call(fn, *args):
    L = sdl.lib()
    return getattr(L, fn)(*args)


FAKE = 0x10000  # never dereferenced: every case below fails or returns first


@pytest.mark.parametrize("M,K,N,rowptr,B,C,expect", [
    (-1, 4, 4, FAKE, FAKE, FAKE, 1),        # negative M
    (4, -1, 4, FAKE, FAKE, FAKE, 1),        # negative K
    (4, 4, -2, FAKE, FAKE, FAKE, 1),        # negative N
    (2 ** 31, 4, 4, FAKE, FAKE, FAKE, 1),   # M too large for int32 rows
    (4, 2 ** 31, 4, FAKE, FAKE, FAKE, 1),   # K too large
    (4, 4, 4, None, FAKE, FAKE, 1),         # rowptr null
    (4, 4, 4, FAKE, None, FAKE, 1),         # B null with K > 0
    (4, 4, 4, FAKE, FAKE, None, 1),         # C null
    (4, 4, 4, FAKE, FAKE, FAKE + 2, 1),     # C misaligned
    (4, 4, 4, FAKE, FAKE + 1, FAKE, 1),     # B misaligned for fp32
    (0, 4, 4, None, None, None, 0),         # M == 0: nothing to do
    (4, 4, 0, None, None, None, 0),         # N == 0: nothing to do
])
def test_host_validation_f32(M, K, N, rowptr, B, C, expect):
    rc = raw_call("spmm_csr_f32", rowptr, FAKE, FAKE, B, C, M, K, N, None)
    assert rc == expect, sdl.lib().spmm_last_error()


def test_host_validation_bf16_alignment():
    # bf16 B needs 2-byte alignment only; an odd address is rejected
    rc = raw_call("spmm_csr_bf16in_f32acc", FAKE, FAKE, FAKE, FAKE + 1, FAKE,
                  4, 4, 4, None)
    assert rc == 1


def test_tuned_rejects_bad_tuning():
    T = _binding._TuningStruct
    bad = T(short_max=10, medium_max=5, chunk_nnz=4, hub_min=-1, slab_rows=0)
    rc = raw_call("spmm_csr_tuned", 0, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 4,
                  ctypes.byref(bad), None)
    assert rc == 1
    reserved = T(short_max=1, medium_max=5, chunk_nnz=4, hub_min=-1, slab_rows=0,
                 reserved=1)
    rc = raw_call("spmm_csr_tuned", 0, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 4,
                  ctypes.byref(reserved), None)
    assert rc == 1
    rc = raw_call("spmm_csr_tuned", 5, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 4,
                  None, None)
    assert rc == 1


@pytest.mark.parametrize("dtype,K,N,hubs", [
    (1, 1048576, 512, True),    # B 1 GiB: hub rows by default
    (0, 1048576, 64, True),     # B exactly 256 MiB
    (0, 262144, 64, False),     # B 64 MiB: the Infinity Cache holds it
    (0, 4096, 256, False),      # B 4 MiB
    (0, 1024, 32, False),
    (0, 0, 64, False),
])
def test_resolve_hub_defaults(dtype, K, N, hubs):
    """Hub rows by default only for a B of at least 256 MiB; slabs of 2 MiB of
    B's rows; the hub threshold at least medium_max and 32 entries per slab."""
    t = sdl.resolve_tuning(dtype, N, K=K)
    esz = 2 if dtype == 1 else 4
    assert t.slab_rows == max(1, (2 << 20) // (N * esz))
    if hubs:
        n_slabs = -(-K // t.slab_rows)
        assert t.hub_min == max(t.medium_max, 32 * n_slabs)
    else:
        assert t.hub_min == 2 ** 31 - 1
    # explicit values win
    u = sdl.resolve_tuning(dtype, N, sdl.Tuning(hub_min=5, slab_rows=9), K=K)
    assert (u.hub_min, u.slab_rows) == (5, 9)


def test_noalloc_rejects_on_the_host():
    """The no-allocation entry point checks like spmm_csr_tuned, and rejects
    an M whose plan does not fit its fixed array, before any HIP call."""
    rc = raw_call("spmm_csr_tuned_noalloc", 0, FAKE, FAKE, FAKE, FAKE, FAKE, -1, 4, 4,
                  None, None)
    assert rc == 1
    rc = raw_call("spmm_csr_tuned_noalloc", 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 22, 4, 4,
                  None, None)
    assert rc == 4
    msg = sdl.lib().spmm_last_error().decode()
    assert "at most" in msg and "rows" in msg
    rc = raw_call("spmm_csr_tuned_noalloc", 0, None, None, None, None, None, 0, 4, 4,
                  None, None)
    assert rc == 0                      # M == 0: nothing to do


def test_wait_bound_hook_range():
    """The wait-bound test hook takes 0 .. the default, or a negative value
    for the default, and refuses a larger bound (host only, no HIP call)."""
    L = sdl.lib()
    assert L.spmm_debug_set_wait_polls(1 << 20) == 1
    assert b"default" in L.spmm_last_error()
    assert L.spmm_debug_set_wait_polls(0) == 0
    assert L.spmm_debug_set_wait_polls(1 << 19) == 0
    assert L.spmm_debug_set_wait_polls(-1) == 0


def test_forced_allocation_failure(monkeypatch):
    monkeypatch.setenv("SPMM_TEST_FAIL_ALLOC", "1")
    rc = raw_call("spmm_csr_f32", FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 4, None)
    assert rc == 3
    assert b"SPMM_TEST_FAIL_ALLOC" in sdl.lib().spmm_last_error()


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU path")
def test_valid_call_without_gpu_reports_hip_error():
    rc = raw_call("spmm_csr_f32", FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 4, None)
    assert rc == 2
    assert sdl.lib().spmm_last_error() != b""


def test_plan_export_validation():
    counts = (ctypes.c_int64 * 6)()
    T = _binding._TuningStruct
    t = T(short_max=-1, medium_max=5, chunk_nnz=4, hub_min=2 ** 31 - 1, slab_rows=1)
    rc = raw_call("spmm_plan_export", FAKE, FAKE, 4, 4, ctypes.byref(t), None, 0, counts,
                  None, None, None, None, None)
    assert rc == 1                      # not resolved
    t = T(short_max=1, medium_max=5, chunk_nnz=4, hub_min=10, slab_rows=1)
    rc = raw_call("spmm_plan_export", FAKE, None, 4, 4, ctypes.byref(t), None, 0, counts,
                  None, None, None, None, None)
    assert rc == 1                      # hub rows possible: colind needed
    t = T(short_max=1, medium_max=5, chunk_nnz=4, hub_min=2 ** 31 - 1, slab_rows=1)
    rc = raw_call("spmm_plan_export", FAKE, None, 0, 4, ctypes.byref(t), None, 0, counts,
                  None, None, None, None, None)
    assert rc == 0 and list(counts) == [0] * 6


def test_timing_read_empty():
    sdl.timing_enable(False)
    assert sdl.timing_read() == (0.0, 0.0, 0)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "_LIB_FILE", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _binding.lib()


def test_binding_checks_operands():
    """Marshalling rejects CPU tensors and wrong dtypes before any call."""
    t = torch.zeros(4, dtype=torch.int32)
    f = torch.zeros(4, dtype=torch.float32)
    with pytest.raises((ValueError, TypeError)):
        sdl.spmm_csr_f32(t, t, f, f, f, 3, 2, 2)


@pytest.mark.parametrize("M,K,N,nnz,rowptr,C,B,A,expect", [
    (-1, 4, 4, 4, FAKE, FAKE, FAKE, FAKE, 1),         # negative M
    (4, 4, 4, -1, FAKE, FAKE, FAKE, FAKE, 1),         # negative nnz
    (4, 4, 4, 2 ** 31, FAKE, FAKE, FAKE, FAKE, 1),    # nnz too large
    (0, 4, 4, 3, FAKE, FAKE, FAKE, FAKE, 1),          # entries without rows
    (4, 4, 0, 3, FAKE, FAKE, FAKE, FAKE, 4),          # N == 0 with entries
    (4, 4, 4, 3, None, FAKE, FAKE, FAKE, 1),          # rowptr null
    (4, 4, 4, 3, FAKE, None, FAKE, FAKE, 1),          # C null
    (4, 4, 4, 3, FAKE, FAKE, FAKE, None, 1),          # A null
    (4, 4, 4, 3, FAKE, FAKE + 2, FAKE, FAKE, 1),      # C misaligned
    (4, 4, 4, 3, FAKE, FAKE, FAKE, FAKE + 1, 1),      # A misaligned
    (4, 4, 4, 0, None, None, None, None, 0),          # no entries: nothing to do
])
def test_sddmm_host_validation(M, K, N, nnz, rowptr, C, B, A, expect):
    rc = raw_call("sddmm_csr_f32", rowptr, FAKE, C, B, A, M, K, N, nnz, None)
    assert rc == expect, sdl.lib().spmm_last_error()


def test_sddmm_bf16_alignment():
    rc = raw_call("sddmm_csr_bf16in_f32acc", FAKE, FAKE, FAKE + 1, FAKE, FAKE,
                  4, 4, 4, 3, None)
    assert rc == 1


@pytest.mark.parametrize("M,K,N,nnz,rowptr,E,D,expect", [
    (-1, 4, 4, 4, FAKE, FAKE, FAKE, 1),      # negative M
    (4, 4, 4, 2 ** 31, FAKE, FAKE, FAKE, 1),  # nnz too large
    (4, 4, 4, 3, None, FAKE, FAKE, 1),       # rowptr null
    (4, 4, 4, 3, FAKE, None, FAKE, 1),       # E null
    (4, 4, 4, 3, FAKE, FAKE, None, 1),       # D null with entries
    (4, 4, 4, 3, FAKE, FAKE + 2, FAKE, 1),   # E misaligned
    (0, 4, 4, 0, None, None, None, 0),       # M == 0: nothing to do
    (4, 4, 0, 0, None, None, None, 0),       # N == 0: nothing to do
])
def test_fusedmm_host_validation(M, K, N, nnz, rowptr, E, D, expect):
    rc = raw_call("fusedmm_csr_f32", rowptr, FAKE, FAKE, FAKE, D, E, M, K, N, nnz, None)
    assert rc == expect, sdl.lib().spmm_last_error()


@pytest.mark.parametrize("M,K,N,nnz,rowptr,C,D,E,expect", [
    (-1, 4, 8, 4, FAKE, FAKE, FAKE, FAKE, 1),        # negative M
    (4, 4, 8, 2 ** 31, FAKE, FAKE, FAKE, FAKE, 1),   # nnz too large
    (4, 4, 8, 3, None, FAKE, FAKE, FAKE, 1),         # rowptr null
    (4, 4, 8, 3, FAKE, None, FAKE, FAKE, 1),         # C null with entries
    (4, 4, 8, 3, FAKE, FAKE, None, FAKE, 1),         # D null with entries
    (4, 4, 8, 3, FAKE, FAKE, FAKE, None, 1),         # E null
    (4, 4, 8, 3, FAKE, FAKE + 1, FAKE, FAKE, 1),     # C not 2-byte aligned
    (4, 4, 8, 3, FAKE, FAKE, FAKE, FAKE + 2, 1),     # E not 4-byte aligned
    (0, 4, 8, 0, None, None, None, None, 0),         # M == 0: nothing to do
    (4, 4, 0, 0, None, None, None, None, 0),         # N == 0: nothing to do
])
def test_fusedmm_bf16_host_validation(M, K, N, nnz, rowptr, C, D, E, expect):
    """bf16 FusedMM refuses bad arguments on the host before any HIP call."""
    rc = raw_call("fusedmm_csr_bf16in_f32acc", rowptr, FAKE, C, FAKE, D, E, M, K, N,
                  nnz, None)
    assert rc == expect, sdl.lib().spmm_last_error()


def test_fusedmm_forced_allocation_failure(monkeypatch):
    monkeypatch.setenv("SPMM_TEST_FAIL_ALLOC", "1")
    rc = raw_call("fusedmm_csr_f32", FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 4, 3, None)
    # without a GPU the device query fails first; with one, the forced failure
    assert rc in (2, 3)


@pytest.mark.parametrize("N,C", [(12, FAKE), (1032, FAKE), (64, FAKE + 2)])
def test_fusedmm_bf16_widened_allocation_failure(monkeypatch, N, C):
    """Shapes outside the one-launch form take the widened copy: its
    allocation is the first thing after the device query that can fail."""
    monkeypatch.setenv("SPMM_TEST_FAIL_ALLOC", "1")
    rc = raw_call("fusedmm_csr_bf16in_f32acc", FAKE, FAKE, C, FAKE, FAKE, FAKE, 4, 4, N,
                  3, None)
    assert rc in (2, 3)
    assert b"SPMM_TEST_FAIL_ALLOC" in sdl.lib().spmm_last_error() or rc == 2


def test_fusedmm_bf16_widened_size_bound():
    """A widened copy whose size would pass 64 bits is refused before any
    HIP call (no size is computed from a wrapped product)."""
    big = 2 ** 31 - 1
    rc = raw_call("fusedmm_csr_bf16in_f32acc", FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big, big,
                  big, 3, None)
    assert rc == 3, sdl.lib().spmm_last_error()
    assert b"2^56" in sdl.lib().spmm_last_error()


def test_sddmm_binding_checks_operands():
    t = torch.zeros(4, dtype=torch.int32)
    f = torch.zeros(4, dtype=torch.float32)
    with pytest.raises((ValueError, TypeError)):
        sdl.sddmm_csr_f32(t, t, f, f, f, 3, 2, 2)
    with pytest.raises((ValueError, TypeError)):
        sdl.fusedmm_csr_f32(t, t, f, f, f, f, 3, 2, 2, 4)
    h = torch.zeros(4, dtype=torch.int16)
    with pytest.raises((ValueError, TypeError)):
        sdl.fusedmm_csr_bf16in_f32acc(t, t, h, h, h, f, 3, 2, 2, 4)
