"""ctypes binding of libsdl_spmm.so: argument marshalling only."""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_FILE = os.path.join(_HERE, "libsdl_spmm.so")

DTYPE_F32 = 0
DTYPE_BF16 = 1

SUCCESS = 0
ERROR_INVALID_VALUE = 1
ERROR_HIP = 2
ERROR_OUT_OF_MEMORY = 3
ERROR_UNSUPPORTED = 4


class SpmmError(RuntimeError):
    """A library call returned a status other than SPMM_SUCCESS."""

    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func}: {status_string(status)} ({detail})")


class _TuningStruct(ctypes.Structure):
    _fields_ = [("short_max", ctypes.c_int32), ("medium_max", ctypes.c_int32),
                ("chunk_nnz", ctypes.c_int32), ("hub_min", ctypes.c_int32),
                ("slab_rows", ctypes.c_int32), ("reserved", ctypes.c_int32)]


@dataclass
class Tuning:
    """Row-routing thresholds (spmm_tuning_t); -1 / 0 ask for defaults."""
    short_max: int = -1
    medium_max: int = -1
    chunk_nnz: int = 0
    hub_min: int = -1
    slab_rows: int = 0

    def _struct(self) -> _TuningStruct:
        return _TuningStruct(self.short_max, self.medium_max, self.chunk_nnz,
                             self.hub_min, self.slab_rows, 0)


_lib = None


def lib_path() -> str:
    return _LIB_FILE


def lib() -> ctypes.CDLL:
    """The loaded shared library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_FILE):
        raise ImportError(
            f"{_LIB_FILE} is missing: build it with __graft_entry__.build() "
            "(or python sparse_dense_linear_amd/build.py)")
    L = ctypes.CDLL(_LIB_FILE)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.spmm_csr_f32.argtypes = [P, P, P, P, P, I64, I64, I64, P]
    L.spmm_csr_bf16in_f32acc.argtypes = [P, P, P, P, P, I64, I64, I64, P]
    L.spmm_csr_tuned.argtypes = [I32, P, P, P, P, P, I64, I64, I64,
                                 ctypes.POINTER(_TuningStruct), P]
    L.spmm_csr_tuned_noalloc.argtypes = [I32, P, P, P, P, P, I64, I64, I64,
                                         ctypes.POINTER(_TuningStruct), P]
    L.spmm_resolve_tuning.argtypes = [I32, I64, I64, ctypes.POINTER(_TuningStruct),
                                      ctypes.POINTER(_TuningStruct)]
    L.spmm_plan_export.argtypes = [P, P, I64, I64, ctypes.POINTER(_TuningStruct), P, I64,
                                   P, P, P, P, P, P]
    L.spmm_status_string.argtypes = [I32]
    L.spmm_status_string.restype = ctypes.c_char_p
    L.spmm_last_error.argtypes = []
    L.spmm_last_error.restype = ctypes.c_char_p
    L.spmm_timing_enable.argtypes = [I32]
    L.spmm_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double),
                                   ctypes.POINTER(ctypes.c_double),
                                   ctypes.POINTER(ctypes.c_int64)]
    L.spmm_stream_faults.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)]
    L.spmm_stream_release.argtypes = [ctypes.c_void_p]
    L.spmm_debug_set_wait_polls.argtypes = [I64]
    L.sddmm_csr_f32.argtypes = [P, P, P, P, P, I64, I64, I64, I64, P]
    L.sddmm_csr_bf16in_f32acc.argtypes = [P, P, P, P, P, I64, I64, I64, I64, P]
    L.fusedmm_csr_f32.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, P]
    L.fusedmm_csr_bf16in_f32acc.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, P]
    L.spmm_csr_eb.argtypes = [I32, P, P, P, P, P, I64, I64, I64, P]
    for name in ("sddmm_csr_f32", "sddmm_csr_bf16in_f32acc", "fusedmm_csr_f32",
                 "fusedmm_csr_bf16in_f32acc", "spmm_csr_eb"):
        getattr(L, name).restype = I32
    for name in ("spmm_csr_f32", "spmm_csr_bf16in_f32acc", "spmm_csr_tuned",
                 "spmm_csr_tuned_noalloc",
                 "spmm_resolve_tuning", "spmm_plan_export", "spmm_timing_enable",
                 "spmm_timing_read", "spmm_stream_faults", "spmm_stream_release",
                 "spmm_debug_set_wait_polls"):
        getattr(L, name).restype = I32
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().spmm_status_string(status).decode()


def _check(status: int, func: str) -> None:
    if status != SUCCESS:
        raise SpmmError(status, func, lib().spmm_last_error().decode())


# ------------------------------------------------------------ marshalling

def _torch():
    import torch
    return torch


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr() if t.numel() > 0 else None


def _stream_handle(device, stream) -> int | None:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _check_operands(rowptr, colind, vals, B, C, M, K, N, val_dtypes, b_dtypes):
    torch = _torch()
    tensors = {"rowptr": rowptr, "colind": colind, "vals": vals, "B": B, "C": C}
    dev = C.device
    for name, t in tensors.items():
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device != dev or dev.type != "cuda":
            raise ValueError(f"{name} must live on the same GPU as C")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if rowptr.dtype != torch.int32 or colind.dtype != torch.int32:
        raise TypeError("rowptr and colind must be int32")
    if vals.dtype not in val_dtypes or B.dtype not in b_dtypes:
        raise TypeError(f"vals/B dtype must be one of {val_dtypes}/{b_dtypes}")
    if C.dtype != torch.float32:
        raise TypeError("C must be float32")
    if rowptr.numel() != M + 1:
        raise ValueError("rowptr must hold M+1 entries")
    if B.numel() != K * N or C.numel() != M * N:
        raise ValueError("B must hold K*N and C M*N elements")
    if colind.numel() != vals.numel():
        raise ValueError("colind and vals must have the same length")
    return dev


def spmm_csr_f32(rowptr, colind, vals, B, C, M: int, K: int, N: int,
                 stream=None) -> None:
    """C = A * B, fp32 values and B (spmm_csr_f32); enqueued on `stream`
    (default: torch's current stream of C's device)."""
    torch = _torch()
    dev = _check_operands(rowptr, colind, vals, B, C, M, K, N,
                          (torch.float32,), (torch.float32,))
    _check(lib().spmm_csr_f32(_ptr(rowptr), _ptr(colind), _ptr(vals), _ptr(B),
                              _ptr(C), M, K, N, _stream_handle(dev, stream)),
           "spmm_csr_f32")


def spmm_csr_bf16in_f32acc(rowptr, colind, vals, B, C, M: int, K: int, N: int,
                           stream=None) -> None:
    """C = A * B, bf16 values and B (torch.bfloat16 or raw int16/uint16 bit
    patterns), fp32 accumulation and C (spmm_csr_bf16in_f32acc)."""
    torch = _torch()
    bf = (torch.bfloat16, torch.int16, torch.uint16)
    dev = _check_operands(rowptr, colind, vals, B, C, M, K, N, bf, bf)
    _check(lib().spmm_csr_bf16in_f32acc(_ptr(rowptr), _ptr(colind), _ptr(vals),
                                        _ptr(B), _ptr(C), M, K, N,
                                        _stream_handle(dev, stream)),
           "spmm_csr_bf16in_f32acc")


def spmm_csr_tuned(dtype: int, rowptr, colind, vals, B, C, M: int, K: int,
                   N: int, tuning: Tuning | None = None, stream=None) -> None:
    """Either element type with explicit routing thresholds (spmm_csr_tuned)."""
    torch = _torch()
    if dtype == DTYPE_F32:
        vd = bd = (torch.float32,)
    else:
        vd = bd = (torch.bfloat16, torch.int16, torch.uint16)
    dev = _check_operands(rowptr, colind, vals, B, C, M, K, N, vd, bd)
    ts = None if tuning is None else ctypes.byref(tuning._struct())
    _check(lib().spmm_csr_tuned(dtype, _ptr(rowptr), _ptr(colind), _ptr(vals),
                                _ptr(B), _ptr(C), M, K, N, ts,
                                _stream_handle(dev, stream)),
           "spmm_csr_tuned")


def spmm_csr_tuned_noalloc(dtype: int, rowptr, colind, vals, B, C, M: int, K: int,
                           N: int, tuning: Tuning | None = None, stream=None) -> None:
    """spmm_csr_tuned with its plan scratch in the library's fixed per-GPU
    array (spmm_csr_tuned_noalloc): no device allocation."""
    torch = _torch()
    if dtype == DTYPE_F32:
        vd = bd = (torch.float32,)
    else:
        vd = bd = (torch.bfloat16, torch.int16, torch.uint16)
    dev = _check_operands(rowptr, colind, vals, B, C, M, K, N, vd, bd)
    ts = None if tuning is None else ctypes.byref(tuning._struct())
    _check(lib().spmm_csr_tuned_noalloc(dtype, _ptr(rowptr), _ptr(colind), _ptr(vals),
                                        _ptr(B), _ptr(C), M, K, N, ts,
                                        _stream_handle(dev, stream)),
           "spmm_csr_tuned_noalloc")


def spmm_csr_eb(dtype: int, rowptr, colind, vals, B, C, M: int, K: int,
                N: int, stream=None) -> None:
    """C = A * B by the element-balanced kernel (spmm_csr_eb)."""
    torch = _torch()
    if dtype == DTYPE_F32:
        vd = bd = (torch.float32,)
    else:
        vd = bd = (torch.bfloat16, torch.int16, torch.uint16)
    dev = _check_operands(rowptr, colind, vals, B, C, M, K, N, vd, bd)
    _check(lib().spmm_csr_eb(dtype, _ptr(rowptr), _ptr(colind), _ptr(vals), _ptr(B),
                             _ptr(C), M, K, N, _stream_handle(dev, stream)),
           "spmm_csr_eb")


def spmm(rowptr, colind, vals, B, M: int | None = None, stream=None):
    """Allocate C and compute C = A * B; the element type follows vals."""
    torch = _torch()
    K, N = B.shape
    M = rowptr.numel() - 1 if M is None else M
    C = torch.empty((M, N), dtype=torch.float32, device=B.device)
    if vals.dtype == torch.float32:
        spmm_csr_f32(rowptr, colind, vals, B, C, M, K, N, stream)
    else:
        spmm_csr_bf16in_f32acc(rowptr, colind, vals, B, C, M, K, N, stream)
    return C


def _check_sddmm(rowptr, colind, C, B, A, M, K, N, dtypes):
    torch = _torch()
    dev = A.device
    for name, t in {"rowptr": rowptr, "colind": colind, "C": C, "B": B, "A": A}.items():
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device != dev or dev.type != "cuda":
            raise ValueError(f"{name} must live on the same GPU as A")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if rowptr.dtype != torch.int32 or colind.dtype != torch.int32:
        raise TypeError("rowptr and colind must be int32")
    if C.dtype not in dtypes or B.dtype not in dtypes:
        raise TypeError(f"C and B must be one of {dtypes}")
    if A.dtype != torch.float32:
        raise TypeError("A must be float32")
    if rowptr.numel() != M + 1:
        raise ValueError("rowptr must hold M+1 entries")
    if C.numel() != M * N or B.numel() != K * N:
        raise ValueError("C must hold M*N and B K*N elements")
    if A.numel() > colind.numel():
        raise ValueError("A holds one value per stored entry: at most len(colind)")
    return dev


def sddmm_csr_f32(rowptr, colind, C, B, A, M: int, K: int, N: int,
                  stream=None) -> None:
    """A[p - rowptr[0]] = <C_i, B_colind[p]> on the CSR pattern, fp32
    (sddmm_csr_f32).  nnz is len(A), which must be rowptr[M] - rowptr[0]."""
    torch = _torch()
    dev = _check_sddmm(rowptr, colind, C, B, A, M, K, N, (torch.float32,))
    _check(lib().sddmm_csr_f32(_ptr(rowptr), _ptr(colind), _ptr(C), _ptr(B),
                               _ptr(A), M, K, N, A.numel(),
                               _stream_handle(dev, stream)), "sddmm_csr_f32")


def sddmm_csr_bf16in_f32acc(rowptr, colind, C, B, A, M: int, K: int, N: int,
                            stream=None) -> None:
    """SDDMM with bf16 C and B (torch.bfloat16 or int16/uint16 bits), fp32
    accumulation and output (sddmm_csr_bf16in_f32acc)."""
    torch = _torch()
    bf = (torch.bfloat16, torch.int16, torch.uint16)
    dev = _check_sddmm(rowptr, colind, C, B, A, M, K, N, bf)
    _check(lib().sddmm_csr_bf16in_f32acc(_ptr(rowptr), _ptr(colind), _ptr(C),
                                         _ptr(B), _ptr(A), M, K, N, A.numel(),
                                         _stream_handle(dev, stream)),
           "sddmm_csr_bf16in_f32acc")


def sddmm(rowptr, colind, C, B, stream=None):
    """Allocate A and compute the SDDMM values; the element type follows C.
    rowptr[0] must be 0 (len(colind) entries)."""
    torch = _torch()
    M, N = C.shape
    K = B.shape[0]
    A = torch.empty(colind.numel(), dtype=torch.float32, device=C.device)
    if C.dtype == torch.float32:
        sddmm_csr_f32(rowptr, colind, C, B, A, M, K, N, stream)
    else:
        sddmm_csr_bf16in_f32acc(rowptr, colind, C, B, A, M, K, N, stream)
    return A


def _check_fusedmm(rowptr, colind, C, B, D, E, M, K, N, nnz, in_types):
    torch = _torch()
    dev = E.device
    for name, t in {"rowptr": rowptr, "colind": colind, "C": C, "B": B, "D": D,
                    "E": E}.items():
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device != dev or dev.type != "cuda":
            raise ValueError(f"{name} must live on the same GPU as E")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if rowptr.dtype != torch.int32 or colind.dtype != torch.int32:
        raise TypeError("rowptr and colind must be int32")
    for name, t in {"C": C, "B": B, "D": D}.items():
        if t.dtype not in in_types:
            raise TypeError(f"{name} must be one of {in_types}")
    if E.dtype != torch.float32:
        raise TypeError("E must be float32")
    if rowptr.numel() != M + 1:
        raise ValueError("rowptr must hold M+1 entries")
    if C.numel() != M * N or B.numel() != K * N or D.numel() != K * N or E.numel() != M * N:
        raise ValueError("C and E must hold M*N, B and D K*N elements")
    if nnz < 0 or nnz > colind.numel():
        raise ValueError("nnz must be in [0, len(colind)]")
    return dev


def fusedmm_csr_f32(rowptr, colind, C, B, D, E, M: int, K: int, N: int,
                    nnz: int, stream=None) -> None:
    """E_i = sum_p <C_i, B_colind[p]> D_colind[p] over the CSR pattern, fp32
    (fusedmm_csr_f32).  nnz must be rowptr[M] - rowptr[0]."""
    torch = _torch()
    dev = _check_fusedmm(rowptr, colind, C, B, D, E, M, K, N, nnz, (torch.float32,))
    _check(lib().fusedmm_csr_f32(_ptr(rowptr), _ptr(colind), _ptr(C), _ptr(B),
                                 _ptr(D), _ptr(E), M, K, N, nnz,
                                 _stream_handle(dev, stream)), "fusedmm_csr_f32")


def fusedmm_csr_bf16in_f32acc(rowptr, colind, C, B, D, E, M: int, K: int,
                              N: int, nnz: int, stream=None) -> None:
    """FusedMM with bf16 C, B and D (torch.bfloat16 or int16/uint16 bits),
    fp32 values, accumulation and E (fusedmm_csr_bf16in_f32acc)."""
    torch = _torch()
    bf = (torch.bfloat16, torch.int16, torch.uint16)
    dev = _check_fusedmm(rowptr, colind, C, B, D, E, M, K, N, nnz, bf)
    _check(lib().fusedmm_csr_bf16in_f32acc(_ptr(rowptr), _ptr(colind), _ptr(C),
                                           _ptr(B), _ptr(D), _ptr(E), M, K, N, nnz,
                                           _stream_handle(dev, stream)),
           "fusedmm_csr_bf16in_f32acc")


def fusedmm(rowptr, colind, C, B, D, stream=None):
    """Allocate E and compute FusedMM; the element type follows C
    (rowptr[0] must be 0)."""
    torch = _torch()
    M, N = C.shape
    K = B.shape[0]
    E = torch.empty((M, N), dtype=torch.float32, device=C.device)
    if C.dtype == torch.float32:
        fusedmm_csr_f32(rowptr, colind, C, B, D, E, M, K, N, colind.numel(), stream)
    else:
        fusedmm_csr_bf16in_f32acc(rowptr, colind, C, B, D, E, M, K, N,
                                  colind.numel(), stream)
    return E


def resolve_tuning(dtype: int, N: int, tuning: Tuning | None = None, K: int = 0) -> Tuning:
    """Thresholds a call with this dtype, K and N would use (host only)."""
    out = _TuningStruct()
    ts = None if tuning is None else ctypes.byref(tuning._struct())
    _check(lib().spmm_resolve_tuning(dtype, K, N, ts, ctypes.byref(out)),
           "spmm_resolve_tuning")
    return Tuning(out.short_max, out.medium_max, out.chunk_nnz, out.hub_min, out.slab_rows)


def plan_export(rowptr, resolved: Tuning, colind=None, K: int = 0,
                cap: int | None = None, stream=None) -> dict:
    """Run only the planning pass on device rowptr (and colind, for the hub
    chunks) and return the plan as numpy arrays (synchronises the stream).
    With cap=None the counts are read first and the arrays sized to hold the
    whole plan."""
    import numpy as np
    M = rowptr.numel() - 1
    ts = resolved._struct()
    handle = _stream_handle(rowptr.device, stream)
    counts = np.zeros(6, dtype=np.int64)
    cptr = None if colind is None else _ptr(colind)
    if cap is None:
        _check(lib().spmm_plan_export(_ptr(rowptr), cptr, M, K, ctypes.byref(ts), handle, 0,
                                      counts.ctypes.data, None, None, None, None, None),
               "spmm_plan_export")
        cap = int(counts[1:].max()) if M > 0 else 0
    cap_rows = max(cap, 1)
    medium = np.zeros(cap_rows, dtype=np.int32)
    long_rows = np.zeros((cap_rows, 3), dtype=np.int32)
    chunks = np.zeros((cap_rows, 4), dtype=np.int32)
    hubs = np.zeros(cap_rows, dtype=np.int32)
    hub_chunks = np.zeros((cap_rows, 4), dtype=np.int32)
    _check(lib().spmm_plan_export(_ptr(rowptr), cptr, M, K, ctypes.byref(ts), handle, cap,
                                  counts.ctypes.data, medium.ctypes.data,
                                  long_rows.ctypes.data, chunks.ctypes.data,
                                  hubs.ctypes.data, hub_chunks.ctypes.data),
           "spmm_plan_export")
    n_short, n_med, n_long, n_ch, n_hub, n_hch = (int(x) for x in counts)
    return {
        "n_short": n_short, "n_medium": n_med, "n_long": n_long, "n_chunks": n_ch,
        "n_hub": n_hub, "n_hub_chunks": n_hch,
        "medium_rows": medium[:min(n_med, cap)],
        "long_rows": long_rows[:min(n_long, cap)],
        "chunks": chunks[:min(n_ch, cap)],
        "hub_rows": hubs[:min(n_hub, cap)],
        "hub_chunks": hub_chunks[:min(n_hch, cap)],
    }


def timing_enable(on: bool = True) -> None:
    _check(lib().spmm_timing_enable(1 if on else 0), "spmm_timing_enable")


def timing_read() -> tuple[float, float, int]:
    """(0.0, call ms, calls) summed over the calls since the last read."""
    p = ctypes.c_double()
    w = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().spmm_timing_read(ctypes.byref(p), ctypes.byref(w), ctypes.byref(n)),
           "spmm_timing_read")
    return p.value, w.value, n.value


def stream_faults(stream=None) -> int:
    """Items left undone because a plan entry never became visible, on
    `stream` (default: torch's current stream), since the last query."""
    n = ctypes.c_int64()
    _check(lib().spmm_stream_faults(_stream_handle(None, stream), ctypes.byref(n)),
           "spmm_stream_faults")
    return n.value


def debug_set_wait_polls(polls: int) -> None:
    """Test hook: calls enqueued afterwards poll at most `polls` times for
    each plan entry (0: give up at once); a negative value restores the
    default bound."""
    _check(lib().spmm_debug_set_wait_polls(int(polls)), "spmm_debug_set_wait_polls")


def stream_release(stream=None) -> None:
    """Free the scratch the library keeps for `stream` (default: torch's
    current stream) after the calls already enqueued on it, and wait for
    the stream; call before the stream is destroyed."""
    _check(lib().spmm_stream_release(_stream_handle(None, stream)),
           "spmm_stream_release")
