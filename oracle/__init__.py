"""CPU oracle for CSR sparse x dense products (fp64) and for the row plan.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The HIP
library and its Python binding never import it, and it imports nothing from
them; the two share no code.

Pages cited:
  [IntelMax] "Performance Optimization of Deep Learning Sparse Matrix Kernels
             on Intel Max Series GPU"
  [Sgap]     "Sgap: Towards Efficient Sparse Tensor Algebra Compilation for GPU"
  [Multilevel] "Sparse Matrix-Matrix Multiplication on Multilevel Memory
             Architectures: Algorithms and Experiments"

Contents
  spmm_ref   -- C = A*B and the bound S = |A|*|B| in fp64 ([IntelMax], SpMM
                operation, Fig. 5 / Algorithm 2), computed by ``spmm_ref.c``.
  sddmm_ref  -- the SDDMM values A[p] = <C_i, B_j> on a CSR pattern and their
                bound ([IntelMax], SDDMM operation, Fig. 3 / Algorithm 1),
                computed by ``sddmm_ref.c``.
  fusedmm_ref -- E_i = sum_p <C_i, B_j> D_j over the pattern and its bound
                ([IntelMax], FusedMM operation, Fig. 6 / Algorithm 3),
                computed by ``sddmm_ref.c``.
  plan_ref   -- the row-binning plan: which rows are short, medium, long or
                hub rows, how long rows are cut into nnz chunks and hub rows
                into column-slab chunks (see its docstring).
  widen_bf16 -- exact bf16 -> float64 widening used by the oracle.

Every function here is pinned by ``tests/test_oracle_pins.py`` against values
fixed by the mathematics (dense brute force, exact integer products, a
hand-built worked example, invariants) rather than against itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spmm_ref.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_spmm.so")

F32 = 0
BF16 = 1

_SDDMM_SRC = os.path.join(_HERE, "sddmm_ref.c")
_SDDMM_LIB_PATH = os.path.join(_HERE, "liboracle_sddmm.so")

_lib = None
_sddmm_lib = None


def compile_oracle(src: str, out: str) -> str:
    """gcc a C oracle source into a shared library (-ffp-contract=off keeps
    every a*b + acc a separate multiply and add, so the fp64 results are
    reproducible)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile ``spmm_ref.c`` into ``liboracle_spmm.so`` and ``sddmm_ref.c``
    into ``liboracle_sddmm.so``; returns the first path."""
    for src, out in ((_SRC, _LIB_PATH), (_SDDMM_SRC, _SDDMM_LIB_PATH)):
        if force or not os.path.exists(out) or \
                os.path.getmtime(out) < os.path.getmtime(src):
            compile_oracle(src, out)
    return _LIB_PATH


def load_library(path: str):
    """Load an oracle shared library built from ``spmm_ref.c`` and declare
    its functions."""
    lib = ctypes.CDLL(path)
    lib.oracle_spmm.restype = ctypes.c_int
    lib.oracle_spmm.argtypes = [
        ctypes.c_int64, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p,
    ]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_set_num_threads.restype = None
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    return lib


def load_sddmm_library(path: str):
    """Load an oracle shared library built from ``sddmm_ref.c``."""
    lib = ctypes.CDLL(path)
    lib.oracle_sddmm.restype = ctypes.c_int
    lib.oracle_sddmm.argtypes = [
        ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p,
    ]
    lib.oracle_fusedmm.restype = ctypes.c_int
    lib.oracle_fusedmm.argtypes = [
        ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
    ]
    return lib


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = load_library(_LIB_PATH)
    return _lib


def _load_sddmm():
    global _sddmm_lib
    if _sddmm_lib is None:
        build(force=False)
        _sddmm_lib = load_sddmm_library(_SDDMM_LIB_PATH)
    return _sddmm_lib


def _same_kind(*arrays) -> int:
    kinds = {_kind_of(a) for a in arrays}
    if len(kinds) != 1:
        raise TypeError("dense operands must all be float32 or all bf16 bits")
    return kinds.pop()


def sddmm_ref(rowptr, colind, C, B, N: int, rows=None, library=None):
    """fp64 oracle for SDDMM on a CSR pattern.

    [IntelMax], SDDMM operation (Fig. 3, Algorithm 1): the entry p of row i
    at column j = colind[p] gets the dot product of row C_i (C is M x N)
    with row B_j (B is K x N; column j of B^T).

    Returns (A, S): float64 arrays with one value per stored entry -- all
    entries in CSR order (index p - rowptr[0]) when ``rows`` is None, else
    the entries of the listed rows packed in list order -- and the bound
    S[p] = sum_n |C[i,n]| |B[j,n]|.
    """
    lib = _load_sddmm() if library is None else library
    rowptr = np.ascontiguousarray(rowptr, dtype=np.int32)
    colind = np.ascontiguousarray(colind, dtype=np.int32)
    C = np.ascontiguousarray(C)
    B = np.ascontiguousarray(B)
    M = rowptr.shape[0] - 1
    if rows is None:
        rows_arr, count, off = None, M, None
        total = int(rowptr[-1]) - int(rowptr[0]) if M >= 0 else 0
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        count = rows_arr.shape[0]
        off = np.empty(count, dtype=np.int64)
        lens = rowptr[1:].astype(np.int64) - rowptr[:-1]
        total = int(lens[rows_arr].sum()) if count else 0
    A = np.empty(total, dtype=np.float64)
    S = np.empty(total, dtype=np.float64)
    rc = lib.oracle_sddmm(M, N, rowptr.ctypes.data, colind.ctypes.data,
                          _same_kind(C, B), C.ctypes.data, B.ctypes.data,
                          None if rows_arr is None else rows_arr.ctypes.data,
                          count, None if off is None else off.ctypes.data,
                          A.ctypes.data, S.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_sddmm rejected its arguments")
    return A, S


def fusedmm_ref(rowptr, colind, C, B, D, N: int, rows=None, library=None):
    """fp64 oracle for FusedMM on a CSR pattern.

    [IntelMax], FusedMM operation (Fig. 6, Algorithm 3): for each stored
    entry of row i (column j) in CSR order, its SDDMM value a = <C_i, B_j>
    is computed and a * D_j is added into E_i (D is K x N).

    Returns (E, T): float64 arrays of shape (len(rows) or M, N), and the
    bound T[i,n] = sum_p S[p] |D[j,n]| with S[p] the SDDMM bound.
    """
    lib = _load_sddmm() if library is None else library
    rowptr = np.ascontiguousarray(rowptr, dtype=np.int32)
    colind = np.ascontiguousarray(colind, dtype=np.int32)
    C = np.ascontiguousarray(C)
    B = np.ascontiguousarray(B)
    D = np.ascontiguousarray(D)
    M = rowptr.shape[0] - 1
    if rows is None:
        rows_arr, count = None, M
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        count = rows_arr.shape[0]
    E = np.empty((count, N), dtype=np.float64)
    T = np.empty((count, N), dtype=np.float64)
    rc = lib.oracle_fusedmm(M, N, rowptr.ctypes.data, colind.ctypes.data,
                            _same_kind(C, B, D), C.ctypes.data, B.ctypes.data,
                            D.ctypes.data,
                            None if rows_arr is None else rows_arr.ctypes.data,
                            count, E.ctypes.data, T.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_fusedmm rejected its arguments")
    return E, T


def num_threads() -> int:
    """Threads the oracle's row loop uses (OpenMP)."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for later oracle calls' row loop (the results do not depend
    on it; used to time the oracle on one core)."""
    _load().oracle_set_num_threads(int(n))


def _kind_of(arr: np.ndarray) -> int:
    if arr.dtype == np.float32:
        return F32
    if arr.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or bf16 bits (uint16), got {arr.dtype}")


def spmm_ref(rowptr, colind, vals, B, N: int, rows=None, with_bound: bool = True,
             library=None):
    """fp64 oracle: rows of C = A*B and of the bound S = |A|*|B|.

    [IntelMax], SpMM operation (Fig. 5, Algorithm 2): row C_i is the sum, over
    the stored entries of row i in CSR order, of value * B[col, :].

    rowptr, colind : int32 arrays (rowptr holds absolute offsets).
    vals, B        : float32 arrays, or uint16 arrays holding bf16 bits.
    B              : K x N, row-major (any shape whose flat layout is that).
    rows           : None for every row, or an int array of row ids (a sample).
    library        : a library from ``load_library`` (default: this oracle).
    Returns (C, S) as float64 arrays of shape (len(rows) or M, N); S is None
    when ``with_bound`` is False.
    """
    lib = _load() if library is None else library
    rowptr = np.ascontiguousarray(rowptr, dtype=np.int32)
    colind = np.ascontiguousarray(colind, dtype=np.int32)
    vals = np.ascontiguousarray(vals)
    B = np.ascontiguousarray(B)
    M = rowptr.shape[0] - 1
    if M < 0:
        raise ValueError("rowptr must hold M+1 entries")
    if rows is None:
        rows_arr = None
        count = M
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        count = rows_arr.shape[0]
    C = np.empty((count, N), dtype=np.float64)
    S = np.empty((count, N), dtype=np.float64) if with_bound else None
    rc = lib.oracle_spmm(
        M, N,
        rowptr.ctypes.data, colind.ctypes.data,
        _kind_of(vals), vals.ctypes.data,
        _kind_of(B), B.ctypes.data,
        None if rows_arr is None else rows_arr.ctypes.data, count,
        C.ctypes.data, None if S is None else S.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_spmm rejected its arguments")
    return C, S


def widen_bf16(bits) -> np.ndarray:
    """bf16 bit patterns -> float64, exactly (bits become the top half of a
    binary32 word)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def plan_ref(rowptr, short_max: int, medium_max: int, chunk_nnz: int,
             hub_min: int | None = None, slab_rows: int | None = None,
             K: int | None = None, colind=None) -> dict:
    """Row-binning plan, derived plainly on the CPU.

    The pages motivate two ways to hand out the work of a row: one worker per
    row, or the row's non-zeros divided among several workers ([Sgap], the
    survey of prior work: Yang et al. choose between an nnz-balanced and a
    row-split algorithm; the DA-SpMM points EB and RB).  [IntelMax] (SDDMM
    implementation) divides the nnzr non-zeros of a row equally among NT
    workers.  The plan below fixes that choice per row by its length:

      len_i = rowptr[i+1] - rowptr[i]
      short  : len_i <= short_max
      medium : short_max < len_i <= medium_max
      long   : medium_max < len_i <= H, cut into n_i = ceil(len_i / chunk_nnz)
               chunks; chunk k (0 <= k < n_i) covers positions
               [rowptr[i] + floor(k*len_i/n_i), rowptr[i] + floor((k+1)*len_i/n_i)),
               so the chunks tile the row in order and none exceeds chunk_nnz.
      hub    : len_i > H, where H = max(hub_min, medium_max) (no hub rows when
               hub_min is None).  A hub row is cut by columns instead: with
               n_slabs = ceil(K / slab_rows), hub chunk s (0 <= s < n_slabs)
               covers positions [b(s), b(s+1)), where b(s) is rowptr[i] plus
               the number of the row's entries whose column is below
               s * slab_rows, b(0) = rowptr[i] and b(n_slabs) = rowptr[i+1].
               For a row whose columns ascend, chunk s holds exactly its
               entries with columns in [s*slab_rows, (s+1)*slab_rows) -- the
               rows of B that one column slab holds ([Multilevel], the access
               pattern: row j of B is read once per non-zero in column j, so
               entries of many rows that fall in one slab reuse the same rows
               of B).  The bounds are stated for ascending rows only.

    Lists are in ascending row order; chunks are ordered by row, then by k;
    hub chunks slab-major: all hubs' chunks of slab 0 (in hub order), then
    slab 1, and so on.
    Returns a dict of int32 arrays:
      medium_rows [n_medium]
      long_rows   [n_long, 3]   (row, first chunk index, number of chunks)
      chunks      [n_chunks, 4] (row, p0, p1, index of the row in long_rows)
      hub_rows    [n_hub]
      hub_chunks  [n_hub * n_slabs, 4] (row, p0, p1, index of the row in hub_rows)
    plus the integer counts n_short, n_medium, n_long, n_chunks, n_hub,
    n_slabs (0 without hub rows).
    """
    if not (0 <= short_max <= medium_max) or chunk_nnz < 1:
        raise ValueError("need 0 <= short_max <= medium_max and chunk_nnz >= 1")
    rp = np.asarray(rowptr, dtype=np.int64)
    lengths = rp[1:] - rp[:-1]
    if hub_min is None:
        top = np.iinfo(np.int64).max
    else:
        if slab_rows is None or slab_rows < 1 or K is None or K < 1 or colind is None:
            raise ValueError("hub rows need slab_rows >= 1, K >= 1 and colind")
        top = max(int(hub_min), int(medium_max))
    is_short = lengths <= short_max
    is_medium = (lengths > short_max) & (lengths <= medium_max)
    is_long = (lengths > medium_max) & (lengths <= top)
    is_hub = lengths > top
    medium_rows = np.nonzero(is_medium)[0].astype(np.int32)
    long_ids = np.nonzero(is_long)[0]
    long_rows = []
    chunks = []
    for li, row in enumerate(long_ids):
        start = int(rp[row])
        length = int(lengths[row])
        n = -(-length // chunk_nnz)
        long_rows.append((int(row), len(chunks), n))
        for k in range(n):
            p0 = start + (k * length) // n
            p1 = start + ((k + 1) * length) // n
            chunks.append((int(row), p0, p1, li))
    hub_ids = np.nonzero(is_hub)[0]
    n_slabs = -(-int(K) // int(slab_rows)) if hub_min is not None else 0
    hub_chunks = []
    if hub_ids.size:
        cols = np.asarray(colind, dtype=np.int64)
        bounds = []                      # per hub: b(0) .. b(n_slabs)
        for row in hub_ids:
            start, end = int(rp[row]), int(rp[row + 1])
            row_cols = cols[start:end]
            b = [start]
            for s in range(1, n_slabs):
                b.append(start + int(np.count_nonzero(row_cols < s * slab_rows)))
            b.append(end)
            bounds.append(b)
        for s in range(n_slabs):
            for hi, row in enumerate(hub_ids):
                hub_chunks.append((int(row), bounds[hi][s], bounds[hi][s + 1], hi))
    return {
        "n_short": int(is_short.sum()),
        "n_medium": int(medium_rows.shape[0]),
        "n_long": len(long_rows),
        "n_chunks": len(chunks),
        "n_hub": int(hub_ids.shape[0]),
        "n_slabs": n_slabs,
        "medium_rows": medium_rows,
        "long_rows": np.array(long_rows, dtype=np.int32).reshape(-1, 3),
        "chunks": np.array(chunks, dtype=np.int32).reshape(-1, 4),
        "hub_rows": hub_ids.astype(np.int32),
        "hub_chunks": np.array(hub_chunks, dtype=np.int32).reshape(-1, 4),
    }
