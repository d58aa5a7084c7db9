"""MI355X (gfx950) CSR sparse x dense products, C = A * B.

Thin Python binding over the C ABI of ``libsdl_spmm.so`` (declared in
``include/spmm.h``).  The functions only marshal arguments -- device
pointers, sizes and the current torch stream -- into the library; every
step of the product runs in the library's HIP kernels.  PyTorch is used for
device memory and streams only.

The binding never falls back to anything else: if the shared library is not
built, importing the functions raises.
"""
from ._binding import (  # noqa: F401
    DTYPE_BF16,
    DTYPE_F32,
    SpmmError,
    Tuning,
    debug_set_wait_polls,
    fusedmm,
    fusedmm_csr_f32,
    fusedmm_csr_bf16in_f32acc,
    lib,
    lib_path,
    plan_export,
    resolve_tuning,
    sddmm,
    sddmm_csr_bf16in_f32acc,
    sddmm_csr_f32,
    spmm,
    spmm_csr_bf16in_f32acc,
    spmm_csr_eb,
    spmm_csr_f32,
    spmm_csr_tuned,
    spmm_csr_tuned_noalloc,
    status_string,
    stream_faults,
    stream_release,
    timing_enable,
    timing_read,
)
