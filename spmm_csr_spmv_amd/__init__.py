"""Sparse x dense products on AMD Instinct MI355X (gfx950).

Python binding of libspmm_csr_spmv.so (C ABI in include/spmm_csr_spmv.h):
CSR SpMV y = alpha A x + beta y, its transpose through a one-time CSC,
CSR SpMM C = alpha A B + beta C, BSR SpMM on MFMA (bf16 in, fp32
accumulate), CSR -> BSR with a fill-ratio gate, BSR SpMV, windowed rows
(WCSR) with a windowed SpMM on MFMA, and a tuning cache.  All
arithmetic runs in the library's HIP kernels; this package only marshals
torch tensors into the C calls.  There is no CPU fallback:
without the built library every call raises.
"""
from ._binding import (  # noqa: F401
    DEFAULT_CANDIDATES,
    EXPORTS,
    LIB_PATH,
    Plan,
    PlanView,
    SparseError,
    autotune_spmv,
    bsr_spmm,
    bsr_spmv,
    csr_build_from_coo,
    csr_build_from_coo_noalloc,
    csr_to_bsr,
    csr_to_csc,
    csr_to_wcsr,
    wcsr_spmm,
    wcsr_spmm_tasks,
    wcsr_tasks,
    WcsrTasks,
    lib,
    options_dict,
    plan_options,
    sp_plan_create,
    sp_version,
    spmm,
    spmv,
    spmv_t,
    status_string,
    tune_cache_clear,
    tune_cache_lookup,
    tune_cache_size,
    tune_cache_store,
    sp_dispatch_key,
)
