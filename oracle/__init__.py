"""CPU oracle for the sparse x dense products -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (``spmm_csr_spmv_amd``)
never imports it, and it never imports the product path: the two share no code.

The arithmetic lives in ``oracle.c`` (plain single-threaded C loops, fp64
accumulation); this module only marshals numpy arrays into it.
"""
from .oracle import (  # noqa: F401
    OracleError,
    build,
    coo_to_csr,
    csr_to_csc,
    spmv,
    spmv_t_scatter,
    spmm,
    bf16_to_float64,
    bsr_to_csr,
    spmm_bf16,
    bsr_spmm_direct,
    csr_to_bsr,
    f32_to_bf16,
    bsr_spmv,
    csr_to_wcsr,
    wcsr_spmm,
    wcsr_tasks,
    row_profile,
    sell_build,
    sell_spmv,
    library_path,
)
