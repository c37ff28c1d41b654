"""Seeded synthetic inputs for the sparse x dense products.

This module draws random inputs only; it holds none of the method's arithmetic
(no format conversion, no product).  CSR workloads are delivered as COO
triples, which is the load format the format survey page describes; turning
them into CSR is the job of the library (and, independently, of the oracle).

Random numbers come from numpy's PCG64 generator seeded per workload, so every
array is reproducible on any machine.  bf16 arrays are produced by rounding
fp32 draws to nearest-even on the bit pattern (stored as uint16).
"""
from .workloads import (  # noqa: F401
    Coo,
    Bsr,
    f32_to_bf16_bits,
    uniform_rows_coo,
    powerlaw_coo,
    stencil27_coo,
    lognormal_coo,
    block_sparse_bsr,
    block_sparse_coo,
    clustered_coo,
    skewed_windows_coo,
    bf16_matrix,
    ragged_coo,
    dense_vector,
    dense_matrix,
    shuffle_coo,
    CONFIGS,
)
