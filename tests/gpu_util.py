"""Helpers shared by the GPU parity tests (no arithmetic of the method here)."""
import sys

import numpy as np
import torch

import spmm_csr_spmv_amd as sp

# Per-output tolerance for fp32 results: |got - ref| <= TOL * scale + 1e-30, where
# scale = |alpha| * sum |a_ij x_j| + |beta| * |y_old| is computed by the oracle.
TOL_F32 = 1e-5
# bf16 BSR: the same form with 2e-2.
TOL_BF16 = 2e-2

# Row-bin settings that force every non-empty row through one kernel, or mix
# all kernels at small sizes.
BINS = {
    "default": {},
    "group": dict(use_sell=0),
    "all_wave": dict(wave_min=0, block_min=2 ** 30, split_min=2 ** 30),
    "all_block": dict(wave_min=0, block_min=0, split_min=2 ** 30),
    "all_split": dict(wave_min=0, block_min=0, split_min=0, split_seg=16),
    "mixed_small": dict(group_nnz=64, wave_min=8, block_min=40, split_min=100, split_seg=32),
    "sell": dict(use_sell=1, sell_sigma=128),
    "no_xcd": dict(xcd_remap=0),
    # column-panel stream (every row up to the split length in one balanced stream)
    "ps1": dict(use_sell=0, col_panels=1),
    "ps2_split": dict(use_sell=0, col_panels=2, wave_min=8, block_min=40, split_min=100, split_seg=32),
    "ps4": dict(use_sell=0, col_panels=4),
    "ps8_split": dict(use_sell=0, col_panels=8, wave_min=8, block_min=20, split_min=40, split_seg=16),
    # x-window stream (products with x windows in LDS, then row sums in CSR order)
    "xw8": dict(use_sell=0, x_window_bits=8),
    "xw15": dict(use_sell=0, x_window_bits=15),
    # phase-swept SpMM copy (SpMM with N in {4, 8, 16}; SpMV is unaffected)
    "sweep8": dict(spmm_phase_bits=8),
}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_close(got, ref, scale, tol=TOL_F32, what=""):
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    scale = np.asarray(scale, np.float64).ravel()
    assert got.shape == ref.shape
    err = np.abs(got - ref)
    bound = tol * scale + 1e-30
    bad = np.flatnonzero(~(err <= bound))
    assert bad.size == 0, "%s: %d of %d outputs outside tolerance; first idx %s got %s ref %s bound %s" % (
        what, bad.size, got.size, bad[:5], got[bad[:5]], ref[bad[:5]], bound[bad[:5]])
    ratio = err / np.maximum(scale, 1e-300)
    return float(ratio.max()) if ratio.size else 0.0


def gpu_csr(coo):
    return sp.csr_build_from_coo(coo.m, coo.n, dev(coo.row), dev(coo.col), dev(coo.val))
