"""Inf and NaN in the dense operand, every product path, against the oracle.

Padding slots (SELL slices, x-window runs, panel chunks) must be skipped, never
multiplied by 0: 0 * Inf is NaN (「稀疏矩阵存储格式:COO、CSR、ELL、Hybrid 与块稀疏,SpMV
的容量与带宽账」 §四 marks padding as slots that hold no entry).  So outputs that
touch no special column must match the oracle within the fp32 tolerance, and
outputs that do must have the oracle's class: the same infinity, or NaN.
Special values sit at window and panel starts (the column a padding slot of
the x-window stream points at) and at scattered columns."""
import numpy as np
import pytest
import torch

import gen
import oracle
import spmm_csr_spmv_amd as sp
from gpu_util import BINS, assert_close, dev, host, say

pytestmark = pytest.mark.gpu

PATHS = ["default", "group", "all_wave", "all_block", "all_split", "mixed_small", "sell", "ps1", "ps4", "ps8_split",
         "xw8", "xw15"]


def _special(n, seed, starts=(256, 1 << 15)):
    """A vector U[-1,1] with +Inf, -Inf and NaN at window starts and scattered places."""
    v = gen.dense_vector(n, seed).astype(np.float32)
    rng = np.random.default_rng(seed + 1000)
    cols = set([0])
    for w in starts:
        cols.update(range(0, n, w))
    cols.update(rng.choice(n, size=min(n, 12), replace=False).tolist())
    cols = sorted(c for c in cols if c < n)
    kinds = np.array([np.inf, -np.inf, np.nan], np.float32)
    for k, c in enumerate(cols):
        v[c] = kinds[k % 3]
    return v


def check_class(got, ref, scale, what):
    """Finite reference outputs within tolerance; the others of the same class."""
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    scale = np.asarray(scale, np.float64).ravel()
    fin = np.isfinite(ref)
    assert_close(got[fin], ref[fin], scale[fin], what=what + " (finite outputs)")
    nan = np.isnan(ref)
    bad = np.flatnonzero(nan & ~np.isnan(got))
    assert bad.size == 0, "%s: %d outputs should be NaN, e.g. idx %s got %s" % (what, bad.size, bad[:5], got[bad[:5]])
    inf = np.isinf(ref)
    bad = np.flatnonzero(inf & (got != ref))
    assert bad.size == 0, "%s: %d outputs should be %s, e.g. idx %s got %s" % (what, bad.size, ref[bad[:1]], bad[:5],
                                                                               got[bad[:5]])
    return int((~fin).sum())


def _matrix():
    coo = gen.ragged_coo(2000, 60000, seed=21, max_len=50, long_rows=(900, 3000, 40000), dup_frac=0.02)
    rp, c, v = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
    cp, ri, cv = oracle.csr_to_csc(coo.m, coo.n, rp, c, v)
    return coo, (rp, c, v), (cp, ri, cv)


_m = {}


def matrix():
    if not _m:
        _m["a"] = _matrix()
    return _m["a"]


@pytest.mark.parametrize("path", PATHS)
def test_spmv_nonfinite_x(path):
    say("nonfinite spmv", path)
    coo, (rp, c, v), (cp, ri, cv) = matrix()
    plan = sp.Plan(coo.m, coo.n, dev(rp), dev(c), dev(v), csc=(dev(cp), dev(ri), dev(cv)), **BINS[path])
    x = _special(coo.n, 3)
    u = _special(coo.m, 4, starts=(256,))
    y = torch.full((coo.m,), float("nan"), device="cuda")
    sp.spmv(plan, 1.0, dev(x), 0.0, y)
    ref, scale = oracle.spmv(rp, c, v, x)
    hit = check_class(host(y), ref, scale, "spmv %s" % path)
    assert 0 < hit < coo.m
    z = torch.full((coo.n,), float("nan"), device="cuda")
    sp.spmv_t(plan, 1.0, dev(u), 0.0, z)
    ref_t, scale_t = oracle.spmv(cp, ri, cv, u)
    hit_t = check_class(host(z), ref_t, scale_t, "spmv_t %s" % path)
    assert 0 < hit_t < coo.n


@pytest.mark.parametrize("N", [3, 8, 16, 32])
@pytest.mark.parametrize("bins", ["default", "all_wave", "all_split", "mixed_small", "sweep8"])
def test_spmm_nonfinite_b(bins, N):
    say("nonfinite spmm", bins, N)
    coo, (rp, c, v), _ = matrix()
    plan = sp.Plan(coo.m, coo.n, dev(rp), dev(c), dev(v), max_N=N, **BINS[bins])
    B = gen.dense_matrix(coo.n, N, 7).astype(np.float32)
    rng = np.random.default_rng(8)
    for k, r in enumerate(rng.choice(coo.n, size=40, replace=False)):
        B[r, k % N] = (np.inf, -np.inf, np.nan)[k % 3]
    C = torch.full((coo.m, N), float("nan"), device="cuda")
    sp.spmm(plan, 1.0, dev(B), 0.0, C)
    ref, scale = oracle.spmm(rp, c, v, B)
    assert check_class(host(C), ref, scale, "spmm %s N=%d" % (bins, N)) > 0


@pytest.mark.parametrize("rowwise", [False, True], ids=["whole_blocks", "rows"])
@pytest.mark.parametrize("bs", [4, 64])
def test_bsr_spmv_nonfinite_x(bs, rowwise):
    """Blocks keep their explicit zeros, so 0 * Inf = NaN inside a stored block
    on both sides; columns past n of the padded last block column are never read."""
    say("nonfinite bsr spmv", bs)
    coo = gen.ragged_coo(1000, 1900, seed=5, max_len=30, empty_frac=0.1)
    rp, c, v = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
    brp, bcol, bval = oracle.csr_to_bsr(coo.m, coo.n, rp, c, v, bs)
    x = _special(coo.n, 11, starts=(512,))
    # x is read only below n: pad it with NaN to the block grid, outside the call's view
    xpad = np.full(((coo.n + bs - 1) // bs) * bs + 16, np.nan, np.float32)
    xpad[:coo.n] = x
    dx = dev(xpad)
    y = torch.full((coo.m,), float("nan"), device="cuda")
    sp.bsr_spmv(coo.m, coo.n, bs, dev(brp), dev(bcol), dev(bval), 1.0, dx[:coo.n], 0.0, y, rowwise=rowwise)
    ref, scale = oracle.bsr_spmv(coo.m, coo.n, bs, brp, bcol, bval, x)
    assert check_class(host(y), ref, scale, "bsr_spmv bs=%d" % bs) > 0


@pytest.mark.parametrize("N", [128, 512])
def test_bsr_spmm_nonfinite_b(N):
    say("nonfinite bsr spmm", N)
    mb, kb = 6, 7
    b = gen.block_sparse_bsr(mb=mb, kb=kb, bs=64, density=0.4, std=0.02, seed=17)
    B = gen.bf16_matrix(kb * 64, N, seed=5).copy()
    rng = np.random.default_rng(3)
    for k, (r, col) in enumerate(zip(rng.choice(kb * 64, size=12, replace=False), rng.choice(N, size=12))):
        B[r, col] = (0x7F80, 0xFF80, 0x7FC0)[k % 3]  # +Inf, -Inf, NaN in bf16
    rp, colx, v64 = oracle.bsr_to_csr(mb, 64, b.brow_ptr, b.bcol, b.bval)
    C = torch.full((mb * 64, N), float("nan"), device="cuda")
    sp.bsr_spmm(mb, kb, 64, dev(b.brow_ptr), dev(b.bcol), dev(b.bval.view(np.int16)), dev(B.view(np.int16)), 1.0,
                0.0, C)
    ref, scale = oracle.spmm_bf16(rp, colx, v64, B)
    assert check_class(host(C), ref, scale, "bsr_spmm N=%d" % N) > 0


@pytest.mark.parametrize("N", [4, 32, 128])
@pytest.mark.parametrize("path", ["window", "tasks"])
def test_wcsr_spmm_nonfinite_b(path, N):
    """Window tiles are dense: a row of the window without an entry at a
    compressed column holds a stored 0 there, so 0 * Inf = NaN on both sides
    (the oracle sums over the stored tile); padding columns (-1) are skipped,
    never read from B."""
    say("nonfinite wcsr spmm", path, N)
    coo = gen.skewed_windows_coo(m=700, n=30000, pool_median=40, pool_sigma=1.2, pool_max=3000, seed=9)
    rp, c, v = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
    wp, wc, vals = oracle.csr_to_wcsr(coo.m, coo.n, rp, c, v, 64, 8)
    B = gen.dense_matrix(coo.n, N, 7).astype(np.float32)
    rng = np.random.default_rng(9)
    used = np.unique(c)
    for k, r in enumerate(rng.choice(used, size=30, replace=False)):
        B[r, k % N] = (np.inf, -np.inf, np.nan)[k % 3]
    B[0, :] = np.nan  # row 0 of B: read only where column 0 is stored
    C = torch.full((coo.m, N), float("nan"), device="cuda")
    if path == "window":
        sp.wcsr_spmm(coo.m, coo.n, dev(wp), dev(wc), dev(vals), 1.0, dev(B), 0.0, C)
    else:
        t = sp.wcsr_tasks(coo.m, dev(wp), wc.size, task_cols=64)
        assert t.nslots > 0
        sp.wcsr_spmm_tasks(coo.m, coo.n, t, dev(wc), dev(vals), 1.0, dev(B), 0.0, C)
    ref, scale = oracle.wcsr_spmm(coo.m, 64, wp, wc, vals, B)
    assert check_class(host(C), ref, scale, "wcsr %s N=%d" % (path, N)) > 0
