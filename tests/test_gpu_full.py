"""GPU parity at the full workload sizes, in the plan configuration bench.py
times (default options).  Conversions are compared with the oracle bit for
bit over the whole matrix; products over every row where the single-threaded
oracle finishes in seconds, else over sampled rows (always including the
longest rows)."""
import numpy as np
import pytest
import torch

import gen
import oracle
import spmm_csr_spmv_amd as sp
from gpu_util import TOL_BF16, assert_close, dev, host, say

pytestmark = pytest.mark.gpu


def _csr_both(coo):
    say("oracle coo_to_csr", coo.m, coo.nnz)
    ref = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
    say("gpu csr_build_from_coo")
    got = sp.csr_build_from_coo(coo.m, coo.n, dev(coo.row), dev(coo.col), dev(coo.val))
    return ref, got


@pytest.fixture(scope="module")
def powerlaw():
    coo = gen.powerlaw_coo(seed=0)
    ref, got = _csr_both(coo)
    return coo, ref, got


def test_powerlaw_conversion_bit_exact(powerlaw):
    coo, (rp, c, v), (g_rp, g_c, g_v) = powerlaw
    np.testing.assert_array_equal(host(g_rp), rp)
    np.testing.assert_array_equal(host(g_c), c)
    np.testing.assert_array_equal(host(g_v).view(np.uint32), v.view(np.uint32))


@pytest.mark.parametrize("opts,path", [(dict(), (15, 0)), (dict(col_panels=8), (0, 8)),
                                       (dict(use_sell=0, col_panels=1, x_window_bits=0), (0, 1)),
                                       (dict(use_sell=0, col_panels=0, x_window_bits=0), (0, 0))],
                         ids=["default_x_windows", "panels8", "entry_balanced_stream", "row_bins"])
def test_powerlaw_spmv_all_rows(powerlaw, opts, path):
    coo, (rp, c, v), (g_rp, g_c, g_v) = powerlaw
    say("powerlaw plan", opts)
    plan = sp.Plan(coo.m, coo.n, g_rp, g_c, g_v, **opts)
    prof = plan.profile()
    # the default picks the x-window stream for these scattered columns
    assert (prof["x_window_bits"], prof["col_panels"]) == path
    exp = oracle.row_profile(rp)
    assert (prof["p95"], prof["p99"], prof["max_len"], prof["empty_rows"]) == (exp["p95"], exp["p99"], exp["max"],
                                                                               exp["empty"])
    assert prof["split_rows"] >= 4  # the planted hub rows take the split path
    x = gen.dense_vector(coo.n, 0, 1)
    y = torch.full((coo.m,), float("nan"), device="cuda")
    say("gpu spmv")
    sp.spmv(plan, 1.0, dev(x), 0.0, y)
    got = host(y)
    say("oracle spmv")
    ref, scale = oracle.spmv(rp, c, v, x)
    ratio = assert_close(got, ref, scale, what="powerlaw spmv")
    say("max error / scale", ratio)
    # beta != 0 with the same plan
    y0 = gen.dense_vector(coo.m, 0, 7)
    y = dev(y0)
    sp.spmv(plan, -0.5, dev(x), 1.25, y)
    ref, scale = oracle.spmv(rp, c, v, x, -0.5, 1.25, y0)
    assert_close(host(y), ref, scale, what="powerlaw spmv axpby")
    # two launches give identical bits
    y2 = dev(y0)
    sp.spmv(plan, -0.5, dev(x), 1.25, y2)
    assert torch.equal(y, y2)


@pytest.fixture(scope="module")
def stencil():
    coo = gen.stencil27_coo(seed=0)
    assert coo.nnz == 478 ** 3 == 109215352
    ref, got = _csr_both(coo)
    return coo, ref, got


def test_stencil_conversions_bit_exact(stencil):
    coo, (rp, c, v), (g_rp, g_c, g_v) = stencil
    np.testing.assert_array_equal(host(g_rp), rp)
    np.testing.assert_array_equal(host(g_c), c)
    np.testing.assert_array_equal(host(g_v).view(np.uint32), v.view(np.uint32))
    say("oracle csr_to_csc")
    cp, ri, cv = oracle.csr_to_csc(coo.m, coo.n, rp, c, v)
    say("gpu csr_to_csc")
    g_cp, g_ri, g_cv = sp.csr_to_csc(coo.m, coo.n, g_rp, g_c, g_v)
    np.testing.assert_array_equal(host(g_cp), cp)
    np.testing.assert_array_equal(host(g_ri), ri)
    np.testing.assert_array_equal(host(g_cv).view(np.uint32), cv.view(np.uint32))


@pytest.mark.parametrize("opts", [dict(), dict(use_sell=0)], ids=["default_sell", "row_bins"])
def test_stencil_operator_pair(stencil, opts):
    """u <- A v - alpha u through the CSR, then v <- A^T u - beta v through the CSC."""
    coo, (rp, c, v), (g_rp, g_c, g_v) = stencil
    csc = sp.csr_to_csc(coo.m, coo.n, g_rp, g_c, g_v)
    cp, ri, cv = (host(t) for t in csc)
    plan = sp.Plan(coo.m, coo.n, g_rp, g_c, g_v, csc=csc, **opts)
    assert (plan.profile()["sell_slots"] > 0) == (not opts)
    u0 = gen.dense_vector(coo.m, 0, 2)
    v0 = gen.dense_vector(coo.n, 0, 3)
    alpha, beta = np.random.default_rng(5).uniform(0.5, 2.0, size=2)
    u = dev(u0)
    v_ = dev(v0)
    say("gpu pair")
    sp.spmv(plan, 1.0, v_, -float(alpha), u)
    u1 = host(u)
    ref, scale = oracle.spmv(rp, c, v, v0, 1.0, -float(alpha), u0)
    assert_close(u1, ref, scale, what="u <- A v - alpha u")
    sp.spmv_t(plan, 1.0, u, -float(beta), v_)
    ref_t, scale_t = oracle.spmv(cp, ri, cv, u1, 1.0, -float(beta), v0)
    assert_close(host(v_), ref_t, scale_t, what="v <- A^T u - beta v")


@pytest.fixture(scope="module")
def lognormal():
    coo = gen.lognormal_coo(seed=0)
    ref, got = _csr_both(coo)
    return coo, ref, got


@pytest.mark.parametrize("N", [8, 32, 128])
def test_spmm_lognormal_all_rows(lognormal, N):
    coo, (rp, c, v), (g_rp, g_c, g_v) = lognormal
    if N == 8:
        np.testing.assert_array_equal(host(g_rp), rp)
        np.testing.assert_array_equal(host(g_c), c)
    plan = sp.Plan(coo.m, coo.n, g_rp, g_c, g_v, max_N=N)
    # N = 8 takes the phase-swept copy (B of 32 MiB in 512 KiB slices), wider N the row bins
    assert plan.profile()["spmm_phase_bits"] == (14 if N == 8 else 0)
    B = gen.dense_matrix(coo.n, N, 0)
    dB = dev(B)
    C = torch.full((coo.m, N), float("nan"), device="cuda")
    say("gpu spmm", N)
    sp.spmm(plan, 1.0, dB, 0.0, C)
    got = host(C)
    say("oracle spmm", N)
    ref, scale = oracle.spmm(rp, c, v, B)
    assert_close(got, ref, scale, what="spmm N=%d" % N)
    del ref, scale, got
    # beta != 0 over every row with the same plan
    C0 = gen.dense_matrix(coo.m, N, 5)
    C = dev(C0)
    say("gpu spmm axpby", N)
    sp.spmm(plan, -0.75, dB, 1.5, C)
    ref, scale = oracle.spmm(rp, c, v, B, -0.75, 1.5, C0)
    assert_close(host(C), ref, scale, what="spmm axpby N=%d" % N)


def test_bsr_full_heavy_rows():
    b = gen.block_sparse_bsr(seed=0)
    N = 512
    B = gen.bf16_matrix(b.kb * b.bs, N, seed=0)
    C = torch.full((b.mb * b.bs, N), float("nan"), device="cuda")
    say("gpu bsr", b.nnzb)
    sp.bsr_spmm(b.mb, b.kb, b.bs, dev(b.brow_ptr), dev(b.bcol), dev(b.bval.view(np.int16)), dev(B.view(np.int16)),
                1.0, 0.0, C)
    counts = np.diff(b.brow_ptr)
    # every row of the 8 heaviest block rows, plus 1024 sampled rows
    heavy = np.argsort(counts, kind="stable")[-8:]
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([(heavy[:, None] * 64 + np.arange(64)[None, :]).ravel(),
                                     rng.choice(b.mb * b.bs, 1024, replace=False)]))
    rp, col, v64 = oracle.bsr_to_csr(b.mb, b.bs, b.brow_ptr, b.bcol, b.bval)
    ref, scale = oracle.spmm_bf16(rp, col, v64, B, rows=rows)
    got = host(C)[rows]
    assert_close(got, ref, scale, tol=TOL_BF16, what="bsr full")
    assert_close(got, ref, scale, tol=1e-5, what="bsr full, fp32 accumulation bound")
    direct = oracle.bsr_spmm_direct(b.mb, b.bs, b.brow_ptr, b.bcol, b.bval, B, rows=rows[:16])
    np.testing.assert_allclose(direct, ref[:16], rtol=1e-12, atol=1e-12)
