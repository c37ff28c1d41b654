"""GPU parity: the HIP library, called through its C ABI, against the CPU
oracle on the same seeded inputs.  Conversions and indices must match
bit for bit; floating-point outputs within the per-output tolerance
|got - ref| <= 1e-5 * scale + 1e-30 (fp32) or 2e-2 * scale (bf16 BSR)."""
import json
import os

import numpy as np
import pytest
import torch

import gen
import oracle
import spmm_csr_spmv_amd as sp
from gpu_util import BINS, TOL_BF16, assert_close, dev, gpu_csr, host, say

pytestmark = pytest.mark.gpu


def small_cases():
    return {
        "uniform4096": lambda: gen.uniform_rows_coo(seed=0),
        "ragged_dups": lambda: gen.ragged_coo(700, 500, seed=1, max_len=40, dup_frac=0.15),
        "ragged_long": lambda: gen.ragged_coo(1500, 9000, seed=2, max_len=30, long_rows=(300, 5000, 9000, 2048, 257)),
        "wide_m_ne_n": lambda: gen.ragged_coo(90, 20000, seed=3, max_len=600, empty_frac=0.3),
        "tall_m_ne_n": lambda: gen.ragged_coo(20000, 70, seed=4, max_len=12, empty_frac=0.5),
        "all_empty": lambda: gen.Coo(37, 11, np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros(0, np.float32)),
        "one_row": lambda: gen.ragged_coo(1, 50000, seed=5, max_len=1, long_rows=(40000,), empty_frac=0.0),
    }


_cache = {}


def case(name):
    if name not in _cache:
        coo = small_cases()[name]()
        rp, c, v = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
        cp, ri, cv = oracle.csr_to_csc(coo.m, coo.n, rp, c, v)
        _cache[name] = (coo, (rp, c, v), (cp, ri, cv))
    return _cache[name]


# ------------------------------------------------------------------ the page's example
@pytest.fixture(scope="module")
def five(golden_dir):
    with open(os.path.join(golden_dir, "five_by_five.json")) as f:
        g = json.load(f)
    v = g["value_of"]
    g["coo_valf"] = np.array([v[s] for s in g["coo_val"]], np.float32)
    g["csr_valf"] = np.array([v[s] for s in g["csr_val"]], np.float32)
    return g


@pytest.mark.parametrize("bins", list(BINS))
def test_five_by_five_exact(five, bins):
    say("five_by_five", bins)
    p = np.random.default_rng(7).permutation(8)
    rp, c, v = sp.csr_build_from_coo(5, 5, dev(np.array(five["coo_row"], np.int32)[p]),
                                     dev(np.array(five["coo_col"], np.int32)[p]), dev(five["coo_valf"][p]))
    assert host(rp).tolist() == five["csr_row_ptr"]
    assert host(c).tolist() == five["csr_col"]
    assert host(v).tolist() == five["csr_valf"].tolist()
    cp, ri, cv = sp.csr_to_csc(5, 5, rp, c, v)
    assert host(cp).tolist() == [0, 2, 3, 5, 6, 8]
    assert host(ri).tolist() == [0, 2, 1, 0, 3, 2, 2, 4]
    assert host(cv).tolist() == [1, 4, 3, 2, 7, 5, 6, 8]
    plan = sp.Plan(5, 5, rp, c, v, csc=(cp, ri, cv), **BINS[bins])
    x = dev(np.arange(1, 6, dtype=np.float32))
    y = torch.full((5,), float("nan"), device="cuda")
    sp.spmv(plan, 1.0, x, 0.0, y)
    assert host(y).tolist() == [7, 6, 54, 21, 40]
    z = torch.full((5,), float("nan"), device="cuda")
    sp.spmv_t(plan, 1.0, x, 0.0, z)
    assert host(z).tolist() == [13, 6, 30, 15, 58]
    assert float(np.dot(host(z), np.arange(1, 6))) == float(np.dot(np.arange(1, 6), host(y))) == 465.0


# ------------------------------------------------------------------ conversions
@pytest.mark.parametrize("name", list(small_cases()))
def test_conversions_bit_exact(name):
    say("conversions", name)
    coo, (rp, c, v), (cp, ri, cv) = case(name)
    g_rp, g_c, g_v = gpu_csr(coo)
    np.testing.assert_array_equal(host(g_rp), rp)
    np.testing.assert_array_equal(host(g_c), c)
    np.testing.assert_array_equal(host(g_v).view(np.uint32), v.view(np.uint32))
    g_cp, g_ri, g_cv = sp.csr_to_csc(coo.m, coo.n, g_rp, g_c, g_v)
    np.testing.assert_array_equal(host(g_cp), cp)
    np.testing.assert_array_equal(host(g_ri), ri)
    np.testing.assert_array_equal(host(g_cv).view(np.uint32), cv.view(np.uint32))
    # round trip: the CSC read as the CSR of A^T, transposed again, is the CSR of A
    b_rp, b_c, b_v = sp.csr_to_csc(coo.n, coo.m, g_cp, g_ri, g_cv)
    np.testing.assert_array_equal(host(b_rp), rp)
    np.testing.assert_array_equal(host(b_c), c)


def test_build_rejects_out_of_range_indices():
    say("bad indices")
    row = np.array([0, 1, 5], np.int32)
    col = np.array([0, 1, 1], np.int32)
    val = np.ones(3, np.float32)
    with pytest.raises(sp.SparseError) as e:
        sp.csr_build_from_coo(4, 4, dev(row), dev(col), dev(val))
    assert e.value.code == 3
    with pytest.raises(sp.SparseError) as e:
        sp.csr_build_from_coo(4, 4, dev(np.array([0, 1, 2], np.int32)), dev(np.array([0, -1, 2], np.int32)), dev(val))
    assert e.value.code == 3


# ------------------------------------------------------------------ SpMV / SpMV^T
AB = [(1.0, 0.0), (1.0, -0.75), (-2.5, 1.5), (0.0, 2.0)]


def _plan(name, bins, max_N=1):
    coo, (rp, c, v), (cp, ri, cv) = case(name)
    g = (dev(rp), dev(c), dev(v))
    gt = (dev(cp), dev(ri), dev(cv))
    return coo, sp.Plan(coo.m, coo.n, *g, csc=gt, max_N=max_N, **BINS[bins])


@pytest.mark.parametrize("bins", list(BINS))
@pytest.mark.parametrize("name", list(small_cases()))
def test_spmv_and_transpose(name, bins):
    say("spmv", name, bins)
    coo, (rp, c, v), (cp, ri, cv) = case(name)
    _, plan = _plan(name, bins)
    x = gen.dense_vector(coo.n, 11)
    u = gen.dense_vector(coo.m, 12)
    for alpha, beta in AB:
        y0 = gen.dense_vector(coo.m, 13)
        z0 = gen.dense_vector(coo.n, 14)
        y = dev(y0) if beta != 0.0 else torch.full((coo.m,), float("nan"), device="cuda")
        sp.spmv(plan, alpha, dev(x), beta, y)
        ref, scale = oracle.spmv(rp, c, v, x, alpha, beta, y0)
        assert_close(host(y), ref, scale, what="spmv %s %s a=%g b=%g" % (name, bins, alpha, beta))
        z = dev(z0) if beta != 0.0 else torch.full((coo.n,), float("nan"), device="cuda")
        sp.spmv_t(plan, alpha, dev(u), beta, z)
        ref_t, scale_t = oracle.spmv(cp, ri, cv, u, alpha, beta, z0)
        assert_close(host(z), ref_t, scale_t, what="spmv_t %s %s a=%g b=%g" % (name, bins, alpha, beta))


@pytest.mark.parametrize("bins", ["default", "all_split", "mixed_small", "sell", "ps4", "ps8_split", "xw8"])
def test_spmv_bitwise_deterministic(bins):
    say("determinism", bins)
    coo, _, _ = case("ragged_long")
    _, plan = _plan("ragged_long", bins)
    x = dev(gen.dense_vector(coo.n, 21))
    outs = []
    for _ in range(3):
        y = torch.zeros(coo.m, device="cuda")
        sp.spmv(plan, 1.0, x, 0.0, y)
        outs.append(host(y).view(np.uint32).copy())
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("name", ["uniform4096", "ragged_long", "tall_m_ne_n", "all_empty"])
def test_profile_matches_oracle(name):
    say("profile", name)
    coo, (rp, _, _), (cp, _, _) = case(name)
    _, plan = _plan(name, "default")
    for transposed, ptr in ((False, rp), (True, cp)):
        got = plan.profile(transposed)
        exp = oracle.row_profile(ptr)
        assert (got["p95"], got["p99"], got["max_len"], got["empty_rows"]) == (exp["p95"], exp["p99"], exp["max"],
                                                                               exp["empty"])
        for k in ("mean", "var", "cv"):
            assert got[k] == pytest.approx(exp[k], rel=1e-12, abs=1e-12)
        # every row is served by exactly one bin
        assert got["group_rows"] + got["wave_rows"] + got["block_rows"] + got["split_rows"] == ptr.size - 1
        assert got["group_nnz"] + got["wave_nnz"] + got["block_nnz"] + got["split_nnz"] == ptr[-1]


@pytest.mark.parametrize("opts", [dict(use_sell=0, col_panels=4), dict(use_sell=0, x_window_bits=10)])
def test_panels_with_concentrated_columns(opts):
    """Forced panels (or x windows) on a matrix whose columns all sit in the
    first panel (the others hold no entries, only zero row sums), then on
    spread columns: both stay exact."""
    say("panels / windows, concentrated and spread columns", opts)
    rng = np.random.default_rng(3)
    m, n = 20000, 100000
    row = np.repeat(np.arange(m, dtype=np.int32), 20)
    val = rng.uniform(-1, 1, size=row.size).astype(np.float32)
    x = gen.dense_vector(n, 5)
    for hi in (1000, n):
        col = rng.integers(0, hi, size=row.size).astype(np.int32)
        rp, c, v = oracle.coo_to_csr(m, n, row, col, val)
        plan = sp.Plan(m, n, dev(rp), dev(c), dev(v), **opts)
        prof = plan.profile()
        assert (prof["col_panels"], prof["x_window_bits"]) == (opts.get("col_panels", 0), opts.get("x_window_bits", 0))
        y = torch.zeros(m, device="cuda")
        sp.spmv(plan, 1.0, dev(x), 0.0, y)
        ref, scale = oracle.spmv(rp, c, v, x)
        assert_close(host(y), ref, scale, what="panels, columns below %d" % hi)


def test_sell_with_wide_column_offsets():
    """SELL stores int16 column offsets from the row when every column lies
    within 32767 of its row (all the small cases above) and int32 columns
    otherwise: a matrix whose columns reach 120000 away takes the second
    form, and both directions stay exact."""
    say("sell, wide column offsets")
    coo = gen.ragged_coo(3000, 120000, seed=9, max_len=40, empty_frac=0.1)
    rp, c, v = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
    assert np.abs(c.astype(np.int64) - np.repeat(np.arange(coo.m), np.diff(rp))).max() > 32767
    cp, ri, cv = oracle.csr_to_csc(coo.m, coo.n, rp, c, v)
    plan = sp.Plan(coo.m, coo.n, dev(rp), dev(c), dev(v), csc=(dev(cp), dev(ri), dev(cv)), use_sell=1, col_panels=0,
                   x_window_bits=0)
    assert plan.profile()["sell_slots"] > 0
    x = gen.dense_vector(coo.n, 3)
    u = gen.dense_vector(coo.m, 4)
    y0 = gen.dense_vector(coo.m, 5)
    y = dev(y0)
    sp.spmv(plan, 1.5, dev(x), -0.5, y)
    ref, scale = oracle.spmv(rp, c, v, x, 1.5, -0.5, y0)
    assert_close(host(y), ref, scale, what="sell wide spmv")
    z = torch.zeros(coo.n, device="cuda")
    sp.spmv_t(plan, 1.0, dev(u), 0.0, z)
    ref_t, scale_t = oracle.spmv(cp, ri, cv, u)
    assert_close(host(z), ref_t, scale_t, what="sell wide spmv_t")


def test_x_windows_profile_and_limits():
    """The x-window stream reports its width; an explicit width that needs
    more than 256 windows is refused, the automatic choice never is."""
    say("x windows: profile and window limit")
    coo, (rp, c, v), _ = case("wide_m_ne_n")  # 20000 columns
    g = (dev(rp), dev(c), dev(v))
    assert sp.Plan(coo.m, coo.n, *g, use_sell=0, x_window_bits=7).profile()["x_window_bits"] == 7
    with pytest.raises(sp.SparseError) as e:
        sp.Plan(coo.m, coo.n, *g, use_sell=0, x_window_bits=6)  # 313 windows
    assert e.value.code == 5
    assert sp.Plan(coo.m, coo.n, *g).profile()["x_window_bits"] == 0  # x of 80 KB: no stream


# ------------------------------------------------------------------ SpMM
@pytest.mark.parametrize("bins", ["default", "all_wave", "all_block", "all_split", "mixed_small"])
@pytest.mark.parametrize("N", [1, 3, 8, 32, 128, 264])
def test_spmm(N, bins):
    name = "ragged_long"
    say("spmm", name, N, bins)
    coo, (rp, c, v), _ = case(name)
    _, plan = _plan(name, bins, max_N=N)
    B = gen.dense_matrix(coo.n, N, 31)
    for alpha, beta in [(1.0, 0.0), (0.5, -1.25)]:
        C0 = gen.dense_matrix(coo.m, N, 32)
        C = dev(C0) if beta != 0.0 else torch.full((coo.m, N), float("nan"), device="cuda")
        sp.spmm(plan, alpha, dev(B), beta, C)
        ref, scale = oracle.spmm(rp, c, v, B, alpha, beta, C0)
        assert_close(host(C), ref, scale, what="spmm N=%d %s a=%g b=%g" % (N, bins, alpha, beta))


def test_spmm_n1_equals_spmv():
    say("spmm N=1 vs spmv")
    coo, _, _ = case("uniform4096")
    _, plan = _plan("uniform4096", "default")
    x = gen.dense_vector(coo.n, 41)
    y = torch.zeros(coo.m, device="cuda")
    sp.spmv(plan, 1.0, dev(x), 0.0, y)
    C = torch.zeros(coo.m, 1, device="cuda")
    sp.spmm(plan, 1.0, dev(x.reshape(-1, 1)), 0.0, C)
    # same entries, same row order: the group path sums in the same order
    ref, scale = oracle.spmv(*case("uniform4096")[1], x)
    assert_close(host(C)[:, 0], ref, scale)
    assert_close(host(y), ref, scale)


# ------------------------------------------------------------------ BSR
@pytest.mark.parametrize("mb,kb,N,density", [(3, 4, 64, 0.5), (8, 6, 128, 0.3), (5, 9, 192, 0.25),
                                             (16, 16, 512, 0.1), (4, 4, 256, 1.0), (6, 3, 128, 0.0),
                                             # long block rows: 94..96 half-block stages, every tail length
                                             (4, 48, 512, 0.98), (4, 47, 256, 1.0),
                                             # several column tiles per block row
                                             (3, 5, 768, 0.6), (2, 7, 1024, 1.0),
                                             # widths with a partial last 64-column tile
                                             (3, 4, 8, 0.5), (4, 5, 72, 0.6), (5, 3, 200, 0.4), (2, 6, 264, 1.0)])
def test_bsr_spmm(mb, kb, N, density):
    say("bsr", mb, kb, N, density)
    b = gen.block_sparse_bsr(mb=mb, kb=kb, bs=64, density=density, std=0.02, seed=mb * 100 + kb)
    B = gen.bf16_matrix(kb * 64, N, seed=3)
    rp, col, v64 = oracle.bsr_to_csr(mb, 64, b.brow_ptr, b.bcol, b.bval)
    for alpha, beta in [(1.0, 0.0), (-0.5, 2.0)]:
        C0 = gen.dense_matrix(mb * 64, N, 4)
        C = dev(C0) if beta != 0.0 else torch.full((mb * 64, N), float("nan"), device="cuda")
        sp.bsr_spmm(mb, kb, 64, dev(b.brow_ptr), dev(b.bcol), dev(b.bval.view(np.int16)),
                    dev(B.view(np.int16)), alpha, beta, C)
        ref, scale = oracle.spmm_bf16(rp, col, v64, B, alpha, beta, C0)
        got = host(C)
        assert_close(got, ref, scale, tol=TOL_BF16, what="bsr a=%g b=%g" % (alpha, beta))
        # fp32 accumulation of exact bf16 products: far inside the bf16 tolerance
        assert_close(got, ref, scale, tol=1e-5, what="bsr fp32-accumulation bound")


@pytest.mark.parametrize("N", [64, 128, 256, 512])
def test_bsr_out_of_range_columns(N):
    """Blocks whose column index lies outside [0, kb) contribute nothing."""
    say("bsr bad columns", N)
    mb, kb = 5, 6
    b = gen.block_sparse_bsr(mb=mb, kb=kb, bs=64, density=0.7, std=0.02, seed=77)
    bad = b.bcol.copy()
    rng = np.random.default_rng(5)
    hit = rng.random(bad.size) < 0.3
    bad[hit] = np.where(rng.random(int(hit.sum())) < 0.5, -1, kb + 3)
    keep = ~hit
    # reference: the same matrix with those blocks removed
    counts = np.array([keep[b.brow_ptr[i]:b.brow_ptr[i + 1]].sum() for i in range(mb)])
    rp_k = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    bval_k = np.ascontiguousarray(b.bval[keep])
    rp, col, v64 = oracle.bsr_to_csr(mb, 64, rp_k, b.bcol[keep], bval_k)
    B = gen.bf16_matrix(kb * 64, N, seed=4)
    C = torch.full((mb * 64, N), float("nan"), device="cuda")
    sp.bsr_spmm(mb, kb, 64, dev(b.brow_ptr), dev(bad), dev(b.bval.view(np.int16)), dev(B.view(np.int16)),
                1.0, 0.0, C)
    ref, scale = oracle.spmm_bf16(rp, col, v64, B, 1.0, 0.0, gen.dense_matrix(mb * 64, N, 4))
    assert_close(host(C), ref, scale, tol=1e-5, what="bsr with skipped blocks")
