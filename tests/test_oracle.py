"""Pins for the CPU oracle.  None of these expected values comes from the
oracle itself: they come from the worked example printed on the format-survey
page (tests/golden/five_by_five.json), from dense brute force in numpy / plain
Python loops, or from invariants that must hold for any correct
implementation.
"""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st, HealthCheck

import gen
import oracle


# --------------------------------------------------------------------------
# helpers that do NOT use the oracle
# --------------------------------------------------------------------------
def dense_from_coo(m, n, row, col, val):
    d = np.zeros((m, n), np.float64)
    np.add.at(d, (np.asarray(row), np.asarray(col)), np.asarray(val, np.float64))
    return d


def dense_from_csr(m, n, row_ptr, col, val):
    d = np.zeros((m, n), np.float64)
    for i in range(m):
        for p in range(row_ptr[i], row_ptr[i + 1]):
            d[i, col[p]] += float(val[p])
    return d


@pytest.fixture(scope="module")
def five(golden_dir):
    with open(os.path.join(golden_dir, "five_by_five.json")) as f:
        g = json.load(f)
    v = g["value_of"]
    g["coo_valf"] = np.array([v[s] for s in g["coo_val"]], np.float32)
    g["csr_valf"] = np.array([v[s] for s in g["csr_val"]], np.float32)
    # the dense matrix as the page describes it, row by row
    dense = np.zeros((g["m"], g["n"]))
    for i, entries in enumerate(g["rows_described"]):
        for c, s in entries:
            dense[i, c] = v[s]
    g["dense"] = dense
    return g


# --------------------------------------------------------------------------
# the page's worked example
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(6))
def test_five_coo_to_csr_matches_page(five, seed):
    rng = np.random.default_rng(seed)
    p = rng.permutation(8) if seed else np.arange(8)
    row = np.array(five["coo_row"])[p]
    col = np.array(five["coo_col"])[p]
    val = five["coo_valf"][p]
    rp, c, v = oracle.coo_to_csr(5, 5, row, col, val)
    assert rp.tolist() == five["csr_row_ptr"]
    assert c.tolist() == five["csr_col"]
    assert v.tolist() == five["csr_valf"].tolist()


def test_five_csc_matches_dense_columns(five):
    rp = np.array(five["csr_row_ptr"], np.int32)
    cp, ri, cv = oracle.csr_to_csc(5, 5, rp, np.array(five["csr_col"]), five["csr_valf"])
    # expected CSC read off the dense matrix column by column, top to bottom
    d = five["dense"]
    exp_ptr, exp_rows, exp_vals = [0], [], []
    for j in range(5):
        for i in range(5):
            if d[i, j] != 0:
                exp_rows.append(i)
                exp_vals.append(d[i, j])
        exp_ptr.append(len(exp_rows))
    assert cp.tolist() == exp_ptr == [0, 2, 3, 5, 6, 8]
    assert ri.tolist() == exp_rows
    assert cv.tolist() == exp_vals


def test_five_products_exact(five):
    d = five["dense"]
    rp = np.array(five["csr_row_ptr"], np.int32)
    col = np.array(five["csr_col"], np.int32)
    val = five["csr_valf"]
    x = np.arange(1, 6, dtype=np.float32)
    u = np.arange(1, 6, dtype=np.float32)
    # brute force in plain Python loops over the page's dense matrix
    ax = [sum(d[i, j] * x[j] for j in range(5)) for i in range(5)]
    atu = [sum(d[i, j] * u[i] for i in range(5)) for j in range(5)]
    y, _ = oracle.spmv(rp, col, val, x)
    assert y.tolist() == ax == [7, 6, 54, 21, 40]
    cp, ri, cv = oracle.csr_to_csc(5, 5, rp, col, val)
    z, _ = oracle.spmv(cp, ri, cv, u)
    assert z.tolist() == atu == [13, 6, 30, 15, 58]
    zs, _ = oracle.spmv_t_scatter(5, 5, rp, col, val, u)
    assert zs.tolist() == atu
    assert float(np.dot(z, x)) == float(np.dot(u, y)) == 465.0


def test_five_ell_slots(five):
    rp = np.array(five["csr_row_ptr"], np.int32)
    col = np.array(five["csr_col"], np.int32)
    val = five["csr_valf"]
    # ELL is SELL with a single slice holding every row and no sorting window
    s = oracle.sell_build(rp, col, val, C=5, sigma=1)
    assert s["slots"] == five["ell_total_slots"] == 15
    assert int((s["col"] >= 0).sum()) == five["ell_valid_slots"] == 8
    v = five["value_of"]
    for i in range(5):
        got_c = [int(s["col"][t * 5 + i]) for t in range(five["ell_K"])]
        got_v = [float(s["val"][t * 5 + i]) for t in range(five["ell_K"])]
        exp_c = [c if c is not None else -1 for c in five["ell_col_rows"][i]]
        exp_v = [v[a] if a is not None else 0.0 for a in five["ell_val_rows"][i]]
        assert got_c == exp_c
        assert got_v == exp_v
    y = oracle.sell_spmv(s, 5, np.arange(1, 6, dtype=np.float32))
    assert y.tolist() == [7, 6, 54, 21, 40]


# --------------------------------------------------------------------------
# dense brute force on small random matrices
# --------------------------------------------------------------------------
@st.composite
def small_coo(draw):
    m = draw(st.integers(0, 16))
    n = draw(st.integers(1, 16))
    nnz = draw(st.integers(0, 60)) if m > 0 else 0
    row = draw(st.lists(st.integers(0, max(m - 1, 0)), min_size=nnz, max_size=nnz))
    col = draw(st.lists(st.integers(0, n - 1), min_size=nnz, max_size=nnz))
    # distinct small integers as values: every entry is identifiable and all
    # products/sums are exact in fp64
    vals = draw(st.permutations(list(range(1, nnz + 1)))) if nnz else []
    sign = draw(st.lists(st.sampled_from([-1, 1]), min_size=nnz, max_size=nnz))
    val = np.array([s * v for s, v in zip(sign, vals)], np.float32)
    return m, n, np.array(row, np.int32), np.array(col, np.int32), val


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(small_coo())
def test_coo_to_csr_brute_force(case):
    m, n, row, col, val = case
    rp, c, v = oracle.coo_to_csr(m, n, row, col, val)
    assert rp[0] == 0 and rp[-1] == row.size
    assert np.all(np.diff(rp) >= 0)
    # the same matrix, duplicates summed
    np.testing.assert_array_equal(dense_from_csr(m, n, rp, c, v), dense_from_coo(m, n, row, col, val))
    # order inside each row: by column, equal columns in input order
    pos_of_val = {float(a): k for k, a in enumerate(val)}
    for i in range(m):
        seg = list(zip(c[rp[i]:rp[i + 1]].tolist(), [pos_of_val[float(a)] for a in v[rp[i]:rp[i + 1]]]))
        assert seg == sorted(seg)
        assert all(row[p] == i for _, p in seg)
    # row lengths equal the number of COO entries of the row
    assert np.diff(rp).tolist() == [int((row == i).sum()) for i in range(m)]


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(small_coo(), st.integers(0, 2 ** 31 - 1))
def test_products_brute_force(case, seed):
    m, n, row, col, val = case
    rng = np.random.default_rng(seed)
    rp, c, v = oracle.coo_to_csr(m, n, row, col, val)
    d = dense_from_coo(m, n, row, col, val)
    x = rng.integers(-4, 5, size=n).astype(np.float32)
    u = rng.integers(-4, 5, size=m).astype(np.float32)
    yo = rng.integers(-4, 5, size=m).astype(np.float32)
    zo = rng.integers(-4, 5, size=n).astype(np.float32)
    alpha, beta = float(rng.integers(-3, 4)), float(rng.integers(-3, 4))
    # y = alpha A x + beta y
    y, sc = oracle.spmv(rp, c, v, x, alpha, beta, yo)
    np.testing.assert_array_equal(y, alpha * (d @ x) + beta * yo)
    abs_d = dense_from_coo(m, n, row, col, np.abs(val))
    np.testing.assert_array_equal(sc, abs(alpha) * (abs_d @ np.abs(x)) + abs(beta) * np.abs(yo))
    # z = alpha A^T u + beta z through the CSC, and through the scatter route
    cp, ri, cv = oracle.csr_to_csc(m, n, rp, c, v)
    z, _ = oracle.spmv(cp, ri, cv, u, alpha, beta, zo)
    zs, _ = oracle.spmv_t_scatter(m, n, rp, c, v, u, alpha, beta, zo)
    np.testing.assert_array_equal(z, alpha * (d.T @ u) + beta * zo)
    np.testing.assert_array_equal(zs, z)
    # C = alpha A B + beta C
    N = int(rng.integers(1, 5))
    B = rng.integers(-4, 5, size=(n, N)).astype(np.float32)
    C0 = rng.integers(-4, 5, size=(m, N)).astype(np.float32)
    Cm, _ = oracle.spmm(rp, c, v, B, alpha, beta, C0)
    np.testing.assert_array_equal(Cm, alpha * (d @ B) + beta * C0)


def test_beta_zero_does_not_read_y():
    coo = gen.ragged_coo(30, 20, seed=3)
    rp, c, v = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
    x = gen.dense_vector(coo.n, 4)
    y_nan = np.full(coo.m, np.nan, np.float32)
    y, _ = oracle.spmv(rp, c, v, x, 2.0, 0.0, y_nan)
    assert np.all(np.isfinite(y))
    B = gen.dense_matrix(coo.n, 3, 5)
    C, _ = oracle.spmm(rp, c, v, B, 1.0, 0.0, np.full((coo.m, 3), np.nan, np.float32))
    assert np.all(np.isfinite(C))


def test_rows_subset_matches_full():
    coo = gen.ragged_coo(50, 40, seed=7, long_rows=(35,))
    rp, c, v = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
    x = gen.dense_vector(coo.n, 8)
    y0 = gen.dense_vector(coo.m, 9)
    full, fs = oracle.spmv(rp, c, v, x, 0.5, -1.5, y0)
    rows = np.array([49, 0, 17, 17, 3])
    sub, ss = oracle.spmv(rp, c, v, x, 0.5, -1.5, y0, rows=rows)
    np.testing.assert_array_equal(sub, full[rows])
    np.testing.assert_array_equal(ss, fs[rows])
    B = gen.dense_matrix(coo.n, 4, 10)
    Cf, _ = oracle.spmm(rp, c, v, B)
    Cs, _ = oracle.spmm(rp, c, v, B, rows=rows)
    np.testing.assert_array_equal(Cs, Cf[rows])


def test_index_errors_rejected():
    with pytest.raises(oracle.OracleError):
        oracle.coo_to_csr(3, 3, [0, 3], [0, 0], [1.0, 2.0])
    with pytest.raises(oracle.OracleError):
        oracle.coo_to_csr(3, 3, [0, 1], [0, -1], [1.0, 2.0])


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(5))
def test_csc_equals_csr_of_transpose_via_coo(seed):
    coo = gen.ragged_coo(60, 45, seed, long_rows=(44,), dup_frac=0.1)
    rp, c, v = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
    cp, ri, cv = oracle.csr_to_csc(coo.m, coo.n, rp, c, v)
    # CSR(A^T) through the COO route on the swapped triples, fed in CSR order so
    # that equal (row, col) pairs keep CSR order as their tie-break
    row_of = np.repeat(np.arange(coo.m, dtype=np.int32), np.diff(rp))
    tp, tc, tv = oracle.coo_to_csr(coo.n, coo.m, c, row_of, v)
    np.testing.assert_array_equal(cp, tp)
    np.testing.assert_array_equal(ri, tc)
    np.testing.assert_array_equal(cv, tv)
    # transposing twice gives the CSR back
    bp, bc, bv = oracle.csr_to_csc(coo.n, coo.m, cp, ri, cv)
    np.testing.assert_array_equal(bp, rp)
    np.testing.assert_array_equal(bc, c)
    np.testing.assert_array_equal(bv, v)


@pytest.mark.parametrize("seed", range(5))
def test_adjoint_identity(seed):
    coo = gen.ragged_coo(70, 55, seed, long_rows=(50,))
    rp, c, v = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
    cp, ri, cv = oracle.csr_to_csc(coo.m, coo.n, rp, c, v)
    x = gen.dense_vector(coo.n, seed, 3)
    u = gen.dense_vector(coo.m, seed, 4)
    ax, _ = oracle.spmv(rp, c, v, x)
    atu, _ = oracle.spmv(cp, ri, cv, u)
    lhs = float(np.dot(atu, x.astype(np.float64)))
    rhs = float(np.dot(u.astype(np.float64), ax))
    assert abs(lhs - rhs) <= 1e-12 * (np.abs(atu) @ np.abs(x) + 1.0)


@pytest.mark.parametrize("N", [1, 3, 8])
def test_spmm_columns_are_spmv(N):
    coo = gen.ragged_coo(40, 30, 11, long_rows=(29,))
    rp, c, v = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
    B = gen.dense_matrix(coo.n, N, 12)
    C0 = gen.dense_matrix(coo.m, N, 13)
    Cm, Cs = oracle.spmm(rp, c, v, B, 1.5, -0.5, C0)
    for j in range(N):
        y, s = oracle.spmv(rp, c, v, np.ascontiguousarray(B[:, j]), 1.5, -0.5, np.ascontiguousarray(C0[:, j]))
        np.testing.assert_array_equal(Cm[:, j], y)
        np.testing.assert_array_equal(Cs[:, j], s)


# --------------------------------------------------------------------------
# BSR
# --------------------------------------------------------------------------
def _bf16_exact(h):
    # exact widening done with numpy bit operations (independent of the C oracle)
    return (np.asarray(h, np.uint32) << 16).view(np.float32).astype(np.float64)


def test_bf16_widening_exact():
    h = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x4049, 0x7F7F, 0x0001, 0x3C00], np.uint16)
    np.testing.assert_array_equal(oracle.bf16_to_float64(h), _bf16_exact(h))
    assert oracle.bf16_to_float64(np.array([0x3F80], np.uint16))[0] == 1.0
    assert oracle.bf16_to_float64(np.array([0xC000], np.uint16))[0] == -2.0


def test_f32_to_bf16_rounding_pins():
    # round-to-nearest-even at the halfway points of the bf16 grid
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -1.5, 3.0e-3], np.float32)
    h = gen.f32_to_bf16_bits(f)
    assert h[0] == 0x3F80
    assert h[1] == 0x3F80      # tie, even stays
    assert h[2] == 0x3F82      # tie, rounds up to even
    assert h[3] == 0x3F80      # below half
    assert h[4] == 0xBFC0
    assert abs(_bf16_exact(h[5:])[0] - 3.0e-3) <= 2 ** -8 * 3.0e-3


def _dense_from_bsr(b):
    d = np.zeros((b.mb * b.bs, b.kb * b.bs))
    for I in range(b.mb):
        for k in range(b.brow_ptr[I], b.brow_ptr[I + 1]):
            J = b.bcol[k]
            d[I * b.bs:(I + 1) * b.bs, J * b.bs:(J + 1) * b.bs] = _bf16_exact(b.bval[k])
    return d


@pytest.mark.parametrize("bs,mb,kb,density", [(1, 12, 9, 0.3), (4, 5, 6, 0.4), (8, 3, 4, 0.5), (16, 2, 2, 1.0)])
def test_bsr_routes_match_dense(bs, mb, kb, density):
    b = gen.block_sparse_bsr(mb=mb, kb=kb, bs=bs, density=density, std=1.0, seed=bs)
    N = 5
    B = gen.bf16_matrix(kb * bs, N, seed=bs)
    Bd = _bf16_exact(B)
    C0 = gen.dense_matrix(mb * bs, N, 21)
    d = _dense_from_bsr(b)
    rp, c, v = oracle.bsr_to_csr(mb, bs, b.brow_ptr, b.bcol, b.bval)
    Cexp = 0.75 * (d @ Bd) - 2.0 * C0
    C1, _ = oracle.spmm_bf16(rp, c, v, B, 0.75, -2.0, C0)
    C2 = oracle.bsr_spmm_direct(mb, bs, b.brow_ptr, b.bcol, b.bval, B, 0.75, -2.0, C0)
    np.testing.assert_allclose(C1, Cexp, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(C2, Cexp, rtol=1e-12, atol=1e-12)
    # expansion keeps every in-block entry
    assert rp[-1] == b.nnzb * bs * bs


def test_bsr_one_by_one_blocks_equal_csr():
    b = gen.block_sparse_bsr(mb=20, kb=15, bs=1, density=0.3, std=1.0, seed=5)
    # the same matrix as a plain fp32 CSR (bf16 values are exact in fp32)
    vals32 = _bf16_exact(b.bval.reshape(-1)).astype(np.float32)
    B = gen.bf16_matrix(15, 3, seed=6)
    C_bsr = oracle.bsr_spmm_direct(20, 1, b.brow_ptr, b.bcol, b.bval, B)
    C_csr, _ = oracle.spmm(b.brow_ptr, b.bcol, vals32, _bf16_exact(B).astype(np.float32))
    np.testing.assert_array_equal(C_bsr, C_csr)


def test_single_dense_block_is_gemm():
    rng = np.random.default_rng(0)
    blk = gen.f32_to_bf16_bits(rng.normal(size=(1, 8, 8)).astype(np.float32)).reshape(1, 8, 8)
    B = gen.bf16_matrix(8, 4, seed=1)
    C = oracle.bsr_spmm_direct(1, 8, np.array([0, 1]), np.array([0]), blk, B)
    np.testing.assert_allclose(C, _bf16_exact(blk[0]) @ _bf16_exact(B), rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# profile and SELL
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(4))
def test_row_profile_against_numpy(seed):
    coo = gen.ragged_coo(997, 300, seed, long_rows=(250, 299))
    rp, _, _ = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
    p = oracle.row_profile(rp)
    L = np.bincount(coo.row, minlength=coo.m)
    assert p["mean"] == pytest.approx(L.mean(), rel=1e-12)
    assert p["var"] == pytest.approx(L.var(), rel=1e-12)
    assert p["cv"] == pytest.approx(L.std() / L.mean(), rel=1e-12)
    assert p["p95"] == int(np.percentile(L, 95, method="inverted_cdf"))
    assert p["p99"] == int(np.percentile(L, 99, method="inverted_cdf"))
    assert p["max"] == L.max()
    assert p["empty"] == int((L == 0).sum())


@pytest.mark.parametrize("C,sigma", [(4, 1), (4, 8), (64, 256), (8, 1000)])
def test_sell_layout_and_product(C, sigma):
    coo = gen.ragged_coo(301, 120, 2, long_rows=(110,))
    rp, c, v = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
    s = oracle.sell_build(rp, c, v, C, sigma)
    L = np.diff(rp)
    # perm is a permutation that only moves rows inside their sigma window,
    # ordered by decreasing length with ties by row index
    assert sorted(s["perm"].tolist()) == list(range(coo.m))
    for w in range(0, coo.m, sigma):
        win = list(range(w, min(coo.m, w + sigma)))
        assert sorted(s["perm"][win].tolist()) == win
        assert s["perm"][win].tolist() == sorted(win, key=lambda r: (-L[r], r))
    # slot count: every slice padded to its longest row
    widths = [max(L[s["perm"][k]] for k in range(j, min(coo.m, j + C))) for j in range(0, coo.m, C)]
    assert s["slots"] == C * sum(widths)
    assert int((s["col"] >= 0).sum()) == rp[-1]
    x = gen.dense_vector(coo.n, 3)
    y = oracle.sell_spmv(s, C, x)
    np.testing.assert_allclose(y, dense_from_csr(coo.m, coo.n, rp, c, v) @ x.astype(np.float64), rtol=1e-12,
                               atol=1e-12)


# --------------------------------------------------------------------------
# CSR -> BSR and BSR SpMV with fp32 blocks
# --------------------------------------------------------------------------
@pytest.fixture(scope="module")
def five_bsr2(golden_dir):
    with open(os.path.join(golden_dir, "five_by_five_bsr2.json")) as f:
        return json.load(f)


def test_five_csr_to_bsr2_matches_hand_derivation(five, five_bsr2):
    g = five_bsr2
    v = five["value_of"]
    brp, bcol, bval = oracle.csr_to_bsr(5, 5, five["csr_row_ptr"], five["csr_col"], five["csr_valf"], 2)
    assert brp.tolist() == g["brow_ptr"]
    assert bcol.tolist() == g["bcol"]
    blocks = np.array([[[v[e] if isinstance(e, str) else e for e in row] for row in blk] for blk in g["blocks"]],
                      np.float32)
    np.testing.assert_array_equal(bval, blocks)
    assert g["nnz"] / (bcol.size * 2 * 2) == pytest.approx(1.0 / 3.0)
    # the page's product, exact in fp32 and fp64
    y, _ = oracle.bsr_spmv(5, 5, 2, brp, bcol, bval, np.arange(1, 6, dtype=np.float32))
    assert y.tolist() == [7, 6, 54, 21, 40]
    y, _ = oracle.bsr_spmv(5, 5, 2, brp, bcol, bval, np.arange(1, 6, dtype=np.float32), 2.0, -1.0,
                           np.ones(5, np.float32))
    assert y.tolist() == [13, 11, 107, 41, 79]


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(small_coo(), st.sampled_from([1, 2, 3, 4, 5, 8]), st.integers(0, 2 ** 31 - 1))
def test_csr_to_bsr_brute_force(case, bs, seed):
    m, n, row, col, val = case
    rp, c, v = oracle.coo_to_csr(m, n, row, col, val)
    brp, bcol, bval = oracle.csr_to_bsr(m, n, rp, c, v, bs)
    mb, kb = (m + bs - 1) // bs, (n + bs - 1) // bs
    # the stored blocks are exactly the distinct (row // bs, col // bs) pairs, block columns ascending
    pairs = sorted(set(zip((row // bs).tolist(), (col // bs).tolist())))
    assert brp.tolist() == [sum(1 for I, _ in pairs if I < k) for k in range(mb + 1)]
    assert bcol.tolist() == [J for _, J in pairs]
    # expanding the blocks (cropped to m x n) gives the dense matrix, duplicates summed in fp32
    d32 = np.zeros((m, n), np.float32)
    for i in range(m):
        for p in range(rp[i], rp[i + 1]):
            d32[i, c[p]] = d32[i, c[p]] + v[p]
    e = np.zeros((mb * bs, kb * bs), np.float32)
    for I in range(mb):
        for k in range(brp[I], brp[I + 1]):
            e[I * bs:(I + 1) * bs, bcol[k] * bs:(bcol[k] + 1) * bs] = bval[k]
    np.testing.assert_array_equal(e[:m, :n], d32)
    assert not e[m:, :].any() and not e[:, n:].any()
    # BSR SpMV equals the dense product (exact: small integers)
    rng = np.random.default_rng(seed)
    x = rng.integers(-4, 5, size=n).astype(np.float32)
    yo = rng.integers(-4, 5, size=m).astype(np.float32)
    alpha, beta = float(rng.integers(-3, 4)), float(rng.integers(-3, 4))
    y, sc = oracle.bsr_spmv(m, n, bs, brp, bcol, bval, x, alpha, beta, yo)
    np.testing.assert_array_equal(y, alpha * (d32.astype(np.float64) @ x) + beta * yo)
    np.testing.assert_array_equal(sc, abs(alpha) * (np.abs(e[:m, :n]).astype(np.float64) @ np.abs(x)) +
                                  abs(beta) * np.abs(yo))


def test_csr_to_bsr_one_by_one_is_csr():
    coo = gen.ragged_coo(40, 30, seed=9, max_len=12)
    rp, c, v = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
    brp, bcol, bval = oracle.csr_to_bsr(coo.m, coo.n, rp, c, v, 1)
    np.testing.assert_array_equal(brp, rp)
    np.testing.assert_array_equal(bcol, c)
    np.testing.assert_array_equal(bval.reshape(-1), v)


def test_csr_to_bsr_duplicates_summed_in_csr_order():
    # three entries at one position: ((a + b) + c) in fp32, a value that differs from (a + (b + c))
    a, b, c3 = np.float32(1.0), np.float32(2.0 ** -24), np.float32(2.0 ** -24)
    rp = np.array([0, 3], np.int32)
    col = np.array([1, 1, 1], np.int32)
    brp, bcol, bval = oracle.csr_to_bsr(1, 2, rp, col, np.array([a, b, c3], np.float32), 2)
    assert bval[0, 0, 1] == (a + b) + c3 == np.float32(1.0)
    assert (a + (b + c3)) != np.float32(1.0)
    # a lone -0.0 is kept, an untouched position is +0.0
    brp, bcol, bval = oracle.csr_to_bsr(1, 2, np.array([0, 1], np.int32), np.array([0], np.int32),
                                        np.array([-0.0], np.float32), 2)
    assert np.signbit(bval[0, 0, 0]) and not np.signbit(bval[0, 0, 1])


def test_oracle_bf16_rounding_matches_generator_and_pins():
    # two independent round-to-nearest-even implementations (the generator's numpy
    # version and the oracle's C version) agree, and the halfway cases are pinned
    rng = np.random.default_rng(4)
    f = np.concatenate([rng.normal(size=2000).astype(np.float32),
                        np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 3.0e38, -0.0, 0.0],
                                 np.float32)])
    np.testing.assert_array_equal(oracle.f32_to_bf16(f), gen.f32_to_bf16_bits(f))
    h = oracle.f32_to_bf16(np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, np.inf, -np.inf, np.float32(3.4e38)],
                                    np.float32))
    assert h.tolist() == [0x3F80, 0x3F82, 0x7F80, 0xFF80, 0x7F80]
    nan = oracle.f32_to_bf16(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


# --------------------------------------------------------------------------
# CSR -> WCSR and SpMM over it
# --------------------------------------------------------------------------
@pytest.fixture(scope="module")
def five_wcsr2(golden_dir):
    with open(os.path.join(golden_dir, "five_by_five_wcsr2.json")) as f:
        return json.load(f)


def test_five_csr_to_wcsr2_matches_hand_derivation(five, five_wcsr2):
    g = five_wcsr2
    v = five["value_of"]
    wp, wc, vals = oracle.csr_to_wcsr(5, 5, five["csr_row_ptr"], five["csr_col"], five["csr_valf"], g["H"], g["pad"])
    assert wp.tolist() == g["window_ptr"]
    assert wc.tolist() == g["window_col"]
    exp = np.array([[v[e] if isinstance(e, str) else e for e in col] for col in g["values_by_column"]], np.float32)
    np.testing.assert_array_equal(vals, exp)
    C, _ = oracle.wcsr_spmm(5, 2, wp, wc, vals, np.arange(1, 6, dtype=np.float32).reshape(5, 1))
    assert C[:, 0].tolist() == [7, 6, 54, 21, 40]


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(small_coo(), st.sampled_from([1, 2, 3, 4, 8]), st.sampled_from([1, 2, 4, 8]), st.integers(0, 2 ** 31 - 1))
def test_csr_to_wcsr_brute_force(case, H, pad, seed):
    m, n, row, col, val = case
    rp, c, v = oracle.coo_to_csr(m, n, row, col, val)
    wp, wc, vals = oracle.csr_to_wcsr(m, n, rp, c, v, H, pad)
    nw = (m + H - 1) // H
    assert wp.size == nw + 1
    for w in range(nw):
        cols = sorted(set(col[(row // H) == w].tolist()))
        seg = wc[wp[w]:wp[w + 1]].tolist()
        # the distinct columns ascending, then -1 up to a multiple of pad
        assert seg[:len(cols)] == cols and all(s == -1 for s in seg[len(cols):])
        assert len(seg) % pad == 0 and len(seg) - len(cols) < pad
    # expanding the windows gives the dense matrix (duplicates summed in fp32 in CSR order)
    d32 = np.zeros((m, n), np.float32)
    for i in range(m):
        for p in range(rp[i], rp[i + 1]):
            d32[i, c[p]] = d32[i, c[p]] + v[p]
    e = np.zeros((nw * H, n), np.float32)
    for w in range(nw):
        for q in range(wp[w], wp[w + 1]):
            if wc[q] >= 0:
                e[w * H:(w + 1) * H, wc[q]] = vals[q]
            else:
                assert not vals[q].any()
    np.testing.assert_array_equal(e[:m], d32)
    assert not e[m:].any()
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 5))
    B = rng.integers(-4, 5, size=(n, N)).astype(np.float32)
    C0 = rng.integers(-4, 5, size=(m, N)).astype(np.float32)
    alpha, beta = float(rng.integers(-3, 4)), float(rng.integers(-3, 4))
    C, sc = oracle.wcsr_spmm(m, H, wp, wc, vals, B, alpha, beta, C0)
    np.testing.assert_array_equal(C, alpha * (d32.astype(np.float64) @ B) + beta * C0)
    np.testing.assert_array_equal(sc, abs(alpha) * (np.abs(d32).astype(np.float64) @ np.abs(B)) + abs(beta) * np.abs(C0))


# --------------------------------------------------------------------------
# WCSR task split ([ASYNC] §4.2)
# --------------------------------------------------------------------------
def test_wcsr_tasks_hand_derivation():
    # windows of 40, 0, 1060, 60, 1540, 512 and 513 compressed columns, T = 512:
    # 1060 -> 512 + 512 + 36, 1540 -> 512 * 3 + 4, 512 stays whole, 513 -> 512 + 1
    wp = [0, 40, 40, 1100, 1160, 2700, 3212, 3725]
    tasks, winfo, slots = oracle.wcsr_tasks(np.array(wp, np.int32), 512)
    assert tasks.tolist() == [[0, 0, 40, -1], [1, 40, 40, -1],
                              [2, 40, 552, 0], [2, 552, 1064, 1], [2, 1064, 1100, 2],
                              [3, 1100, 1160, -1],
                              [4, 1160, 1672, 3], [4, 1672, 2184, 4], [4, 2184, 2696, 5], [4, 2696, 2700, 6],
                              [5, 2700, 3212, -1],
                              [6, 3212, 3724, 7], [6, 3724, 3725, 8]]
    assert winfo.tolist() == [[-1, 1], [-1, 1], [0, 3], [-1, 1], [3, 4], [-1, 1], [7, 2]]
    assert slots == 9
    tasks, winfo, slots = oracle.wcsr_tasks(np.zeros(1, np.int32), 32)
    assert tasks.shape == (0, 4) and winfo.shape == (0, 2) and slots == 0


@settings(max_examples=200, deadline=None)
@given(st.lists(st.integers(0, 300), min_size=1, max_size=40), st.sampled_from([1, 3, 32, 64]),
       st.integers(0, 2 ** 31 - 1))
def test_wcsr_tasks_cover_each_window_once(widths, T, seed):
    wp = np.concatenate([[0], np.cumsum(widths)]).astype(np.int32)
    tasks, winfo, slots = oracle.wcsr_tasks(wp, T)
    nw = len(widths)
    # tasks run window by window; each window's tasks tile its range in order
    k = 0
    next_slot = 0
    for w in range(nw):
        c = widths[w]
        nt = 1 if c <= T else -(-c // T)
        mine = tasks[k:k + nt]
        assert (mine[:, 0] == w).all()
        assert mine[0, 1] == wp[w] and mine[-1, 2] == wp[w + 1]
        assert (mine[1:, 1] == mine[:-1, 2]).all()
        if nt == 1:
            assert mine[0, 3] == -1 and winfo[w].tolist() == [-1, 1]
        else:
            assert ((mine[:, 2] - mine[:, 1]) <= T).all() and ((mine[:-1, 2] - mine[:-1, 1]) == T).all()
            assert mine[-1, 2] - mine[-1, 1] >= 1
            assert mine[:, 3].tolist() == list(range(next_slot, next_slot + nt))
            assert winfo[w].tolist() == [next_slot, nt]
            next_slot += nt
        k += nt
    assert k == len(tasks) and slots == next_slot
    # the sum of the tasks' partial products is the product of the whole window
    rng = np.random.default_rng(seed)
    total = int(wp[-1])
    H, N = 3, 2
    vals = rng.integers(-3, 4, size=(total, H)).astype(np.float64)
    Bq = rng.integers(-3, 4, size=(total, N)).astype(np.float64)  # B row of each compressed column
    whole = np.stack([vals[wp[w]:wp[w + 1]].T @ Bq[wp[w]:wp[w + 1]] for w in range(nw)])
    parts = np.zeros_like(whole)
    for w, b, e, _ in tasks:
        parts[w] += vals[b:e].T @ Bq[b:e]
    np.testing.assert_array_equal(parts, whole)
