"""GPU parity at the limits of the layouts: the x-window stream at its widest
x (256 windows of 2^15 columns) and one column past it, rows whose lengths
sit on the row-chunk size (15360 entries) and the chunk row cap (1536 rows),
one row of 4 M entries, and SELL's int16 column offsets at exactly 32767 and
32768.  Each case against the CPU oracle, both directions where the plan
holds a CSC."""
import numpy as np
import pytest
import torch

import gen
import oracle
import spmm_csr_spmv_amd as sp
from gpu_util import assert_close, dev, host, say

pytestmark = pytest.mark.gpu

CHUNK = 15360          # entries of a row chunk of the x-window stream
MAX_WINDOWS = 256
WINDOW = 1 << 15       # widest window


def _csr(coo):
    return oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)


def _check_spmv(plan, m, n, rp, c, v, seed, what, alpha=1.25, beta=-0.5):
    x = gen.dense_vector(n, seed)
    y0 = gen.dense_vector(m, seed + 1)
    y = dev(y0)
    sp.spmv(plan, alpha, dev(x), beta, y)
    ref, scale = oracle.spmv(rp, c, v, x, alpha, beta, y0)
    assert_close(host(y), ref, scale, what=what)


def _check_spmv_t(plan, m, n, cp, ri, cv, seed, what):
    u = gen.dense_vector(m, seed)
    z = torch.zeros(n, device="cuda")
    sp.spmv_t(plan, 1.0, dev(u), 0.0, z)
    ref, scale = oracle.spmv(cp, ri, cv, u)
    assert_close(host(z), ref, scale, what=what)


def test_x_windows_at_the_widest_x():
    """2^23 columns = exactly 256 windows of 2^15: accepted, exact, and the
    automatic choice may take it; one column more needs 257 windows: an
    explicit width is refused and the automatic choice falls back."""
    m = 1 << 16
    for n, fits in ((MAX_WINDOWS * WINDOW, True), (MAX_WINDOWS * WINDOW + 1, False)):
        say("x windows at n = %d" % n)
        coo = gen.ragged_coo(m, n, seed=11, max_len=40, empty_frac=0.1, shuffled=False)
        rp, c, v = _csr(coo)
        g = (dev(rp), dev(c), dev(v))
        if fits:
            plan = sp.Plan(m, n, *g, use_sell=0, x_window_bits=15)
            assert plan.profile()["x_window_bits"] == 15
            _check_spmv(plan, m, n, rp, c, v, 20, "256 windows")
        else:
            with pytest.raises(sp.SparseError) as e:
                sp.Plan(m, n, *g, use_sell=0, x_window_bits=15)
            assert e.value.code == 5
        plan = sp.Plan(m, n, *g)
        assert plan.profile()["x_window_bits"] in ((0, 15) if fits else (0,))
        _check_spmv(plan, m, n, rp, c, v, 22, "default plan, n = %d" % n)


@pytest.mark.parametrize("bits", [10, 12, 15])
def test_x_window_chunk_edges(bits):
    """Rows one short of, exactly at, and one past the chunk length and twice
    it (segments, a last segment of one entry), long runs of one-entry rows
    (chunks closed by the row cap), empty rows; both directions."""
    say("x-window chunk edges, bits", bits)
    coo = gen.ragged_coo(6000, 200000, seed=12, max_len=1, empty_frac=0.2,
                         long_rows=(CHUNK - 1, CHUNK, CHUNK + 1, 2 * CHUNK, 2 * CHUNK + 1, 1536, 1537))
    rp, c, v = _csr(coo)
    lens = np.diff(rp)
    assert {CHUNK - 1, CHUNK, CHUNK + 1, 2 * CHUNK, 2 * CHUNK + 1} <= set(lens.tolist())
    cp, ri, cv = oracle.csr_to_csc(coo.m, coo.n, rp, c, v)
    plan = sp.Plan(coo.m, coo.n, dev(rp), dev(c), dev(v), csc=(dev(cp), dev(ri), dev(cv)), use_sell=0,
                   x_window_bits=bits)
    assert plan.profile()["x_window_bits"] == bits
    # repeated calls: the long rows' arrival counters are back at zero after each
    for k, (alpha, beta) in enumerate(((1.25, -0.5), (1.0, 0.0), (-2.0, 1.5))):
        _check_spmv(plan, coo.m, coo.n, rp, c, v, 30 + 2 * k, "chunk edges, bits %d, call %d" % (bits, k),
                    alpha, beta)
    _check_spmv_t(plan, coo.m, coo.n, cp, ri, cv, 38, "chunk edges transposed, bits %d" % bits)


@pytest.mark.parametrize("opts", [dict(use_sell=0, x_window_bits=15), dict(use_sell=0, x_window_bits=0, col_panels=0)])
def test_one_row_of_four_million_entries(opts):
    """A row holding every column of a 2^22-column x (274 chunk segments in
    the x-window stream; the split-row bin otherwise) between two short rows."""
    say("one dense row of 2^22 entries", opts)
    n = 1 << 22
    rng = np.random.default_rng(13)
    row = np.concatenate([np.zeros(5, np.int32), np.ones(n, np.int32), np.full(3, 2, np.int32)])
    col = np.concatenate([rng.choice(n, 5, replace=False), np.arange(n), rng.choice(n, 3, replace=False)]).astype(np.int32)
    val = rng.uniform(-1, 1, row.size).astype(np.float32)
    rp, c, v = oracle.coo_to_csr(3, n, row, col, val)
    plan = sp.Plan(3, n, dev(rp), dev(c), dev(v), **opts)
    assert plan.profile()["x_window_bits"] == opts["x_window_bits"]
    _check_spmv(plan, 3, n, rp, c, v, 40, "dense row %s" % opts)


@pytest.mark.parametrize("reach", [32767, 32768])
def test_sell_offsets_at_the_int16_limit(reach):
    """Every row r holds columns r - 32767, r and r + 32767 (where they exist),
    the largest offset int16 holds; with reach 32768 one entry lies one
    further and the plan must keep int32 columns.  Both directions exact."""
    say("sell offsets, reach", reach)
    m = n = 70000
    r = np.arange(m, dtype=np.int64)
    rows = [r, r[r + 32767 < n], r[r >= 32767]]
    cols = [r, r[r + 32767 < n] + 32767, r[r >= 32767] - 32767]
    if reach > 32767:
        rows.append(np.array([5], np.int64))
        cols.append(np.array([5 + reach], np.int64))
    row = np.concatenate(rows).astype(np.int32)
    col = np.concatenate(cols).astype(np.int32)
    val = np.random.default_rng(14).uniform(-1, 1, row.size).astype(np.float32)
    rp, c, v = oracle.coo_to_csr(m, n, row, col, val)
    assert np.abs(c.astype(np.int64) - np.repeat(np.arange(m), np.diff(rp))).max() == reach
    cp, ri, cv = oracle.csr_to_csc(m, n, rp, c, v)
    plan = sp.Plan(m, n, dev(rp), dev(c), dev(v), csc=(dev(cp), dev(ri), dev(cv)), use_sell=1, col_panels=0,
                   x_window_bits=0)
    assert plan.profile()["sell_slots"] > 0
    _check_spmv(plan, m, n, rp, c, v, 50, "sell reach %d" % reach)
    _check_spmv_t(plan, m, n, cp, ri, cv, 52, "sell reach %d transposed" % reach)


@pytest.mark.parametrize("order", ["shuffled", "row_major"])
def test_conversions_with_long_segments(order):
    """COO -> CSR and CSR -> CSC bit for bit where rows and columns are longer
    than one 4096-key sort chunk (one key past it, a power of two and one
    past it, 18 chunks), plus random entries with duplicates, in shuffled and
    in row-major input order (row-major input gives long runs of one row
    inside a wave)."""
    say("conversions with long segments", order)
    m, n = 30000, 90000
    rng = np.random.default_rng(15)
    rows, cols = [], []
    # long rows 11..14 take columns >= 100, long columns 5..7 rows >= 100, the
    # random entries both, so the long segments have exactly these lengths
    for r, L in ((11, 4097), (12, 8192), (13, 8193), (14, 70000)):
        rows.append(np.full(L, r))
        cols.append(100 + rng.choice(n - 100, L, replace=False))
    for c, L in ((5, 4097), (6, 16384), (7, 29899)):
        rows.append(100 + rng.choice(m - 100, L, replace=False))
        cols.append(np.full(L, c))
    r_rand = rng.integers(100, m, 200000)
    c_rand = rng.integers(100, n, 200000)
    dup = rng.random(r_rand.size) < 0.05
    rows += [r_rand, r_rand[dup]]
    cols += [c_rand, c_rand[dup]]
    row = np.concatenate(rows).astype(np.int32)
    col = np.concatenate(cols).astype(np.int32)
    val = rng.uniform(-1, 1, row.size).astype(np.float32)
    p = rng.permutation(row.size) if order == "shuffled" else np.lexsort((col, row))
    row, col, val = row[p], col[p], val[p]
    rp, c, v = oracle.coo_to_csr(m, n, row, col, val)
    cp, ri, cv = oracle.csr_to_csc(m, n, rp, c, v)
    lens, clens = np.diff(rp), np.diff(cp)
    assert [lens[r] for r in (11, 12, 13, 14)] == [4097, 8192, 8193, 70000]
    assert [clens[c] for c in (5, 6, 7)] == [4097, 16384, 29899]
    g_rp, g_c, g_v = sp.csr_build_from_coo(m, n, dev(row), dev(col), dev(val))
    np.testing.assert_array_equal(host(g_rp), rp)
    np.testing.assert_array_equal(host(g_c), c)
    np.testing.assert_array_equal(host(g_v).view(np.uint32), v.view(np.uint32))
    g_cp, g_ri, g_cv = sp.csr_to_csc(m, n, g_rp, g_c, g_v)
    np.testing.assert_array_equal(host(g_cp), cp)
    np.testing.assert_array_equal(host(g_ri), ri)
    np.testing.assert_array_equal(host(g_cv).view(np.uint32), cv.view(np.uint32))


def test_conversions_with_many_long_segments():
    """More than 1024 rows longer than one sort chunk, so the table of long
    segments takes several passes of its one-workgroup prefix sum; then the
    transpose, whose columns are all short."""
    say("conversions with 1100 long rows")
    m, n = 1100, 200000
    rng = np.random.default_rng(16)
    lens = rng.integers(4097, 4400, m)
    row = np.repeat(np.arange(m), lens).astype(np.int32)
    col = np.concatenate([rng.choice(n, L, replace=False) for L in lens]).astype(np.int32)
    val = rng.uniform(-1, 1, row.size).astype(np.float32)
    p = rng.permutation(row.size)
    row, col, val = row[p], col[p], val[p]
    rp, c, v = oracle.coo_to_csr(m, n, row, col, val)
    cp, ri, cv = oracle.csr_to_csc(m, n, rp, c, v)
    g_rp, g_c, g_v = sp.csr_build_from_coo(m, n, dev(row), dev(col), dev(val))
    np.testing.assert_array_equal(host(g_rp), rp)
    np.testing.assert_array_equal(host(g_c), c)
    np.testing.assert_array_equal(host(g_v).view(np.uint32), v.view(np.uint32))
    g_cp, g_ri, g_cv = sp.csr_to_csc(m, n, g_rp, g_c, g_v)
    np.testing.assert_array_equal(host(g_cp), cp)
    np.testing.assert_array_equal(host(g_ri), ri)
    np.testing.assert_array_equal(host(g_cv).view(np.uint32), cv.view(np.uint32))
