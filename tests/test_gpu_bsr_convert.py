"""GPU parity of CSR -> BSR (analyze + fill, fill-ratio gate) and of BSR SpMV
with fp32 blocks, called through the C ABI, against the CPU oracle.
Conversions must match bit for bit (fp32 and bf16 blocks); products within
|got - ref| <= 1e-5 * scale + 1e-30 per row."""
import json
import os

import numpy as np
import pytest
import torch

import gen
import oracle
import spmm_csr_spmv_amd as sp
from gpu_util import assert_close, dev, host, say

pytestmark = pytest.mark.gpu

BLOCKS = [1, 2, 4, 8, 16, 32, 64]
AB = [(1.0, 0.0), (1.0, -0.75), (-2.5, 1.5), (0.0, 2.0)]


def cases():
    return {
        "ragged_dups": lambda: gen.ragged_coo(700, 500, seed=1, max_len=40, dup_frac=0.15),
        "ragged_long": lambda: gen.ragged_coo(301, 1999, seed=2, max_len=30, long_rows=(300, 1500, 1999, 257)),
        "tall_empty": lambda: gen.ragged_coo(3000, 70, seed=4, max_len=12, empty_frac=0.5),
        "block_dense": lambda: gen.block_sparse_coo(mb=5, kb=7, bs=64, density=0.3, std=1.0, seed=3),
        "all_empty": lambda: gen.Coo(37, 11, np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros(0, np.float32)),
    }


_cache = {}


def case(name):
    if name not in _cache:
        coo = cases()[name]()
        _cache[name] = (coo, oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val))
    return _cache[name]


def test_five_by_five_bsr2_exact(golden_dir):
    say("bsr five_by_five")
    with open(os.path.join(golden_dir, "five_by_five.json")) as f:
        g = json.load(f)
    with open(os.path.join(golden_dir, "five_by_five_bsr2.json")) as f:
        gb = json.load(f)
    v = g["value_of"]
    val = np.array([v[s] for s in g["csr_val"]], np.float32)
    brp, bcol, bval, fill = sp.csr_to_bsr(5, 5, dev(np.array(g["csr_row_ptr"], np.int32)),
                                          dev(np.array(g["csr_col"], np.int32)), dev(val), 2)
    assert host(brp).tolist() == gb["brow_ptr"]
    assert host(bcol).tolist() == gb["bcol"]
    blocks = np.array([[[v[e] if isinstance(e, str) else e for e in row] for row in blk] for blk in gb["blocks"]],
                      np.float32)
    np.testing.assert_array_equal(host(bval), blocks)
    assert fill == pytest.approx(1.0 / 3.0)
    for rowwise in (False, True):
        y = torch.full((5,), float("nan"), device="cuda")
        sp.bsr_spmv(5, 5, 2, brp, bcol, bval, 1.0, dev(np.arange(1, 6, dtype=np.float32)), 0.0, y, rowwise=rowwise)
        assert host(y).tolist() == [7, 6, 54, 21, 40]


@pytest.mark.parametrize("bs", BLOCKS)
@pytest.mark.parametrize("name", list(cases()))
def test_conversion_bit_exact(name, bs):
    say("csr_to_bsr", name, bs)
    coo, (rp, c, v) = case(name)
    erp, ecol, eval32 = oracle.csr_to_bsr(coo.m, coo.n, rp, c, v, bs)
    for out in ("f32", "bf16"):
        brp, bcol, bval, fill = sp.csr_to_bsr(coo.m, coo.n, dev(rp), dev(c), dev(v), bs, out=out)
        np.testing.assert_array_equal(host(brp), erp)
        np.testing.assert_array_equal(host(bcol), ecol)
        got = host(bval)
        if out == "f32":
            np.testing.assert_array_equal(got.view(np.uint32), eval32.view(np.uint32))
        else:
            np.testing.assert_array_equal(got.view(np.uint16), oracle.f32_to_bf16(eval32))
        nnzb = ecol.size
        assert fill == pytest.approx(c.size / (nnzb * bs * bs) if nnzb else 1.0, rel=1e-12)


@pytest.mark.parametrize("rowwise", [False, True], ids=["whole_blocks", "rows"])
@pytest.mark.parametrize("bs", BLOCKS)
@pytest.mark.parametrize("name", list(cases()))
def test_bsr_spmv(name, bs, rowwise):
    say("bsr_spmv", name, bs, rowwise)
    coo, (rp, c, v) = case(name)
    erp, ecol, eval32 = oracle.csr_to_bsr(coo.m, coo.n, rp, c, v, bs)
    brp, bcol, bval = dev(erp), dev(ecol), dev(eval32)
    x = gen.dense_vector(coo.n, 11)
    for alpha, beta in AB:
        y0 = gen.dense_vector(coo.m, 13)
        y = dev(y0) if beta != 0.0 else torch.full((coo.m,), float("nan"), device="cuda")
        sp.bsr_spmv(coo.m, coo.n, bs, brp, bcol, bval, alpha, dev(x), beta, y, rowwise=rowwise)
        ref, scale = oracle.bsr_spmv(coo.m, coo.n, bs, erp, ecol, eval32, x, alpha, beta, y0)
        assert_close(host(y), ref, scale, what="bsr_spmv %s bs=%d a=%g b=%g" % (name, bs, alpha, beta))
        # the CSR route computes the same product up to the fp32 sums of
        # duplicate entries that the conversion makes
        ref_csr, _ = oracle.spmv(rp, c, v, x, alpha, beta, y0)
        assert_close(ref, ref_csr, scale, what="BSR and CSR routes of the oracle")


@pytest.mark.parametrize("rowwise", [False, True], ids=["whole_blocks", "rows"])
@pytest.mark.parametrize("bs", [4, 64])
def test_bsr_spmv_bitwise_deterministic(bs, rowwise):
    say("bsr_spmv determinism", bs, rowwise)
    coo, (rp, c, v) = case("ragged_long")
    brp, bcol, bval, _ = sp.csr_to_bsr(coo.m, coo.n, dev(rp), dev(c), dev(v), bs)
    x = dev(gen.dense_vector(coo.n, 21))
    outs = []
    for _ in range(3):
        y = torch.zeros(coo.m, device="cuda")
        sp.bsr_spmv(coo.m, coo.n, bs, brp, bcol, bval, 1.0, x, 0.0, y, rowwise=rowwise)
        outs.append(host(y).view(np.uint32).copy())
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_fill_gate_and_input_errors():
    say("csr_to_bsr gate and errors")
    coo, (rp, c, v) = case("ragged_dups")
    # scattered entries fill 8 x 8 blocks poorly: the gate refuses, the block count is still reported
    erp, ecol, _ = oracle.csr_to_bsr(coo.m, coo.n, rp, c, v, 8)
    fill = c.size / (ecol.size * 64)
    assert fill < 0.2
    with pytest.raises(sp.SparseError) as e:
        sp.csr_to_bsr(coo.m, coo.n, dev(rp), dev(c), dev(v), 8, min_fill=0.5)
    assert e.value.code == 8
    brp, bcol, _, got_fill = sp.csr_to_bsr(coo.m, coo.n, dev(rp), dev(c), dev(v), 8, min_fill=fill * 0.999)
    assert got_fill == pytest.approx(fill, rel=1e-12) and bcol.numel() == ecol.size
    # a dense block pattern passes a strict gate
    coo2, (rp2, c2, v2) = case("block_dense")
    _, _, _, f2 = sp.csr_to_bsr(coo2.m, coo2.n, dev(rp2), dev(c2), dev(v2), 64, min_fill=0.999)
    assert f2 == 1.0
    # a row not sorted by column, and a column outside [0, n)
    bad = c.copy()
    i = int(np.argmax(np.diff(rp) >= 2))
    bad[rp[i]], bad[rp[i] + 1] = c[rp[i] + 1], c[rp[i]]
    if bad[rp[i]] != bad[rp[i] + 1]:
        with pytest.raises(sp.SparseError) as e:
            sp.csr_to_bsr(coo.m, coo.n, dev(rp), dev(bad), dev(v), 4)
        assert e.value.code == 5
    bad = c.copy()
    bad[-1] = coo.n
    with pytest.raises(sp.SparseError) as e:
        sp.csr_to_bsr(coo.m, coo.n, dev(rp), dev(bad), dev(v), 4)
    assert e.value.code == 3


def test_block_sparse_workload_full():
    """The 16384 x 16384 workload with 10 % of 64 x 64 blocks (26.8 M entries):
    conversion bit-exact, fill ratio 1, BSR SpMV on every row."""
    say("bsr full workload")
    coo = gen.block_sparse_coo(seed=0)
    rp, c, v = sp.csr_build_from_coo(coo.m, coo.n, dev(coo.row), dev(coo.col), dev(coo.val))
    hrp, hc, hv = host(rp), host(c), host(v)
    erp, ecol, eval32 = oracle.csr_to_bsr(coo.m, coo.n, hrp, hc, hv, 64)
    brp, bcol, bval, fill = sp.csr_to_bsr(coo.m, coo.n, rp, c, v, 64, min_fill=0.5)
    assert fill == 1.0
    np.testing.assert_array_equal(host(brp), erp)
    np.testing.assert_array_equal(host(bcol), ecol)
    np.testing.assert_array_equal(host(bval).view(np.uint32), eval32.view(np.uint32))
    x = gen.dense_vector(coo.n, 0, 1)
    ref, scale = oracle.bsr_spmv(coo.m, coo.n, 64, erp, ecol, eval32, x)
    for rowwise in (False, True):
        y = torch.full((coo.m,), float("nan"), device="cuda")
        sp.bsr_spmv(coo.m, coo.n, 64, brp, bcol, bval, 1.0, dev(x), 0.0, y, rowwise=rowwise)
        assert_close(host(y), ref, scale, what="bsr_spmv full, rowwise=%s" % rowwise)
