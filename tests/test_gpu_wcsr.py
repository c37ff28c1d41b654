"""GPU parity of CSR -> WCSR (windows of 64 rows) and of the windowed SpMM on
MFMA, through the C ABI, against the CPU oracle: conversion bit-exact, products
within |got - ref| <= 1e-5 * scale + 1e-30 per output."""
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

AB = [(1.0, 0.0), (1.0, -0.75), (-2.5, 1.5), (0.0, 2.0)]


def cases():
    return {
        "ragged_dups": lambda: gen.ragged_coo(700, 500, seed=1, max_len=40, dup_frac=0.15),
        "ragged_long": lambda: gen.ragged_coo(301, 1999, seed=2, max_len=30, long_rows=(300, 1500, 1999, 257)),
        "tall_empty": lambda: gen.ragged_coo(3000, 70, seed=4, max_len=12, empty_frac=0.5),
        "clustered": lambda: gen.clustered_coo(m=4100, n=50000, seed=5),
        "all_empty": lambda: gen.Coo(37, 11, np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros(0, np.float32)),
    }


_cache = {}


def case(name):
    if name not in _cache:
        coo = cases()[name]()
        _cache[name] = (coo, oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val))
    return _cache[name]


def test_five_by_five_single_window(golden_dir):
    say("wcsr five_by_five")
    with open(os.path.join(golden_dir, "five_by_five.json")) as f:
        g = json.load(f)
    v = g["value_of"]
    val = np.array([v[s] for s in g["csr_val"]], np.float32)
    rp, c = np.array(g["csr_row_ptr"], np.int32), np.array(g["csr_col"], np.int32)
    wp, wc, vals, fill = sp.csr_to_wcsr(5, 5, dev(rp), dev(c), dev(val), pad=8)
    # one window: the union of all five rows' columns, 0..4, padded to 8
    assert host(wp).tolist() == [0, 8] and host(wc).tolist() == [0, 1, 2, 3, 4, -1, -1, -1]
    ewp, ewc, evals = oracle.csr_to_wcsr(5, 5, rp, c, val, 64, 8)
    np.testing.assert_array_equal(host(vals), evals)
    assert fill == pytest.approx(8 / (8 * 64))
    C = torch.full((5, 4), float("nan"), device="cuda")
    B = np.repeat(np.arange(1, 6, dtype=np.float32)[:, None], 4, axis=1)
    sp.wcsr_spmm(5, 5, wp, wc, vals, 1.0, dev(B), 0.0, C)
    assert host(C)[:, 0].tolist() == [7, 6, 54, 21, 40] and (host(C) == host(C)[:, :1]).all()


@pytest.mark.parametrize("pad", [1, 8, 32])
@pytest.mark.parametrize("name", list(cases()))
def test_conversion_bit_exact(name, pad):
    say("csr_to_wcsr", name, pad)
    coo, (rp, c, v) = case(name)
    ewp, ewc, evals = oracle.csr_to_wcsr(coo.m, coo.n, rp, c, v, 64, pad)
    wp, wc, vals, fill = sp.csr_to_wcsr(coo.m, coo.n, dev(rp), dev(c), dev(v), pad=pad)
    np.testing.assert_array_equal(host(wp), ewp)
    np.testing.assert_array_equal(host(wc), ewc)
    np.testing.assert_array_equal(host(vals).view(np.uint32), evals.view(np.uint32))
    assert fill == pytest.approx(c.size / (ewc.size * 64) if ewc.size else 1.0, rel=1e-12)


@pytest.mark.parametrize("N", [4, 8, 32, 100, 128, 192])
@pytest.mark.parametrize("name", list(cases()))
def test_wcsr_spmm(name, N):
    say("wcsr_spmm", name, N)
    coo, (rp, c, v) = case(name)
    ewp, ewc, evals = oracle.csr_to_wcsr(coo.m, coo.n, rp, c, v, 64, 8)
    wp, wc, vals = dev(ewp), dev(ewc), dev(evals)
    B = gen.dense_matrix(coo.n, N, 3)
    for alpha, beta in AB:
        C0 = gen.dense_matrix(coo.m, N, 4)
        C = dev(C0) if beta != 0.0 else torch.full((coo.m, N), float("nan"), device="cuda")
        sp.wcsr_spmm(coo.m, coo.n, wp, wc, vals, alpha, dev(B), beta, C)
        ref, scale = oracle.wcsr_spmm(coo.m, 64, ewp, ewc, evals, B, alpha, beta, C0)
        assert_close(host(C), ref, scale, what="wcsr_spmm %s N=%d a=%g b=%g" % (name, N, alpha, beta))
    # the CSR route gives the same product, up to the fp32 sums of duplicates
    ref_csr, _ = oracle.spmm(rp, c, v, B)
    ref_w, scale_w = oracle.wcsr_spmm(coo.m, 64, ewp, ewc, evals, B)
    assert_close(ref_w, ref_csr, scale_w, what="WCSR and CSR routes of the oracle")


def test_wcsr_bitwise_deterministic_and_errors():
    say("wcsr determinism and errors")
    coo, (rp, c, v) = case("clustered")
    wp, wc, vals, _ = sp.csr_to_wcsr(coo.m, coo.n, dev(rp), dev(c), dev(v))
    B = dev(gen.dense_matrix(coo.n, 32, 9))
    outs = []
    for _ in range(3):
        C = torch.zeros(coo.m, 32, device="cuda")
        sp.wcsr_spmm(coo.m, coo.n, wp, wc, vals, 1.0, B, 0.0, C)
        outs.append(host(C).view(np.uint32).copy())
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    coo2, (rp2, c2, v2) = case("ragged_dups")
    bad = c2.copy()
    i = int(np.argmax(np.diff(rp2) >= 2))
    bad[rp2[i]], bad[rp2[i] + 1] = c2[rp2[i] + 1], c2[rp2[i]]
    if bad[rp2[i]] != bad[rp2[i] + 1]:
        with pytest.raises(sp.SparseError) as e:
            sp.csr_to_wcsr(coo2.m, coo2.n, dev(rp2), dev(bad), dev(v2))
        assert e.value.code == 5
    bad = c2.copy()
    bad[-1] = -1
    with pytest.raises(sp.SparseError) as e:
        sp.csr_to_wcsr(coo2.m, coo2.n, dev(rp2), dev(bad), dev(v2))
    assert e.value.code == 3


def test_clustered_workload_full():
    """The 2^20 x 2^20 clustered workload (19.9 M entries): conversion bit-exact,
    windowed SpMM with N = 8 on every row."""
    say("wcsr full workload")
    coo = gen.clustered_coo(seed=0)
    rp, c, v = sp.csr_build_from_coo(coo.m, coo.n, dev(coo.row), dev(coo.col), dev(coo.val))
    hrp, hc, hv = host(rp), host(c), host(v)
    ewp, ewc, evals = oracle.csr_to_wcsr(coo.m, coo.n, hrp, hc, hv, 64, 8)
    wp, wc, vals, fill = sp.csr_to_wcsr(coo.m, coo.n, rp, c, v, pad=8)
    np.testing.assert_array_equal(host(wp), ewp)
    np.testing.assert_array_equal(host(wc), ewc)
    np.testing.assert_array_equal(host(vals).view(np.uint32), evals.view(np.uint32))
    B = gen.dense_matrix(coo.n, 8, 0)
    C = torch.full((coo.m, 8), float("nan"), device="cuda")
    sp.wcsr_spmm(coo.m, coo.n, wp, wc, vals, 1.0, dev(B), 0.0, C)
    ref, scale = oracle.wcsr_spmm(coo.m, 64, ewp, ewc, evals, B)
    assert_close(host(C), ref, scale, what="wcsr_spmm full")
