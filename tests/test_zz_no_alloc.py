"""csr_build_from_coo_noalloc: the COO -> CSR conversion with the library's
static per-GPU scratch instead of a caller workspace, for callers that cannot
allocate device memory.  Called through the C ABI and compared bit for bit
with csr_build_from_coo (and so with the oracle's CSR), on consecutive calls
whose second input is smaller (the array keeps the first call's contents)."""
import ctypes

import numpy as np
import pytest
import torch

import gen
import oracle
import spmm_csr_spmv_amd as sp
from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def _noalloc(coo, d):
    L = sp.lib()
    rp = torch.full((coo.m + 1,), -7, dtype=torch.int32, device="cuda")
    ci = torch.full((coo.nnz,), -7, dtype=torch.int32, device="cuda")
    vv = torch.full((coo.nnz,), float("nan"), device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr()) if t.numel() else ctypes.c_void_p(0)  # noqa: E731
    rc = L.csr_build_from_coo_noalloc(coo.m, coo.n, coo.nnz, P(d[0]), P(d[1]), P(d[2]), P(rp), P(ci), P(vv),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, sp.status_string(rc)
    return rp, ci, vv


def _check_same(coo, tag):
    d = (dev(coo.row), dev(coo.col), dev(coo.val))
    got = _noalloc(coo, d)
    ref = sp.csr_build_from_coo(coo.m, coo.n, *d)
    for g, r, name in zip(got, ref, ("row_ptr", "col_idx", "val")):
        a, b = host(g), host(r)
        if a.dtype == np.float32:
            a, b = a.view(np.uint32), b.view(np.uint32)
        np.testing.assert_array_equal(a, b, err_msg="%s: %s differs" % (tag, name))
    return got


def test_noalloc_matches_workspace_entry_point_twice():
    say("noalloc: large then smaller")
    big = gen.ragged_coo(60000, 50000, seed=11, max_len=60, long_rows=(5000, 30000), dup_frac=0.05)
    small = gen.ragged_coo(900, 700, seed=12, max_len=20, dup_frac=0.2)
    assert big.nnz > 10 * small.nnz
    _check_same(big, "first call")
    got = _check_same(small, "second call, smaller")
    # and the oracle's CSR of the smaller input
    rp, c, v = oracle.coo_to_csr(small.m, small.n, small.row, small.col, small.val)
    np.testing.assert_array_equal(host(got[0]), rp)
    np.testing.assert_array_equal(host(got[1]), c)
    np.testing.assert_array_equal(host(got[2]).view(np.uint32), v.view(np.uint32))


def test_noalloc_edge_sizes_and_limit():
    say("noalloc: empty, one entry, limit")
    empty = gen.Coo(5, 4, np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros(0, np.float32))
    got = _check_same(empty, "empty")
    assert host(got[0]).tolist() == [0] * 6
    one = gen.Coo(3, 3, np.array([2], np.int32), np.array([1], np.int32), np.array([1.5], np.float32))
    _check_same(one, "one entry")
    # the binding wrapper gives the same result
    d = (dev(one.row), dev(one.col), dev(one.val))
    rp, ci, vv = sp.csr_build_from_coo_noalloc(one.m, one.n, *d)
    assert host(rp).tolist() == [0, 0, 0, 1] and host(ci).tolist() == [1] and host(vv).tolist() == [1.5]
    # bad indices are still reported
    bad = gen.Coo(3, 3, np.array([0, 3], np.int32), np.array([0, 0], np.int32), np.ones(2, np.float32))
    with pytest.raises(sp.SparseError) as e:
        sp.csr_build_from_coo_noalloc(bad.m, bad.n, dev(bad.row), dev(bad.col), dev(bad.val))
    assert e.value.code == 3
    # beyond the static scratch: refused before any work
    L = sp.lib()
    f = ctypes.c_void_p(0x1000)
    assert L.csr_build_from_coo_noalloc(1000, 1000, 5_000_000, f, f, f, f, f, f, None) == 4
