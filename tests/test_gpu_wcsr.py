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


WIDE = {
    # windows of about 5000 entries (one workgroup each, a column bitmap in 4 passes of 2^19 columns)
    "wide_multipass": lambda: gen.ragged_coo(200, 3 * 2 ** 19 + 7, seed=11, max_len=160, empty_frac=0.1,
                                             dup_frac=0.05),
    # as wide, but more columns than the bitmap path takes: the wave merge
    "wide_huge_n": lambda: gen.ragged_coo(130, 5_000_000, seed=12, max_len=160, empty_frac=0.1, dup_frac=0.05),
}


@pytest.mark.parametrize("pad", [1, 8])
@pytest.mark.parametrize("name", list(WIDE))
def test_wide_window_conversion(name, pad):
    say("csr_to_wcsr wide windows", name, pad)
    coo = WIDE[name]()
    rp, c, v = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
    per_window = rp[np.minimum(np.arange(1, (coo.m + 63) // 64 + 1) * 64, coo.m)] - rp[np.arange(0, coo.m, 64)]
    assert (per_window > 4096).sum() >= 2
    ewp, ewc, evals = oracle.csr_to_wcsr(coo.m, coo.n, rp, c, v, 64, pad)
    wp, wc, vals, fill = sp.csr_to_wcsr(coo.m, coo.n, dev(rp), dev(c), dev(v), pad=pad)
    np.testing.assert_array_equal(host(wp), ewp)
    np.testing.assert_array_equal(host(wc), ewc)
    np.testing.assert_array_equal(host(vals).view(np.uint32), evals.view(np.uint32))
    B = gen.dense_matrix(coo.n, 4, 3)
    C = torch.full((coo.m, 4), float("nan"), device="cuda")
    sp.wcsr_spmm(coo.m, coo.n, wp, wc, vals, 1.0, dev(B), 0.0, C)
    ref, scale = oracle.wcsr_spmm(coo.m, 64, ewp, ewc, evals, B)
    assert_close(host(C), ref, scale, what="wcsr_spmm %s" % name)


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
    # the same checks inside a window of more than 4096 entries (converted by a workgroup of its own)
    coo3 = WIDE["wide_multipass"]()
    rp3, c3, v3 = oracle.coo_to_csr(coo3.m, coo3.n, coo3.row, coo3.col, coo3.val)
    i = 5
    assert rp3[i + 1] - rp3[i] >= 2 and rp3[64] - rp3[0] > 4096
    bad = c3.copy()
    bad[rp3[i]], bad[rp3[i] + 1] = c3[rp3[i] + 1], c3[rp3[i]]
    if bad[rp3[i]] != bad[rp3[i] + 1]:
        with pytest.raises(sp.SparseError) as e:
            sp.csr_to_wcsr(coo3.m, coo3.n, dev(rp3), dev(bad), dev(v3))
        assert e.value.code == 5
    bad = c3.copy()
    bad[rp3[i]] = coo3.n
    with pytest.raises(sp.SparseError) as e:
        sp.csr_to_wcsr(coo3.m, coo3.n, dev(rp3), dev(bad), dev(v3))
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


# --------------------------------------------------------------------------
# task split ([ASYNC] §4.2)
# --------------------------------------------------------------------------
def skewed():
    return gen.skewed_windows_coo(m=1500, n=40000, pool_median=48, pool_sigma=1.5, pool_max=4000, seed=3)


def task_case(name):
    if name == "skewed":
        if name not in _cache:
            coo = skewed()
            _cache[name] = (coo, oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val))
        return _cache[name]
    return case(name)


TASK_CASES = list(cases()) + ["skewed"]


def table_parts(t, nw):
    """(head, splits, tasks) read from the task table as the header lays it out."""
    raw = host(t.table)
    head = raw[:16].view(np.int32)
    splits = raw[256:256 + 16 * int(head[3])].view(np.int32).reshape(-1, 4)
    off = 256 + (16 * nw + 255) // 256 * 256
    tasks = raw[off:off + 16 * t.ntasks].view(np.int32).reshape(-1, 4)
    return head, splits, tasks


@pytest.mark.parametrize("task_cols", [32, 96, 512])
@pytest.mark.parametrize("name", TASK_CASES)
def test_task_table_bit_exact(name, task_cols):
    say("wcsr task table", name, task_cols)
    coo, (rp, c, v) = task_case(name)
    ewp, ewc, evals = oracle.csr_to_wcsr(coo.m, coo.n, rp, c, v, 64, 8)
    etasks, ewinfo, eslots = oracle.wcsr_tasks(ewp, task_cols)
    t = sp.wcsr_tasks(coo.m, dev(ewp), ewc.size, task_cols=task_cols)
    assert (t.ntasks, t.nslots) == (len(etasks), eslots)
    nw = ewp.size - 1
    head, splits, tasks = table_parts(t, nw)
    esplit = [[w, p, k, 0] for w, (p, k) in enumerate(ewinfo.tolist()) if p >= 0]
    assert head.tolist() == [len(etasks), eslots, 0, len(esplit)]
    assert splits.tolist() == esplit
    # launch order: widest first, equal widths in the oracle's (window, column) order
    order = np.argsort(-(etasks[:, 2] - etasks[:, 1]), kind="stable")
    np.testing.assert_array_equal(tasks, etasks[order])


@pytest.mark.parametrize("task_cols", [32, 512, 2048])
@pytest.mark.parametrize("N", [4, 32, 100, 192])
@pytest.mark.parametrize("name", TASK_CASES)
def test_wcsr_spmm_tasks(name, N, task_cols):
    say("wcsr_spmm_tasks", name, N, task_cols)
    coo, (rp, c, v) = task_case(name)
    ewp, ewc, evals = oracle.csr_to_wcsr(coo.m, coo.n, rp, c, v, 64, 8)
    wp, wc, vals = dev(ewp), dev(ewc), dev(evals)
    t = sp.wcsr_tasks(coo.m, wp, ewc.size, task_cols=task_cols)
    _, ewinfo, _ = oracle.wcsr_tasks(ewp, task_cols)
    whole = np.repeat(ewinfo[:, 0] < 0, 64)[:coo.m]  # rows of windows that are one task
    B = gen.dense_matrix(coo.n, N, 3)
    for alpha, beta in AB:
        C0 = gen.dense_matrix(coo.m, N, 4)
        C = dev(C0) if beta != 0.0 else torch.full((coo.m, N), float("nan"), device="cuda")
        sp.wcsr_spmm_tasks(coo.m, coo.n, t, wc, vals, alpha, dev(B), beta, C)
        ref, scale = oracle.wcsr_spmm(coo.m, 64, ewp, ewc, evals, B, alpha, beta, C0)
        got = host(C)
        assert_close(got, ref, scale, what="wcsr_spmm_tasks %s N=%d T=%d a=%g b=%g" % (name, N, task_cols, alpha,
                                                                                        beta))
        # windows that are one task: bit for bit the one-workgroup-per-window kernel
        C1 = dev(C0) if beta != 0.0 else torch.full((coo.m, N), float("nan"), device="cuda")
        sp.wcsr_spmm(coo.m, coo.n, wp, wc, vals, alpha, dev(B), beta, C1)
        np.testing.assert_array_equal(got[whole].view(np.uint32), host(C1)[whole].view(np.uint32))
    # reproducible: the same bits on a second call with a reused workspace
    work = torch.empty(max(t.workspace_bytes(N), 1), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(2):
        C = torch.zeros(coo.m, N, device="cuda")
        sp.wcsr_spmm_tasks(coo.m, coo.n, t, wc, vals, 1.0, dev(B), 0.0, C, work=work)
        outs.append(host(C).view(np.uint32).copy())
    np.testing.assert_array_equal(outs[0], outs[1])


def test_wcsr_tasks_errors():
    say("wcsr task split errors")
    coo, (rp, c, v) = task_case("skewed")
    ewp, ewc, evals = oracle.csr_to_wcsr(coo.m, coo.n, rp, c, v, 64, 8)
    wp, wc, vals = dev(ewp), dev(ewc), dev(evals)
    for bad_cols in (0, 48, -32):
        with pytest.raises(sp.SparseError) as e:
            sp.wcsr_tasks(coo.m, wp, ewc.size, task_cols=bad_cols)
        assert e.value.code == 5
    bad = ewp.copy()
    bad[3], bad[4] = bad[4], bad[3] - 1  # a window that ends before it starts
    with pytest.raises(sp.SparseError) as e:
        sp.wcsr_tasks(coo.m, dev(bad), ewc.size, task_cols=32)
    assert e.value.code == 3
    with pytest.raises(sp.SparseError) as e:  # window_ptr past total_cols
        sp.wcsr_tasks(coo.m, wp, ewc.size - 8, task_cols=32)
    assert e.value.code == 3
    t = sp.wcsr_tasks(coo.m, wp, ewc.size, task_cols=64)
    assert t.nslots > 0
    L = sp.lib()
    B = dev(gen.dense_matrix(coo.n, 32, 1))
    C = torch.full((coo.m, 32), float("nan"), device="cuda")
    need = t.workspace_bytes(32)
    work = torch.empty(need, dtype=torch.uint8, device="cuda")

    def call(ntasks=t.ntasks, nslots=t.nslots, wbytes=need, work_ptr=work.data_ptr()):
        return L.wcsr_spmm_tasks(coo.m, coo.n, t.table.data_ptr(), ntasks, nslots, wc.data_ptr(), vals.data_ptr(),
                                 32, 1.0, B.data_ptr(), 32, 0.0, C.data_ptr(), 32, work_ptr, wbytes, None)

    assert call(wbytes=need - 1) == 4
    assert call(work_ptr=None) == 1
    assert call(ntasks=(coo.m + 63) // 64 - 1) == 2
    # a workspace sized for fewer slots than the table needs: nothing is written
    fewer = t.nslots - 1
    assert call(nslots=fewer, wbytes=t.workspace_bytes(32)) == 0
    torch.cuda.synchronize()
    assert torch.isnan(C).all()
    assert call() == 0
    torch.cuda.synchronize()
    assert not torch.isnan(C).any()


def test_skewed_workload_task_split_sampled():
    """The 2^20-row skewed-window matrix (windows of 1 to 16384 compressed
    columns): task split with 2048 columns per task, N = 32 (the benchmarked
    call), checked against the oracle on every split window and on 200 sampled
    others."""
    say("wcsr task split, skewed workload")
    coo = gen.skewed_windows_coo(seed=0)
    rp, c, v = sp.csr_build_from_coo(coo.m, coo.n, dev(coo.row), dev(coo.col), dev(coo.val))
    wp, wc, vals, fill = sp.csr_to_wcsr(coo.m, coo.n, rp, c, v, pad=8)
    # the conversion, bit for bit (windows of up to 180 k entries take the wide-window kernel)
    ewp, ewc, evals = oracle.csr_to_wcsr(coo.m, coo.n, host(rp), host(c), host(v), 64, 8)
    np.testing.assert_array_equal(host(wp), ewp)
    np.testing.assert_array_equal(host(wc), ewc)
    np.testing.assert_array_equal(host(vals).view(np.uint32), evals.view(np.uint32))
    del ewc, evals
    t = sp.wcsr_tasks(coo.m, wp, wc.numel(), task_cols=2048)
    N = 32
    B = gen.dense_matrix(coo.n, N, 0)
    C = torch.full((coo.m, N), float("nan"), device="cuda")
    sp.wcsr_spmm_tasks(coo.m, coo.n, t, wc, vals, 1.0, dev(B), 0.0, C)
    hwp, hwc, hvals, got = host(wp), host(wc), host(vals), host(C)
    _, winfo, _ = oracle.wcsr_tasks(hwp, 2048)
    split = np.flatnonzero(winfo[:, 0] >= 0)
    assert split.size > 100
    rng = np.random.default_rng(0)
    others = rng.choice(np.flatnonzero(winfo[:, 0] < 0), size=200, replace=False)
    for w in np.concatenate([split, others]):
        q0, q1 = hwp[w], hwp[w + 1]
        r0, r1 = 64 * w, min(coo.m, 64 * w + 64)
        ref, scale = oracle.wcsr_spmm(r1 - r0, 64, np.array([0, q1 - q0], np.int32), hwc[q0:q1], hvals[q0:q1], B)
        assert_close(got[r0:r1], ref, scale, what="skewed window %d" % w)


@pytest.mark.parametrize("seed", range(12))
def test_wcsr_tasks_random(seed):
    """Random shapes, pads, task widths, N and alpha / beta: the task table
    against the oracle's (widest first) and the product against the oracle."""
    rng = np.random.default_rng(100 + seed)
    m, n = int(rng.integers(1, 2500)), int(rng.integers(1, 6000))
    coo = gen.skewed_windows_coo(m=m, n=n, pool_median=int(rng.integers(4, 80)), pool_sigma=float(rng.uniform(0.5, 2.0)),
                                 pool_max=int(min(n, rng.integers(64, 4000))), seed=seed)
    pad = int(rng.choice([1, 2, 8, 32]))
    T = 32 * int(rng.integers(1, 33))
    N = 4 * int(rng.integers(1, 65))
    alpha, beta = float(rng.uniform(-2, 2)), float(rng.choice([0.0, rng.uniform(-2, 2)]))
    say("wcsr tasks random", seed, m, n, coo.nnz, pad, T, N)
    rp, c, v = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
    ewp, ewc, evals = oracle.csr_to_wcsr(coo.m, coo.n, rp, c, v, 64, pad)
    etasks, ewinfo, eslots = oracle.wcsr_tasks(ewp, T)
    t = sp.wcsr_tasks(coo.m, dev(ewp), ewc.size, task_cols=T)
    assert (t.ntasks, t.nslots) == (len(etasks), eslots)
    _, splits, tasks = table_parts(t, ewp.size - 1)
    order = np.argsort(-(etasks[:, 2] - etasks[:, 1]), kind="stable")
    np.testing.assert_array_equal(tasks, etasks[order])
    B = gen.dense_matrix(coo.n, N, seed)
    C0 = gen.dense_matrix(coo.m, N, seed + 1)
    C = dev(C0) if beta != 0.0 else torch.full((coo.m, N), float("nan"), device="cuda")
    sp.wcsr_spmm_tasks(coo.m, coo.n, t, dev(ewc), dev(evals), alpha, dev(B), beta, C)
    ref, scale = oracle.wcsr_spmm(coo.m, 64, ewp, ewc, evals, B, alpha, beta, C0)
    assert_close(host(C), ref, scale, what="wcsr tasks random seed %d" % seed)
