"""Streams and plan views, through the C ABI, against the oracle.

A plan's tables are read-only after bind; what a product writes besides its
output (split-row partials and arrival counters, panel row sums, x-window
products) lives in the per-call scratch of the plan or view it runs on
(「CUDA LSMR 专栏（二）」 §5.1: set up once, each call only swaps vectors).
These tests run products of two views of one plan at the same time on two
streams, and conversions and plans on a side stream."""
import numpy as np
import pytest
import torch

import gen
import oracle
import spmm_csr_spmv_amd as sp
from gpu_util import BINS, assert_close, dev, host, say

pytestmark = pytest.mark.gpu

# paths whose products use per-call scratch: split partials + counters, the
# panel sums, the x-window products and long-row partials
VIEW_BINS = ["all_split", "mixed_small", "ps8_split", "xw8", "xw15", "default", "sweep8"]


def _matrix(seed=1):
    coo = gen.ragged_coo(3000, 2500, seed=seed, max_len=60, long_rows=(900, 2400, 1300), dup_frac=0.05)
    rp, c, v = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
    cp, ri, cv = oracle.csr_to_csc(coo.m, coo.n, rp, c, v)
    return coo, (rp, c, v), (cp, ri, cv)


def test_conversions_and_plan_on_side_stream():
    say("side stream conversions")
    coo, (rp, c, v), (cp, ri, cv) = _matrix(3)
    s2 = torch.cuda.Stream()
    d_row, d_col, d_val = dev(coo.row), dev(coo.col), dev(coo.val)
    torch.cuda.synchronize()
    with torch.cuda.stream(s2):
        g = sp.csr_build_from_coo(coo.m, coo.n, d_row, d_col, d_val, stream=s2)
        gt = sp.csr_to_csc(coo.m, coo.n, *g, stream=s2)
        plan = sp.Plan(coo.m, coo.n, *g, csc=gt, stream=s2, **BINS["all_split"])
        # scratch that the allocator could hand out to the side stream's next work
        junk = [torch.full((1 << 16,), 7.0, device="cuda") for _ in range(8)]
        x = dev(gen.dense_vector(coo.n, 5))
        y = torch.full((coo.m,), float("nan"), device="cuda")
        sp.spmv(plan, 1.0, x, 0.0, y, stream=s2)
        del junk
    s2.synchronize()
    np.testing.assert_array_equal(host(g[0]), rp)
    np.testing.assert_array_equal(host(g[1]), c)
    np.testing.assert_array_equal(host(g[2]).view(np.uint32), v.view(np.uint32))
    np.testing.assert_array_equal(host(gt[0]), cp)
    np.testing.assert_array_equal(host(gt[1]), ri)
    np.testing.assert_array_equal(host(gt[2]).view(np.uint32), cv.view(np.uint32))
    ref, scale = oracle.spmv(rp, c, v, gen.dense_vector(coo.n, 5))
    assert_close(host(y), ref, scale, what="spmv on side stream")


@pytest.mark.parametrize("bins", VIEW_BINS)
def test_two_views_two_streams(bins):
    say("views", bins)
    coo, (rp, c, v), (cp, ri, cv) = _matrix(1)
    plan = sp.Plan(coo.m, coo.n, dev(rp), dev(c), dev(v), csc=(dev(cp), dev(ri), dev(cv)), max_N=8, **BINS[bins])
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    views = [plan.view(max_N=8, stream=s) for s in streams]
    assert views[0].workspace_bytes <= plan.workspace_bytes
    xs = [gen.dense_vector(coo.n, 40 + k) for k in range(2)]
    us = [gen.dense_vector(coo.m, 50 + k) for k in range(2)]
    Bs = [gen.dense_matrix(coo.n, 8, 60 + k) for k in range(2)]
    dx, du, dB = [dev(a) for a in xs], [dev(a) for a in us], [dev(a) for a in Bs]
    reps = 6
    ys = [[torch.empty(coo.m, device="cuda") for _ in range(reps)] for _ in range(2)]
    zs = [[torch.empty(coo.n, device="cuda") for _ in range(reps)] for _ in range(2)]
    Cs = [torch.empty(coo.m, 8, device="cuda") for _ in range(2)]
    torch.cuda.synchronize()
    # interleave the launches so that both streams' kernels overlap on the GPU
    for r in range(reps):
        for k in range(2):
            with torch.cuda.stream(streams[k]):
                sp.spmv(views[k], 1.0, dx[k], 0.0, ys[k][r], stream=streams[k])
                sp.spmv_t(views[k], 1.0, du[k], 0.0, zs[k][r], stream=streams[k])
    for k in range(2):
        with torch.cuda.stream(streams[k]):
            sp.spmm(views[k], 1.0, dB[k], 0.0, Cs[k], stream=streams[k])
    torch.cuda.synchronize()
    for k in range(2):
        ref, scale = oracle.spmv(rp, c, v, xs[k])
        ref_t, scale_t = oracle.spmv(cp, ri, cv, us[k])
        first = host(ys[k][0]).view(np.uint32).copy()
        for r in range(reps):
            assert_close(host(ys[k][r]), ref, scale, what="view %d spmv rep %d %s" % (k, r, bins))
            assert_close(host(zs[k][r]), ref_t, scale_t, what="view %d spmv_t rep %d %s" % (k, r, bins))
            assert np.array_equal(host(ys[k][r]).view(np.uint32), first), "view results differ between reps"
        refC, scC = oracle.spmm(rp, c, v, Bs[k])
        assert_close(host(Cs[k]), refC, scC, what="view %d spmm %s" % (k, bins))
    # the plan itself still works after its views ran (its counters untouched)
    y = torch.empty(coo.m, device="cuda")
    sp.spmv(plan, 1.0, dx[0], 0.0, y)
    ref, scale = oracle.spmv(rp, c, v, xs[0])
    assert_close(host(y), ref, scale, what="plan after views %s" % bins)


def test_view_lifetime_rules():
    say("view lifetime")
    coo, (rp, c, v), _ = _matrix(2)
    plan = sp.Plan(coo.m, coo.n, dev(rp), dev(c), dev(v), **BINS["all_split"])
    view = plan.view()
    assert view.profile()["nnz"] == plan.profile()["nnz"]
    # a plan with a live view is not freed
    with pytest.raises(sp.SparseError) as e:
        plan.destroy()
    assert e.value.code == 7
    # re-binding the plan retires the view until it is bound again
    L = sp.lib()
    assert L.sp_plan_bind(plan.handle, sp._binding._ptr(plan.work), plan.workspace_bytes, 1, None) == 0
    x, y = dev(gen.dense_vector(coo.n, 9)), torch.empty(coo.m, device="cuda")
    with pytest.raises(sp.SparseError) as e:
        sp.spmv(view, 1.0, x, 0.0, y)
    assert e.value.code == 7
    assert L.sp_plan_bind(view.handle, sp._binding._ptr(view.work), view.workspace_bytes, 1, None) == 0
    sp.spmv(view, 1.0, x, 0.0, y)
    ref, scale = oracle.spmv(rp, c, v, gen.dense_vector(coo.n, 9))
    assert_close(host(y), ref, scale, what="rebound view")
    # spmm above the view's max_N is refused like the plan's
    with pytest.raises(sp.SparseError) as e:
        sp.spmm(view, 1.0, dev(gen.dense_matrix(coo.n, 4, 1)), 0.0, torch.empty(coo.m, 4, device="cuda"))
    assert e.value.code == 2
    view.destroy()
    plan.destroy()


def test_wcsr_task_split_two_streams():
    """One WCSR task table (read-only after the build) on two streams at the
    same time, each with its own partial-tile workspace: every repetition
    equals the single-stream result bit for bit and the oracle within
    tolerance."""
    say("wcsr task split, two streams")
    coo = gen.skewed_windows_coo(m=1500, n=40000, pool_median=48, pool_sigma=1.5, pool_max=4000, seed=3)
    rp, c, v = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
    wp, wc, vals = oracle.csr_to_wcsr(coo.m, coo.n, rp, c, v, 64, 8)
    dwp, dwc, dvals = dev(wp), dev(wc), dev(vals)
    t = sp.wcsr_tasks(coo.m, dwp, wc.size, task_cols=64)
    assert t.nslots > 0
    N = 32
    Bs = [gen.dense_matrix(coo.n, N, 70 + k) for k in range(2)]
    dB = [dev(b) for b in Bs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    works = [torch.empty(t.workspace_bytes(N), dtype=torch.uint8, device="cuda") for _ in range(2)]
    single = []
    for k in range(2):
        C = torch.empty(coo.m, N, device="cuda")
        sp.wcsr_spmm_tasks(coo.m, coo.n, t, dwc, dvals, 1.0, dB[k], 0.0, C, work=works[k])
        single.append(host(C).view(np.uint32).copy())
    reps = 6
    Cs = [[torch.empty(coo.m, N, device="cuda") for _ in range(reps)] for _ in range(2)]
    torch.cuda.synchronize()
    for r in range(reps):
        for k in range(2):
            with torch.cuda.stream(streams[k]):
                sp.wcsr_spmm_tasks(coo.m, coo.n, t, dwc, dvals, 1.0, dB[k], 0.0, Cs[k][r], work=works[k],
                                   stream=streams[k])
    torch.cuda.synchronize()
    for k in range(2):
        ref, scale = oracle.wcsr_spmm(coo.m, 64, wp, wc, vals, Bs[k])
        for r in range(reps):
            got = host(Cs[k][r])
            assert np.array_equal(got.view(np.uint32), single[k]), "stream %d rep %d differs" % (k, r)
        assert_close(host(Cs[k][0]), ref, scale, what="wcsr tasks stream %d" % k)
