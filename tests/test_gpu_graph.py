"""The products captured in a HIP graph (torch.cuda.CUDAGraph around the C ABI
calls) and replayed several times, with eager work and synchronisations
between the replays: every replay must equal the eager result bit for bit
(the kernels are deterministic and allocate nothing while running)."""
import numpy as np
import pytest
import torch

import gen
import oracle
import spmm_csr_spmv_amd as sp
from gpu_util import dev, say

pytestmark = pytest.mark.gpu


def _replays_match(run, outs, replays=3):
    """run() issues the products into `outs`; capture it, then compare each
    replay with an eager run made between the replays."""
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for k in range(replays):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        for o in outs:
            o.fill_(float("nan"))
        run()  # eager
        torch.cuda.synchronize()
        for a, b in zip(got, outs):
            assert torch.equal(a, b), "replay %d differs from the eager result" % k


@pytest.mark.parametrize("bins", [dict(), dict(use_sell=0, col_panels=4, wave_min=8, block_min=20, split_min=40,
                                               split_seg=16), dict(use_sell=1, sell_sigma=64),
                                  dict(use_sell=0, x_window_bits=6),
                                  dict(wave_min=0, block_min=0, split_min=0, split_seg=16),
                                  dict(spmm_phase_bits=6)])  # SpMM through the phase-swept copy
def test_spmv_spmv_t_spmm_graph_replays(bins):
    say("graph replays", bins)
    coo = gen.ragged_coo(1500, 900, seed=2, max_len=30, long_rows=(300, 800, 257))
    rp, c, v = sp.csr_build_from_coo(coo.m, coo.n, dev(coo.row), dev(coo.col), dev(coo.val))
    csc = sp.csr_to_csc(coo.m, coo.n, rp, c, v)
    plan = sp.Plan(coo.m, coo.n, rp, c, v, csc=csc, max_N=8, **bins)
    if "spmm_phase_bits" in bins:
        assert plan.profile()["spmm_phase_bits"] == bins["spmm_phase_bits"]
    x = dev(gen.dense_vector(coo.n, 1))
    u = dev(gen.dense_vector(coo.m, 2))
    B = dev(gen.dense_matrix(coo.n, 8, 3))
    y = torch.empty(coo.m, device="cuda")
    z = torch.empty(coo.n, device="cuda")
    C = torch.empty(coo.m, 8, device="cuda")

    def run():
        sp.spmv(plan, 1.0, x, 0.0, y)
        sp.spmv_t(plan, 2.0, u, 0.0, z)
        sp.spmm(plan, 1.0, B, 0.0, C)

    _replays_match(run, [y, z, C])
    # and the replayed result is the right one
    hrp, hc, hv = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
    ref, scale = oracle.spmv(hrp, hc, hv, x.cpu().numpy())
    assert np.all(np.abs(y.cpu().numpy() - ref) <= 1e-5 * scale + 1e-30)


def test_x_window_long_rows_graph_replays():
    """Rows longer than a row chunk are finished by the workgroup that stores
    their last segment sum, through an arrival counter the kernel puts back
    to zero: every replay and every eager call gives the same result, and it
    is the oracle's."""
    say("graph replays, x windows with long rows")
    coo = gen.ragged_coo(3000, 100000, seed=21, max_len=20, long_rows=(40000, 30721, 15361))
    rp, c, v = sp.csr_build_from_coo(coo.m, coo.n, dev(coo.row), dev(coo.col), dev(coo.val))
    plan = sp.Plan(coo.m, coo.n, rp, c, v, use_sell=0, x_window_bits=12)
    assert plan.profile()["x_window_bits"] == 12
    x = dev(gen.dense_vector(coo.n, 1))
    y = torch.empty(coo.m, device="cuda")

    def run():
        sp.spmv(plan, 1.0, x, 0.0, y)

    _replays_match(run, [y], replays=4)
    hrp, hc, hv = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
    assert np.diff(hrp).max() == 40000
    ref, scale = oracle.spmv(hrp, hc, hv, x.cpu().numpy())
    assert np.all(np.abs(y.cpu().numpy() - ref) <= 1e-5 * scale + 1e-30)


def test_bsr_spmv_and_bsr_spmm_graph_replays():
    say("graph replays, BSR")
    coo = gen.block_sparse_coo(mb=6, kb=5, bs=64, density=0.4, std=1.0, seed=7)
    rp, c, v = sp.csr_build_from_coo(coo.m, coo.n, dev(coo.row), dev(coo.col), dev(coo.val))
    brp, bcol, bval, _ = sp.csr_to_bsr(coo.m, coo.n, rp, c, v, 64)
    _, _, bval16, _ = sp.csr_to_bsr(coo.m, coo.n, rp, c, v, 64, out="bf16")
    x = dev(gen.dense_vector(coo.n, 4))
    B = dev(gen.bf16_matrix(coo.n, 256, seed=5).view(np.int16))
    y = torch.empty(coo.m, device="cuda")
    C = torch.empty(coo.m, 256, device="cuda")

    def run():
        sp.bsr_spmv(coo.m, coo.n, 64, brp, bcol, bval, 1.0, x, 0.0, y)
        sp.bsr_spmm(6, 5, 64, brp, bcol, bval16, B, 1.0, 0.0, C)

    _replays_match(run, [y, C])


def test_wcsr_spmm_graph_replays():
    say("graph replays, WCSR")
    coo = gen.clustered_coo(m=2000, n=30000, seed=8)
    rp, c, v = sp.csr_build_from_coo(coo.m, coo.n, dev(coo.row), dev(coo.col), dev(coo.val))
    wp, wc, vals, _ = sp.csr_to_wcsr(coo.m, coo.n, rp, c, v)
    B = dev(gen.dense_matrix(coo.n, 32, 6))
    C = torch.empty(coo.m, 32, device="cuda")

    def run():
        sp.wcsr_spmm(coo.m, coo.n, wp, wc, vals, 1.0, B, 0.0, C)

    _replays_match(run, [C])


def test_wcsr_spmm_tasks_graph_replays():
    """The task-split windowed SpMM (counter clear and product) captured and replayed."""
    say("graph replays, WCSR task split")
    coo = gen.skewed_windows_coo(m=1500, n=40000, pool_median=48, pool_sigma=1.5, pool_max=4000, seed=3)
    rp, c, v = sp.csr_build_from_coo(coo.m, coo.n, dev(coo.row), dev(coo.col), dev(coo.val))
    wp, wc, vals, _ = sp.csr_to_wcsr(coo.m, coo.n, rp, c, v)
    t = sp.wcsr_tasks(coo.m, wp, wc.numel(), task_cols=64)
    assert t.nslots > 0
    B = dev(gen.dense_matrix(coo.n, 32, 6))
    C = torch.empty(coo.m, 32, device="cuda")
    work = torch.empty(t.workspace_bytes(32), dtype=torch.uint8, device="cuda")

    def run():
        sp.wcsr_spmm_tasks(coo.m, coo.n, t, wc, vals, 1.0, B, 0.0, C, work=work)

    _replays_match(run, [C])


def test_view_products_graph_replays():
    """A view's products (its own scratch: split partials and counters, x-window
    products) captured and replayed like the plan's."""
    say("graph replays on a view")
    coo = gen.ragged_coo(1500, 900, seed=5, max_len=30, long_rows=(300, 800, 257))
    rp, c, v = sp.csr_build_from_coo(coo.m, coo.n, dev(coo.row), dev(coo.col), dev(coo.val))
    csc = sp.csr_to_csc(coo.m, coo.n, rp, c, v)
    for bins in (dict(use_sell=0, x_window_bits=6), dict(wave_min=0, block_min=0, split_min=0, split_seg=16)):
        plan = sp.Plan(coo.m, coo.n, rp, c, v, csc=csc, max_N=8, **bins)
        view = plan.view(max_N=8)
        x = dev(gen.dense_vector(coo.n, 1))
        u = dev(gen.dense_vector(coo.m, 2))
        B = dev(gen.dense_matrix(coo.n, 8, 3))
        y = torch.empty(coo.m, device="cuda")
        z = torch.empty(coo.n, device="cuda")
        C = torch.empty(coo.m, 8, device="cuda")

        def run():
            sp.spmv(view, 1.0, x, 0.0, y)
            sp.spmv_t(view, 2.0, u, 0.0, z)
            sp.spmm(view, 1.0, B, 0.0, C)

        _replays_match(run, [y, z, C])
        hrp, hc, hv = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
        ref, scale = oracle.spmv(hrp, hc, hv, x.cpu().numpy())
        assert np.all(np.abs(y.cpu().numpy() - ref) <= 1e-5 * scale + 1e-30)
        view.destroy()
        plan.destroy()
