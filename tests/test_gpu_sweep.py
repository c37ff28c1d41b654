"""Phase-swept SpMM (N in {4, 8, 16}) against the oracle, through the C ABI.

The plan's copy cuts the columns into phases of 2^b columns; each workgroup
keeps 2048 rows of C in LDS and sweeps the phases in order, each wave summing
its 256 rows in a fixed order.  These cases cover several phase widths (many
phases, one phase), row counts that are not a multiple of 2048 (a partial last
block, waves with no rows), rows far longer than a wave step, empty rows,
duplicates, alpha/beta, a leading dimension above N, bitwise determinism and
the automatic choice."""
import numpy as np
import pytest
import torch

import gen
import oracle
import spmm_csr_spmv_amd as sp
from gpu_util import assert_close, dev, host, say

pytestmark = pytest.mark.gpu

_cases = {}


def case(name):
    if name not in _cases:
        coo = {
            "ragged_long": lambda: gen.ragged_coo(5000, 9000, seed=2, max_len=30,
                                                  long_rows=(300, 5000, 9000, 2048, 257)),
            "tall_dups": lambda: gen.ragged_coo(2049, 40000, seed=8, max_len=50, empty_frac=0.3, dup_frac=0.1),
            "tiny": lambda: gen.ragged_coo(37, 70, seed=4, max_len=12, empty_frac=0.3),
        }[name]()
        _cases[name] = (coo, oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val))
    return _cases[name]


@pytest.mark.parametrize("bits", [5, 8, 14])
@pytest.mark.parametrize("N", [4, 8, 16])
@pytest.mark.parametrize("name", ["ragged_long", "tall_dups", "tiny"])
def test_sweep_spmm(name, N, bits):
    say("sweep", name, N, bits)
    coo, (rp, c, v) = case(name)
    plan = sp.Plan(coo.m, coo.n, dev(rp), dev(c), dev(v), max_N=N, spmm_phase_bits=bits)
    assert plan.profile()["spmm_phase_bits"] == bits
    B = gen.dense_matrix(coo.n, N, 31)
    dB = dev(B)
    for alpha, beta in [(1.0, 0.0), (0.5, -1.25)]:
        C0 = gen.dense_matrix(coo.m, N, 32)
        C = dev(C0) if beta != 0.0 else torch.full((coo.m, N), float("nan"), device="cuda")
        sp.spmm(plan, alpha, dB, beta, C)
        ref, scale = oracle.spmm(rp, c, v, B, alpha, beta, C0)
        assert_close(host(C), ref, scale, what="sweep %s N=%d bits=%d a=%g b=%g" % (name, N, bits, alpha, beta))


def test_sweep_strides_views_and_determinism():
    say("sweep strides and determinism")
    coo, (rp, c, v) = case("ragged_long")
    N, ld = 8, 20
    plan = sp.Plan(coo.m, coo.n, dev(rp), dev(c), dev(v), max_N=N, spmm_phase_bits=9)
    B = gen.dense_matrix(coo.n, ld, 5)
    ref, scale = oracle.spmm(rp, c, v, np.ascontiguousarray(B[:, :N]))
    dB = dev(B)
    L = sp.lib()
    outs = []
    for k in range(3):
        Cw = torch.full((coo.m, ld), -3.0, device="cuda")
        target = plan if k < 2 else plan.view(max_N=N)
        rc = L.spmm(target.handle, N, 1.0, sp._binding._ptr(dB), ld, 0.0, sp._binding._ptr(Cw), ld,
                    sp._binding._stream())
        assert rc == 0
        got = host(Cw)
        assert np.all(got[:, N:] == -3.0), "columns past N were written"
        assert_close(got[:, :N], ref, scale, what="strided sweep")
        outs.append(got[:, :N].view(np.uint32).copy())
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    # N outside {4, 8, 16} takes the row-bin kernels on the same plan
    B3 = gen.dense_matrix(coo.n, 3, 6)
    C3 = torch.full((coo.m, 3), float("nan"), device="cuda")
    sp.spmm(plan, 1.0, dev(B3), 0.0, C3)
    r3, s3 = oracle.spmm(rp, c, v, B3)
    assert_close(host(C3), r3, s3, what="N=3 on a sweep plan")


def test_sweep_automatic_rule():
    """Built by default for max_N = 8 when B passes 8 MiB and the columns spread;
    not for max_N = 32, nor for narrow B."""
    say("sweep automatic rule")
    m, n = 20000, 300000  # B at N = 8: 9.6 MB
    coo = gen.ragged_coo(m, n, seed=12, max_len=40, empty_frac=0.1)
    rp, c, v = oracle.coo_to_csr(coo.m, coo.n, coo.row, coo.col, coo.val)
    g = (dev(rp), dev(c), dev(v))
    p8 = sp.Plan(m, n, *g, max_N=8)
    assert p8.profile()["spmm_phase_bits"] == 14  # 2^14 rows of B at N = 8: 512 KiB slices
    assert sp.Plan(m, n, *g, max_N=32).profile()["spmm_phase_bits"] == 0
    assert sp.Plan(m, n, *g, max_N=8, spmm_phase_bits=0).profile()["spmm_phase_bits"] == 0
    B = gen.dense_matrix(n, 8, 3)
    C = torch.full((m, 8), float("nan"), device="cuda")
    sp.spmm(p8, 1.0, dev(B), 0.0, C)
    ref, scale = oracle.spmm(rp, c, v, B)
    assert_close(host(C), ref, scale, what="automatic sweep")
    small = gen.ragged_coo(3000, 5000, seed=13, max_len=40)
    r2, c2, v2 = oracle.coo_to_csr(small.m, small.n, small.row, small.col, small.val)
    assert sp.Plan(small.m, small.n, dev(r2), dev(c2), dev(v2), max_N=8).profile()["spmm_phase_bits"] == 0
