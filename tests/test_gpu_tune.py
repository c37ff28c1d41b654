"""Dispatch key, tuning cache and micro-autotune on the GPU: the key follows
the matrix's row-length profile, options cached for a key reach plan creation
(for that matrix version only), and the autotune times every candidate,
caches the fastest and the tuned plan stays exact."""
import math

import numpy as np
import pytest
import torch

import gen
import oracle
import spmm_csr_spmv_amd as sp
from gpu_util import assert_close, dev, gpu_csr, host, say

pytestmark = pytest.mark.gpu


def _matrix():
    coo = gen.ragged_coo(3000, 100000, seed=2, max_len=30, long_rows=(300, 5000, 2048))
    return coo, gpu_csr(coo)


def test_dispatch_key_follows_profile():
    say("dispatch key")
    coo, (rp, c, v) = _matrix()
    csc = sp.csr_to_csc(coo.m, coo.n, rp, c, v)
    plan = sp.Plan(coo.m, coo.n, rp, c, v, csc=csc)
    for transposed, ptr, rows, cols in ((False, host(rp), coo.m, coo.n), (True, host(csc[0]), coo.n, coo.m)):
        k = plan.dispatch_key(transposed=transposed, N=8, version=5)
        p = oracle.row_profile(ptr)
        assert (k.format, k.dtype, k.index_bits, k.transposed, k.arch) == (0, 0, 32, int(transposed), 950)
        assert (k.rows, k.cols, k.nnz, k.N, k.version) == (rows, cols, int(ptr[-1]), 8, 5)
        assert k.avg_len_q == math.floor(4 * math.log2(1 + p["mean"]))
        assert k.p95_len_q == math.floor(4 * math.log2(1 + p["p95"]))
        assert k.max_len_q == math.floor(4 * math.log2(1 + p["max"]))
        assert k.cv_q == math.floor(8 * p["cv"])


def test_cached_options_reach_plan_creation():
    say("tuning cache -> plan")
    coo, (rp, c, v) = _matrix()
    sp.tune_cache_clear()
    base = sp.Plan(coo.m, coo.n, rp, c, v, tuned=True)
    assert base.profile()["col_panels"] == 0 and base.profile()["sell_slots"] == 0   # defaults: neither
    key = base.dispatch_key()
    # options cached for another matrix version do not apply
    k7 = base.dispatch_key(version=7)
    sp.tune_cache_store(k7, use_sell=0, col_panels=4)
    assert sp.Plan(coo.m, coo.n, rp, c, v, tuned=True).profile()["col_panels"] == 0
    # options cached for this key (version 0, N = 1) do
    sp.tune_cache_store(key, use_sell=0, col_panels=4)
    tuned = sp.Plan(coo.m, coo.n, rp, c, v, tuned=True)
    assert tuned.profile()["col_panels"] == 4
    sp.tune_cache_store(key, use_sell=1, sell_sigma=64)
    assert sp.Plan(coo.m, coo.n, rp, c, v, tuned=True).profile()["sell_slots"] > 0
    # explicit options are never replaced
    assert sp.Plan(coo.m, coo.n, rp, c, v).profile()["sell_slots"] == 0
    x = gen.dense_vector(coo.n, 3)
    y = torch.full((coo.m,), float("nan"), device="cuda")
    sp.spmv(tuned, 1.0, dev(x), 0.0, y)
    ref, scale = oracle.spmv(host(rp), host(c), host(v), x)
    assert_close(host(y), ref, scale, what="tuned plan")
    sp.tune_cache_clear()


def test_autotune_times_candidates_and_caches_the_fastest():
    say("autotune")
    coo, (rp, c, v) = _matrix()
    sp.tune_cache_clear()
    x = dev(gen.dense_vector(coo.n, 4))
    best, ms, opts = sp.autotune_spmv(coo.m, coo.n, rp, c, v, x, reps=10, version=3)
    assert len(ms) == len(sp.DEFAULT_CANDIDATES) and all(t > 0 for t in ms)
    assert ms[best] == min(ms)
    assert opts == sp.options_dict(sp.plan_options(**sp.DEFAULT_CANDIDATES[best]))
    plan = sp.Plan(coo.m, coo.n, rp, c, v)
    assert sp.tune_cache_lookup(plan.dispatch_key(version=3)) == opts
    assert sp.tune_cache_lookup(plan.dispatch_key(version=0)) is None
    assert sp.tune_cache_size() == 1
    # the winner, used through the cache, is exact
    best0, _, opts0 = sp.autotune_spmv(coo.m, coo.n, rp, c, v, x, reps=5, candidates=[dict(use_sell=0, col_panels=8),
                                                                                     dict(use_sell=0, col_panels=0)])
    tuned = sp.Plan(coo.m, coo.n, rp, c, v, tuned=True)
    assert tuned.profile()["col_panels"] == (8 if best0 == 0 else 0)
    y = torch.full((coo.m,), float("nan"), device="cuda")
    sp.spmv(tuned, 1.0, x, 0.0, y)
    ref, scale = oracle.spmv(host(rp), host(c), host(v), host(x))
    assert_close(host(y), ref, scale, what="autotuned plan")
    sp.tune_cache_clear()
