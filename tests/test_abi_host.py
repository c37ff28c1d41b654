"""Host-only checks of the C ABI: the library loads, exports every function the
public header declares, and rejects bad arguments before touching a GPU.
No call here launches a kernel or reaches the device."""
import ctypes
import os
import re

import pytest

import spmm_csr_spmv_amd as sp

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "spmm_csr_spmv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("csr_build_from_coo", "csr_to_csc", "spmv", "spmv_t", "spmm", "bsr_spmm"):
        assert required in names
    assert sorted(sp.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(sp.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings_and_version():
    for code in range(9):
        s = sp.status_string(code)
        assert s.startswith("SP_")
    assert sp.status_string(99) == "unknown status"
    assert sp.sp_version() >= 100


def test_option_defaults():
    o = sp.plan_options()
    assert (o.group_nnz, o.wave_min, o.block_min, o.split_min, o.split_seg) == (2048, 256, 4096, 32768, 8192)
    assert (o.use_sell, o.sell_sigma, o.xcd_remap, o.col_panels, o.x_window_bits) == (-1, 1024, 1, -1, -1)
    assert o.spmm_phase_bits == -1


SZ = ctypes.c_size_t
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below returns before using it


@pytest.mark.parametrize("m,n,nnz", [(-1, 4, 4), (4, -1, 4), (4, 4, -1), (2 ** 31, 4, 4), (4, 4, 2 ** 31),
                                     (2 ** 31 - 1, 4, 4)])
def test_bufsize_rejects_bad_sizes(m, n, nnz):
    L = sp.lib()
    b = SZ()
    assert L.csr_build_from_coo_bufsize(m, n, nnz, ctypes.byref(b)) == 2
    assert L.csr_to_csc_bufsize(m, n, nnz, ctypes.byref(b)) == 2


def test_bufsize_null_and_growth():
    L = sp.lib()
    assert L.csr_build_from_coo_bufsize(4, 4, 4, None) == 1
    a, b = SZ(), SZ()
    assert L.csr_build_from_coo_bufsize(1000, 1000, 10_000, ctypes.byref(a)) == 0
    assert L.csr_build_from_coo_bufsize(1000, 1000, 20_000, ctypes.byref(b)) == 0
    assert b.value > a.value >= 8 * 2 * 10_000


def test_conversion_argument_errors():
    L = sp.lib()
    # NULL outputs
    assert L.csr_build_from_coo(4, 4, 3, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 20, None) == 1
    assert L.csr_to_csc(4, 4, 3, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == 1
    # missing workspace
    assert L.csr_build_from_coo(4, 4, 3, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 4
    assert L.csr_to_csc(4, 4, 3, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 4
    # sizes
    assert L.csr_build_from_coo(-2, 4, 3, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == 2


@pytest.mark.parametrize("field,value", [("group_nnz", 32), ("group_nnz", 8192), ("wave_min", 5000),
                                         ("block_min", 10), ("split_min", 100), ("split_seg", 8),
                                         ("use_sell", 2), ("use_sell", -2), ("sell_sigma", 0), ("xcd_remap", 3),
                                         ("col_panels", 3), ("col_panels", 16), ("col_panels", -2),
                                         ("x_window_bits", 4), ("x_window_bits", 16), ("x_window_bits", -2)])
def test_plan_rejects_bad_options(field, value):
    L = sp.lib()
    o = sp.plan_options()
    setattr(o, field, value)
    h = ctypes.c_void_p()
    assert L.sp_plan_create(ctypes.byref(h), 8, 8, 8, FAKE, FAKE, FAKE, None, None, None, ctypes.byref(o),
                            None) == 5
    assert not h.value


def test_plan_argument_errors():
    L = sp.lib()
    h = ctypes.c_void_p()
    assert L.sp_plan_create(None, 8, 8, 8, FAKE, FAKE, FAKE, None, None, None, None, None) == 1
    assert L.sp_plan_create(ctypes.byref(h), 8, 8, 8, None, FAKE, FAKE, None, None, None, None, None) == 1
    assert L.sp_plan_create(ctypes.byref(h), 8, 8, 8, FAKE, None, FAKE, None, None, None, None, None) == 1
    assert L.sp_plan_create(ctypes.byref(h), 8, 8, 8, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None) == 1
    assert L.sp_plan_create(ctypes.byref(h), 2 ** 31, 8, 8, FAKE, FAKE, FAKE, None, None, None, None, None) == 2
    b = SZ()
    assert L.sp_plan_workspace_size(None, 1, ctypes.byref(b)) == 1
    assert L.sp_plan_bind(None, FAKE, 100, 1, None) == 1
    assert L.sp_plan_profile(None, 0, None) == 1
    assert L.sp_plan_destroy(None) == 0
    assert L.spmv(None, 1.0, FAKE, 0.0, FAKE, None) == 1
    assert L.spmv_t(None, 1.0, FAKE, 0.0, FAKE, None) == 1
    assert L.spmm(None, 4, 1.0, FAKE, 4, 0.0, FAKE, 4, None) == 1


def test_bsr_argument_errors():
    L = sp.lib()
    b = SZ()
    assert L.bsr_spmm_bufsize(4, 4, 32, 8, 64, ctypes.byref(b)) == 5
    assert L.bsr_spmm_bufsize(4, 4, 64, 8, 64, ctypes.byref(b)) == 0
    assert L.bsr_spmm_bufsize(-1, 4, 64, 8, 64, ctypes.byref(b)) == 2
    args = dict(mb=4, kb=4, bs=64, nnzb=8, brow=FAKE, bcol=FAKE, bval=FAKE, N=128, B=FAKE, ldb=128, alpha=1.0,
                beta=0.0, C=FAKE, ldc=128)

    def call(**kw):
        a = dict(args, **kw)
        return L.bsr_spmm(a["mb"], a["kb"], a["bs"], a["nnzb"], a["brow"], a["bcol"], a["bval"], a["N"], a["B"],
                          a["ldb"], a["alpha"], a["beta"], a["C"], a["ldc"], None, 0, None)

    assert call(bs=16) == 5
    assert call(N=100, ldb=104, ldc=104) == 5     # N not a multiple of 8
    assert call(ldb=132) == 5                     # ldb not a multiple of 8
    assert call(ldb=100) == 2                     # ldb < N
    assert call(ldc=64) == 2                      # ldc < N
    assert call(B=None) == 1
    assert call(C=ctypes.c_void_p(0x1004)) == 5   # misaligned C
    assert call(mb=2 ** 31) == 2


def test_csr_to_bsr_and_bsr_spmv_argument_errors():
    L = sp.lib()
    b = SZ()
    assert L.csr_to_bsr_bufsize(100, 100, 50, 3, ctypes.byref(b)) == 5      # block size not supported
    assert L.csr_to_bsr_bufsize(100, 100, 50, 8, ctypes.byref(b)) == 0 and b.value > 0
    assert L.csr_to_bsr_bufsize(-1, 100, 50, 8, ctypes.byref(b)) == 2
    assert L.csr_to_bsr_bufsize(100, 100, 50, 8, None) == 1
    nnzb, fill = ctypes.c_int64(), ctypes.c_double()
    # analyze: missing outputs, missing or small workspace, bad block size (no GPU work is reached)
    assert L.csr_to_bsr_analyze(10, 10, 5, FAKE, FAKE, 2, 0.0, None, ctypes.byref(nnzb), ctypes.byref(fill),
                                FAKE, 1 << 20, None) == 1
    assert L.csr_to_bsr_analyze(10, 10, 5, FAKE, FAKE, 2, 0.0, FAKE, ctypes.byref(nnzb), ctypes.byref(fill),
                                None, 0, None) == 4
    assert L.csr_to_bsr_analyze(10, 10, 5, FAKE, FAKE, 5, 0.0, FAKE, ctypes.byref(nnzb), ctypes.byref(fill),
                                FAKE, 1 << 20, None) == 5
    # fill: bad output type, missing arrays, misaligned fp32 blocks
    assert L.csr_to_bsr_fill(10, 10, 5, FAKE, FAKE, FAKE, 4, FAKE, 3, FAKE, FAKE, 2, None) == 5
    assert L.csr_to_bsr_fill(10, 10, 5, FAKE, FAKE, FAKE, 4, FAKE, 3, None, FAKE, 0, None) == 1
    assert L.csr_to_bsr_fill(10, 10, 5, FAKE, FAKE, FAKE, 4, FAKE, 3, FAKE, ctypes.c_void_p(0x1004), 0, None) == 5
    # bsr_spmv: empty output is a no-op, then argument checks
    assert L.bsr_spmv(0, 10, 4, 0, None, None, None, 1.0, None, 0.0, None, None) == 0
    assert L.bsr_spmv(10, 10, 3, 2, FAKE, FAKE, FAKE, 1.0, FAKE, 0.0, FAKE, None) == 5
    assert L.bsr_spmv(10, 10, 4, 2, FAKE, FAKE, FAKE, 1.0, FAKE, 0.0, None, None) == 1
    assert L.bsr_spmv(10, 10, 4, 2, FAKE, FAKE, ctypes.c_void_p(0x1004), 1.0, FAKE, 0.0, FAKE, None) == 5
    assert L.bsr_spmv(10, 10, 4, 2, FAKE, FAKE, FAKE, 1.0, ctypes.c_void_p(0x1004), 0.0, FAKE, None) == 5
    assert L.bsr_spmv(2 ** 31, 10, 4, 2, FAKE, FAKE, FAKE, 1.0, FAKE, 0.0, FAKE, None) == 2


def _key(**kw):
    k = sp.sp_dispatch_key()
    fields = dict(format=0, dtype=0, index_bits=32, transposed=0, rows=1000, cols=900, nnz=12345, N=1, arch=950,
                  avg_len_q=14, p95_len_q=20, max_len_q=30, cv_q=6, version=0)
    fields.update(kw)
    for f, v in fields.items():
        setattr(k, f, v)
    return k


def test_tune_cache_store_lookup_version_and_clear():
    sp.tune_cache_clear()
    assert sp.tune_cache_size() == 0
    assert sp.tune_cache_lookup(_key()) is None
    sp.tune_cache_store(_key(), use_sell=1, sell_sigma=64)
    got = sp.tune_cache_lookup(_key())
    assert got["use_sell"] == 1 and got["sell_sigma"] == 64 and got["group_nnz"] == 2048
    # any differing field of the key misses: a new matrix version, another N, the transpose
    assert sp.tune_cache_lookup(_key(version=1)) is None
    assert sp.tune_cache_lookup(_key(N=8)) is None
    assert sp.tune_cache_lookup(_key(transposed=1)) is None
    sp.tune_cache_store(_key(version=1), col_panels=8, use_sell=0)
    assert sp.tune_cache_size() == 2
    assert sp.tune_cache_lookup(_key(version=1))["col_panels"] == 8
    assert sp.tune_cache_lookup(_key())["use_sell"] == 1   # the other version is untouched
    # invalid options are refused, nothing is stored
    with pytest.raises(sp.SparseError):
        sp.tune_cache_store(_key(version=2), col_panels=3)
    assert sp.tune_cache_size() == 2
    sp.tune_cache_clear()
    assert sp.tune_cache_size() == 0 and sp.tune_cache_lookup(_key()) is None


def test_autotune_argument_errors():
    L = sp.lib()
    o = sp.plan_options()
    best, ms, b = ctypes.c_int32(), (ctypes.c_float * 4)(), SZ()
    assert L.sp_autotune_spmv(10, 10, 5, FAKE, FAKE, FAKE, ctypes.byref(o), 0, FAKE, FAKE, 5, 0, FAKE, 1 << 20,
                              ctypes.byref(best), ms, None) == 2       # no candidate
    assert L.sp_autotune_spmv(10, 10, 5, FAKE, FAKE, FAKE, ctypes.byref(o), 1, FAKE, FAKE, 0, 0, FAKE, 1 << 20,
                              ctypes.byref(best), ms, None) == 2       # no repetition
    assert L.sp_autotune_spmv(10, 10, 5, FAKE, FAKE, FAKE, ctypes.byref(o), 1, FAKE, FAKE, 5, 0, FAKE, 1 << 20,
                              None, ms, None) == 1
    assert L.sp_autotune_workspace_size(10, 10, 5, FAKE, FAKE, FAKE, ctypes.byref(o), 17, ctypes.byref(b), None) == 2
    assert L.sp_plan_dispatch_key(None, 0, 1, 0, None) == 1


def test_wcsr_argument_errors():
    L = sp.lib()
    b = SZ()
    assert L.csr_to_wcsr_bufsize(100, 100, 50, ctypes.byref(b)) == 0 and b.value > 0
    assert L.csr_to_wcsr_bufsize(-1, 100, 50, ctypes.byref(b)) == 2
    tot, fill = ctypes.c_int64(), ctypes.c_double()
    assert L.csr_to_wcsr_analyze(10, 10, 5, FAKE, FAKE, 3, FAKE, ctypes.byref(tot), ctypes.byref(fill), FAKE,
                                 1 << 20, None) == 5                 # pad not supported
    assert L.csr_to_wcsr_analyze(10, 10, 5, FAKE, FAKE, 8, None, ctypes.byref(tot), ctypes.byref(fill), FAKE,
                                 1 << 20, None) == 1
    assert L.csr_to_wcsr_analyze(10, 10, 5, FAKE, FAKE, 8, FAKE, ctypes.byref(tot), ctypes.byref(fill), None, 0,
                                 None) == 4
    assert L.csr_to_wcsr_fill(10, 10, 5, FAKE, FAKE, FAKE, FAKE, 8, None, FAKE, None) == 1
    assert L.wcsr_spmm(0, 10, None, None, None, 4, 1.0, None, 4, 0.0, None, 4, None) == 0   # no rows: no-op
    assert L.wcsr_spmm(10, 10, FAKE, FAKE, FAKE, 6, 1.0, FAKE, 6, 0.0, FAKE, 6, None) == 5  # N % 4 != 0
    assert L.wcsr_spmm(10, 10, FAKE, FAKE, FAKE, 8, 1.0, FAKE, 4, 0.0, FAKE, 8, None) == 2  # ldb < N
    assert L.wcsr_spmm(10, 10, FAKE, FAKE, FAKE, 8, 1.0, ctypes.c_void_p(0x1004), 8, 0.0, FAKE, 8, None) == 5
    assert L.wcsr_spmm(10, 10, None, FAKE, FAKE, 8, 1.0, FAKE, 8, 0.0, FAKE, 8, None) == 1


def test_wcsr_task_split_argument_errors():
    L = sp.lib()
    b = SZ()
    nt, ns = ctypes.c_int64(), ctypes.c_int64()
    assert L.wcsr_tasks_bufsize(100, 1000, 512, ctypes.byref(b)) == 0 and b.value > 0
    assert L.wcsr_tasks_bufsize(100, 1000, 48, ctypes.byref(b)) == 5   # not a multiple of 32
    assert L.wcsr_tasks_bufsize(100, 1000, 0, ctypes.byref(b)) == 5
    assert L.wcsr_tasks_bufsize(100, -1, 32, ctypes.byref(b)) == 2
    assert L.wcsr_tasks_bufsize(100, 1000, 32, None) == 1
    assert L.wcsr_tasks_build(0, None, 0, 32, None, 0, ctypes.byref(nt), ctypes.byref(ns), None) == 0
    assert (nt.value, ns.value) == (0, 0)
    assert L.wcsr_tasks_build(100, None, 1000, 32, FAKE, 1 << 20, ctypes.byref(nt), ctypes.byref(ns), None) == 1
    assert L.wcsr_tasks_build(100, FAKE, 1000, 32, FAKE, 16, ctypes.byref(nt), ctypes.byref(ns), None) == 4
    assert L.wcsr_tasks_build(100, FAKE, 1000, 32, ctypes.c_void_p(0x1008), 1 << 20, ctypes.byref(nt),
                              ctypes.byref(ns), None) == 5        # table not 16-byte aligned
    assert L.wcsr_tasks_build(100, FAKE, 1000, 32, FAKE, 1 << 20, None, ctypes.byref(ns), None) == 1
    assert L.wcsr_spmm_tasks_bufsize(0, 32, ctypes.byref(b)) == 0 and b.value == 0
    assert L.wcsr_spmm_tasks_bufsize(3, 32, ctypes.byref(b)) == 0 and b.value >= 3 * 64 * 32 * 4
    assert L.wcsr_spmm_tasks_bufsize(-1, 32, ctypes.byref(b)) == 2
    # 2^31 - 1 slots of 64 x (2^31 - 1) floats do not fit in size_t
    assert L.wcsr_spmm_tasks_bufsize(2 ** 31 - 1, 2 ** 31 - 1, ctypes.byref(b)) == 2

    def call(m=100, ntasks=2, nslots=0, N=8, ldb=8, table=FAKE, work=None, wbytes=0, B=FAKE):
        return L.wcsr_spmm_tasks(m, 10, table, ntasks, nslots, FAKE, FAKE, N, 1.0, B, ldb, 0.0, FAKE, N, work,
                                 wbytes, None)

    assert call(m=0) == 0                       # no rows: no-op
    assert call(N=6, ldb=6) == 5                # N % 4 != 0
    assert call(ldb=4) == 2                     # ldb < N
    assert call(ntasks=1) == 2                  # fewer tasks than the 2 windows of 100 rows
    assert call(table=None) == 1
    assert call(nslots=2) == 1                  # slots but no workspace
    assert call(nslots=2, work=FAKE, wbytes=100) == 4
    assert call(B=ctypes.c_void_p(0x1004)) == 5


def test_view_argument_errors():
    L = sp.lib()
    v = ctypes.c_void_p()
    assert L.sp_plan_view_create(None, ctypes.byref(v)) == 1
    assert L.sp_plan_view_create(FAKE, None) == 1
    assert L.sp_plan_destroy(None) == 0


def test_noalloc_conversion_refuses_before_work():
    L = sp.lib()
    b = SZ()
    # the static scratch holds 64 MiB: a conversion needing more is refused
    assert L.csr_build_from_coo_bufsize(1000, 1000, 5_000_000, ctypes.byref(b)) == 0 and b.value > 64 << 20
    assert L.csr_build_from_coo_noalloc(1000, 1000, 5_000_000, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 4
    assert L.csr_build_from_coo_noalloc(-1, 4, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert L.csr_build_from_coo_noalloc(4, 4, 3, FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == 1
