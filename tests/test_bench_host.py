"""bench.py on the host: it refuses more than one GPU, its algorithmic byte
and flop models give the figures of the measurement plan (8 bytes per entry,
the LSMR page's section 1 bound, plus the vectors once), and a committed HBM
traffic summary counts only while the kernels it was taken on are
unchanged."""
import json
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_byte_and_flop_models():
    # SpMV: values and column indices, row pointer, x and y once (y twice with beta)
    assert bench.spmv_bytes(4, 5, 7) == 8 * 7 + 4 * 5 + 4 * 5 + 4 * 4
    assert bench.spmv_bytes(4, 5, 7, True) - bench.spmv_bytes(4, 5, 7) == 4 * 4
    assert bench.spmv_flops(4, 7) == 14 and bench.spmv_flops(4, 7, True) == 22
    # the workloads' figures: power-law SpMV, one stencil direction (beta != 0)
    assert bench.spmv_bytes(1 << 22, 1 << 22, 46823854) == 424922484
    assert bench.spmv_bytes(4096000, 4096000, 109215352, True) == 939258820
    # SpMM reads B and writes C once
    assert bench.spmm_bytes(3, 4, 5, 8) == 8 * 5 + 4 * 4 + 4 * 4 * 8 + 4 * 3 * 8
    # BSR SpMM: 6554 bf16 64 x 64 blocks, B 16384 x 512 bf16, C fp32: about 104.0 MB, 27.49 GFLOP
    b = bench.bsr_bytes(256, 256, 64, 6554, 512)
    assert b == 2 * 6554 * 4096 + 4 * (6554 + 256 + 1) + 2 * 16384 * 512 + 4 * 16384 * 512
    assert abs(b / 1e6 - 104.0) < 0.1
    assert bench.bsr_flops(6554, 64, 512) == 2 * 6554 * 64 * 64 * 512  # 27.49 GFLOP
    # BSR SpMV with fp32 blocks
    assert bench.bsr_spmv_bytes(16384, 16384, 64, 6554) == 4 * 6554 * 4096 + 4 * (6554 + 256 + 1) + 8 * 16384


def test_traffic_counts_only_for_unchanged_kernels(tmp_path, monkeypatch):
    wl = "spmv_powerlaw"
    for f in bench.KERNEL_SOURCES["spmv"]:
        os.makedirs(tmp_path / os.path.dirname(f), exist_ok=True)
        shutil.copy(os.path.join(ROOT, f), tmp_path / f)
    monkeypatch.setattr(bench, "HERE", str(tmp_path))
    assert bench.load_traffic(wl, 1) is None  # no summary
    os.makedirs(tmp_path / "profiles")
    with open(tmp_path / "profiles" / ("traffic_%s.json" % wl), "w") as fh:
        json.dump(dict(kernel_fingerprint=bench.kernel_fingerprint(wl), bytes_per_launch=123), fh)
    assert bench.load_traffic(wl, 1) == 123
    # any change to a source of that workload's kernels retires the summary
    with open(tmp_path / bench.KERNEL_SOURCES["spmv"][0], "a") as fh:
        fh.write("\n")
    assert bench.load_traffic(wl, 1) is None
    # the other families do not depend on it
    assert bench.kernel_family("bsr_blocks") == "bsr" and bench.kernel_family("spmm_lognormal_N32") == "spmm"
    assert bench.kernel_family("spmm_clustered_N32") == "wcsr" and bench.kernel_family("bsr_spmv") == "bsr_spmv"


def test_storage_accounts_of_the_pages():
    """The format page's section 1 example (10^6 rows, 10^7 fp64 entries, int32
    indices): COO 16 bytes per entry = 160 MB; CSR 12 bytes per entry plus 4 MB
    of row pointers = 124 MB (the page counts 10^6 pointers, the end pointer
    adds 4 bytes); fp16 values bring CSR to 6 bytes per entry.  Its section 5:
    one 4-byte index per 16 x 16 block is 0.0156 bytes per value.  The LSMR
    page's section 4: values and indices of the CSR + CSC pair at nnz =
    19,747,202 are about 301 MiB."""
    assert bench.coo_storage_bytes(10 ** 7) == 160 * 10 ** 6
    assert bench.csr_storage_bytes(10 ** 6, 10 ** 7) == 124 * 10 ** 6 + 4
    assert bench.csr_storage_bytes(10 ** 6, 10 ** 7, val_bytes=2) - 4 * (10 ** 6 + 1) == 6 * 10 ** 7
    assert round(bench.block_index_bytes_per_value(16), 4) == 0.0156
    assert bench.block_index_bytes_per_value(16) == 4 / 256
    mib = bench.dual_value_index_bytes(19747202) / 2 ** 20
    assert abs(mib - 301.3) < 0.05
    assert bench.dual_storage_bytes(10, 20, 7) == 2 * 8 * 7 + 4 * 11 + 4 * 21


def test_gather_aware_spmm_bound():
    # every entry reads at least a 128-byte line of B, or its 4N-byte row segment
    assert bench.spmm_gather_bytes(3, 5, 8) == 8 * 5 + 4 * 4 + 5 * 128 + 4 * 3 * 8
    assert bench.spmm_gather_bytes(3, 5, 64) == 8 * 5 + 4 * 4 + 5 * 256 + 4 * 3 * 64


def test_workload_names_and_cpu_row_ranges():
    import numpy as np
    assert bench.parse_workload("spmm_lognormal_N128") == ("spmm_lognormal", 128)
    assert bench.parse_workload("spmm_clustered_N32") == ("spmm_clustered", 32)
    assert bench.parse_workload("spmm_skewed_N32") == ("spmm_skewed", 32)
    assert bench.kernel_family("spmm_skewed_N32") == bench.kernel_family("spmm_clustered_N32") == "wcsr"
    assert bench.parse_workload("stencil27") == ("stencil27", None)
    assert bench.ALL_WORKLOADS[0] == bench.HEADLINE
    rp = np.array([0, 3, 3, 10, 12, 20], np.int64)
    # ranges of about equal entry counts, covering [0, hi) once, none empty
    for hi in range(1, 6):
        for parts in (1, 2, 3, 8):
            r = bench._ranges(rp, hi, parts)
            assert r[0][0] == 0 and r[-1][1] == hi
            assert all(a < b for a, b in r) and all(r[i][1] == r[i + 1][0] for i in range(len(r) - 1))
    # the row sample stops before the flop budget is exceeded (all rows when they fit)
    assert bench._sample_rows(rp, 2, 25) == 4 and rp[4] * 2 <= 25
    assert bench._sample_rows(rp, 2, 40) == 5
    assert 1 <= bench.cpu_threads() <= 16


def test_counter_traffic_accounting():
    # ROCm's FETCH_SIZE expression, written out: it counts a 128-byte request
    # as 64 bytes unless TCC_BUBBLE counts it
    def fetch_size(c):
        return (128 * c["TCC_BUBBLE_sum"] + 64 * (c["TCC_EA0_RDREQ_sum"] - c["TCC_BUBBLE_sum"]
                - c["TCC_EA0_RDREQ_32B_sum"]) + 32 * c["TCC_EA0_RDREQ_32B_sum"])
    stream = dict(TCC_EA0_RDREQ_sum=1000.0, TCC_EA0_RDREQ_32B_sum=0.0, TCC_EA0_RDREQ_64B_sum=0.0,
                  TCC_EA0_RDREQ_128B_sum=1000.0, TCC_EA0_WRREQ_sum=1000.0, TCC_EA0_WRREQ_64B_sum=1000.0,
                  TCC_BUBBLE_sum=0.0)
    rd, wr, other = bench._request_bytes(stream)
    assert (rd, wr, other) == (128000.0, 64000.0, 0.0)
    assert fetch_size(stream) * 2 == rd  # the factor a streaming copy shows
    mixed = dict(stream, TCC_EA0_RDREQ_sum=10.0, TCC_EA0_RDREQ_32B_sum=3.0, TCC_EA0_RDREQ_64B_sum=2.0,
                 TCC_EA0_RDREQ_128B_sum=4.0, TCC_EA0_WRREQ_sum=5.0, TCC_EA0_WRREQ_64B_sum=2.0)
    rd, wr, other = bench._request_bytes(mixed)
    # one request of no listed size is taken as 64 bytes, as FETCH_SIZE does
    assert other == 1.0 and rd == 3 * 32 + 3 * 64 + 4 * 128 and wr == 3 * 32 + 2 * 64


def test_kernel_short_names():
    assert bench._short_kernel("void spx::(anonymous namespace)::bsr_spmm_dma<256>(int const*, float)") == \
        "bsr_spmm_dma<256>"
    assert bench._short_kernel("spx::(anonymous namespace)::xw_rows_kernel(spx::(anonymous namespace)::A)") == \
        "xw_rows_kernel"
    assert bench._short_kernel("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_counter_run_call_selection():
    # setup kernels first (one of them as often as the call's kernels), then
    # 3 calls of two kernels, the last call of one kernel shared by two calls
    # per step; only the last calls' dispatches are taken
    k = lambda n: "void spx::(anonymous namespace)::%s(int)" % n
    setup = [(i, k("sort"), {"x": 1.0}) for i in range(3)] + [(3, "torch_fill", {"x": 9.0})]
    calls = []
    for c in range(3):
        calls += [(10 + 2 * c, k("products"), {"x": 2.0}), (11 + 2 * c, k("rows"), {"x": 3.0})]
    names, tail = bench._call_dispatches(setup + calls, 3)
    assert names == [k("products"), k("rows")] and len(tail) == 6 and tail[0][0] == 10
    one = [(i, k("sell"), {"x": 1.0}) for i in range(4)]
    names, tail = bench._call_dispatches(setup + one, 4)
    assert names == [k("sell")] and len(tail) == 4
    import pytest
    with pytest.raises(RuntimeError):
        bench._call_dispatches(setup + calls, 4)  # a setup kernel inside the span


def test_probe_library_loads_and_refuses_bad_arguments():
    # the measurement probes bench.py loads (not part of the product ABI);
    # argument checks return before any launch
    import ctypes
    import os

    from spmm_csr_spmv_amd import build as b
    if not os.path.exists(b.PROBE_LIB):
        import pytest
        pytest.skip("probe library not built")
    L = ctypes.CDLL(b.PROBE_LIB)
    for name in ("spx_probe_out_bytes", "spx_probe_entries", "spx_probe_gather", "spx_feed_probe_waves",
                 "spx_probe_feed"):
        assert hasattr(L, name), name
    L.spx_probe_entries.restype = ctypes.c_int64
    L.spx_probe_entries.argtypes = [ctypes.c_int64]
    assert L.spx_probe_entries(5000) == 4096 and L.spx_probe_entries(-3) == 0
    L.spx_feed_probe_waves.restype = ctypes.c_int64
    assert L.spx_feed_probe_waves() == 2048
    L.spx_probe_feed.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p,
                                 ctypes.c_void_p]
    fake = ctypes.c_void_p(256)
    assert L.spx_probe_feed(fake, 3, 10, 0, fake, None) == 1      # not a power of two
    assert L.spx_probe_feed(None, 1024, 10, 0, fake, None) == 1   # null source
    assert L.spx_probe_feed(fake, 1024, 0, 0, fake, None) == 1    # no pieces per wave
