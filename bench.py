#!/usr/bin/env python3
"""Throughput of the sparse x dense products on one MI355X.

Headline workload: CSR SpMV y = A x on the power-law matrix (2^22 x 2^22,
lognormal row lengths plus planted hub rows, ~46.8M entries, fp32).  One step
is one `spmv` call over the whole matrix with the plan's default path.  The
one-time work (COO -> CSR build, plan) is timed separately under "setup".

Prints ONE JSON line: the headline's metric, value, timing, roofline and CPU
baseline at the top level, and under "configs" the same record for every other
workload, each timed in this run the same way:
  spmv_uniform (4096^2, rows of 1..16 entries), stencil27 (u <- A v - a u,
  v <- A^T u - b v per step through the CSR and the CSC), spmm_lognormal_N8 /
  _N32 / _N128, bsr_blocks (bf16 64 x 64 blocks on MFMA), and the extra paths
  bsr_spmv (fp32 64 x 64 blocks), spmm_clustered_N32 (windowed rows) and
  spmm_skewed_N32 (windowed rows of very different widths, task split).
--config NAME runs only that workload (as the headline), for profiling.

CPU baseline ("cpu_baseline" of each record): the oracle (plain C, fp64
accumulation) on the host's cores, threads over row ranges of equal entry
counts, and on one core; on a bounded row sample when a full pass is long.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
METRIC = "SpMV/SpMM GFLOP/s + achieved HBM GB/s vs MI355X peak (fp32), 1 GPU"
HEADLINE = "spmv_powerlaw"
# compressed columns per task of the skewed-window SpMM (a window of more is
# split); tasks run widest first
SKEWED_TASK_COLS = 2048
# every workload of a default run, in order (the headline first)
ALL_WORKLOADS = ["spmv_powerlaw", "spmv_uniform", "stencil27", "spmm_lognormal_N8", "spmm_lognormal_N32",
                 "spmm_lognormal_N128", "bsr_blocks", "bsr_spmv", "spmm_clustered_N32", "spmm_skewed_N32"]
# Sources whose code decides the kernels each workload runs and the layouts
# they stream (a committed traffic summary is used only while these are
# unchanged).
_CSRC = "spmm_csr_spmv_amd/csrc/"
KERNEL_SOURCES = {
    "spmv": [_CSRC + f for f in ("spmv.hip", "pstream.hip", "xwin.hip", "seg_rows.h", "device_common.h", "internal.h",
                                 "layout.h", "api.cpp", "plan_host.cpp")],
    "spmm": [_CSRC + f for f in ("spmm.hip", "device_common.h", "internal.h", "layout.h", "api.cpp", "plan_host.cpp")],
    "bsr": [_CSRC + f for f in ("bsr.hip", "device_common.h", "internal.h", "layout.h")],
    "bsr_spmv": [_CSRC + f for f in ("bsr_convert.hip", "device_common.h", "internal.h", "layout.h")],
    "wcsr": [_CSRC + f for f in ("wcsr.hip", "device_common.h", "internal.h", "layout.h", "plan_host.cpp")],
}


# --------------------------------------------------------------------------
# byte / flop model (algorithmic: every array the method must touch, once)
# --------------------------------------------------------------------------
def spmv_bytes(m, k, nnz, beta_nonzero=False):
    """CSR SpMV: values + column indices (8 B per entry), row_ptr, x read once,
    y written (and read when beta != 0).  The 8 B per entry is the lower bound
    of the LSMR page's section 1."""
    return 8 * nnz + 4 * (m + 1) + 4 * k + 4 * m + (4 * m if beta_nonzero else 0)


def spmv_flops(m, nnz, beta_nonzero=False):
    return 2 * nnz + (2 * m if beta_nonzero else 0)


def spmm_bytes(m, k, nnz, N, beta_nonzero=False):
    return 8 * nnz + 4 * (m + 1) + 4 * k * N + 4 * m * N + (4 * m * N if beta_nonzero else 0)


def spmm_gather_bytes(m, nnz, N, line=128):
    """What a row-by-row SpMM without B reuse must read: per entry its B row
    segment, at least one 128-byte cache line, plus the matrix and C once."""
    return 8 * nnz + 4 * (m + 1) + nnz * max(4 * N, line) + 4 * m * N


def bsr_bytes(mb, kb, bs, nnzb, N, beta_nonzero=False):
    return 2 * nnzb * bs * bs + 4 * (nnzb + mb + 1) + 2 * kb * bs * N + 4 * mb * bs * N * (2 if beta_nonzero else 1)


def bsr_flops(nnzb, bs, N):
    return 2 * nnzb * bs * bs * N


def bsr_spmv_bytes(m, n, bs, nnzb, beta_nonzero=False):
    """BSR SpMV with fp32 blocks: every stored block (4 bs^2 B), block column
    indices and block row pointer, x and y once."""
    mb = (m + bs - 1) // bs
    return 4 * nnzb * bs * bs + 4 * (nnzb + mb + 1) + 4 * n + 4 * m + (4 * m if beta_nonzero else 0)


# Storage accounts of the format page (section 1: COO and CSR of a 10^6-row
# matrix with 10^7 fp64 entries; section 5: block index cost per value) and of
# the LSMR page (section 4: the CSR + CSC pair).
def csr_storage_bytes(m, nnz, val_bytes=8, idx_bytes=4):
    """Values and column indices per entry plus one row pointer per row (the
    format page counts m pointers; the extra end pointer is kept here)."""
    return nnz * (val_bytes + idx_bytes) + (m + 1) * idx_bytes


def coo_storage_bytes(nnz, val_bytes=8, idx_bytes=4):
    return nnz * (val_bytes + 2 * idx_bytes)


def dual_value_index_bytes(nnz, val_bytes=4, idx_bytes=4):
    """Values and indices of both the CSR and the CSC (pointers not counted)."""
    return 2 * nnz * (val_bytes + idx_bytes)


def dual_storage_bytes(m, n, nnz):
    """CSR + CSC of an fp32/int32 matrix, pointers included."""
    return dual_value_index_bytes(nnz) + 4 * (m + 1) + 4 * (n + 1)


def block_index_bytes_per_value(bs, idx_bytes=4):
    return idx_bytes / float(bs * bs)


def kernel_family(workload):
    if workload == "bsr_spmv":
        return "bsr_spmv"
    if workload.startswith("spmm_clustered") or workload.startswith("spmm_skewed"):
        return "wcsr"
    return "bsr" if workload.startswith("bsr") else ("spmm" if workload.startswith("spmm") else "spmv")


def kernel_fingerprint(workload):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel_family(workload)]:
        with open(os.path.join(HERE, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic_record(workload):
    """The committed rocprofv3 counter summary of a workload, if it was taken on
    the current kernels (same fingerprint); else None."""
    path = os.path.join(HERE, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_fingerprint") != kernel_fingerprint(workload):
        return None
    return t


def load_traffic(workload, launches_bytes=None):
    """HBM bytes per launch from the committed counter summary, or None."""
    t = load_traffic_record(workload)
    return None if t is None else t.get("bytes_per_launch")


def parse_workload(name):
    """'spmm_lognormal_N32' -> ('spmm_lognormal', 32); others -> (name, None)."""
    for base in ("spmm_lognormal", "spmm_clustered", "spmm_skewed"):
        if name.startswith(base + "_N"):
            return base, int(name[len(base) + 2:])
    return name, None


# --------------------------------------------------------------------------
# host facts for the CPU baseline
# --------------------------------------------------------------------------
def cpu_threads():
    """Threads the oracle baseline uses: the cores this process may run on,
    at most 16 (the host's CPU share per GPU on an MI355X node)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------
# CPU baseline: the oracle over row ranges
# --------------------------------------------------------------------------
class CpuLeg:
    """One pass of the oracle over a workload: phases run in order, each over
    the rows [0, rows_hi) of its own row pointer (a sample when rows_hi < m),
    split among threads into ranges of equal entry counts.  flops and bytes are
    those of the sampled rows on the GPU side's models."""

    def __init__(self, phases, flops, nbytes, desc, max_threads=None):
        self.phases = phases  # [(row_ptr, rows_hi, fn(lo, hi))]
        self.flops = flops
        self.nbytes = nbytes
        self.desc = desc
        self.max_threads = max_threads  # 1: the oracle call cannot be split by rows


def _ranges(row_ptr, rows_hi, parts):
    import numpy as np
    hi_nz = int(row_ptr[rows_hi])
    cuts = np.searchsorted(row_ptr[:rows_hi + 1], np.linspace(0, hi_nz, parts + 1)[1:-1])
    b = [0] + [int(c) for c in cuts] + [rows_hi]
    return [(b[i], b[i + 1]) for i in range(parts) if b[i + 1] > b[i]]


def time_cpu_leg(leg, threads, seconds):
    import numpy as np  # noqa: F401
    plans = [(fn, _ranges(rp, hi, threads)) for rp, hi, fn in leg.phases]
    reps, t = 0, 0.0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        t0 = time.perf_counter()
        while True:
            for fn, rr in plans:
                list(ex.map(lambda r, fn=fn: fn(r[0], r[1]), rr))
            reps += 1
            t = time.perf_counter() - t0
            if t >= seconds or reps >= 1000:
                break
    return t / reps, reps, t


def cpu_baseline(leg, seconds):
    threads = cpu_threads() if leg.max_threads is None else min(cpu_threads(), leg.max_threads)
    per_1, reps_1, t_1 = time_cpu_leg(leg, 1, seconds / 2)
    if threads > 1:
        per_all, reps_all, t_all = time_cpu_leg(leg, threads, seconds / 2)
    else:
        per_all, reps_all, t_all = per_1, reps_1, t_1
    gf = lambda per: leg.flops / per / 1e9  # noqa: E731
    gb = lambda per: leg.nbytes / per / 1e9  # noqa: E731
    return dict(value=round(gf(per_all), 4), unit="GFLOP/s", cores=threads, kind="oracle",
                gbs=round(gb(per_all), 3), value_1core=round(gf(per_1), 4), gbs_1core=round(gb(per_1), 3),
                cores_all=threads, value_all=round(gf(per_all), 4), cpu_model=cpu_model(), nproc=os.cpu_count(),
                sample="%s; %d passes on %d threads in %.1f s, %d passes on 1 thread in %.1f s"
                       % (leg.desc, reps_all, threads, t_all, reps_1, t_1))


def _sample_rows(row_ptr, per_entry_flops, budget_flops):
    """Rows [0, hi) whose entries cost at most budget_flops (all rows if they fit)."""
    import numpy as np
    m = row_ptr.size - 1
    if int(row_ptr[m]) * per_entry_flops <= budget_flops:
        return m
    return max(1, int(np.searchsorted(row_ptr, budget_flops / per_entry_flops)) - 1)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
class Workload:
    """What one workload's measurement needs (fields filled by prepare())."""

    def __init__(self, name):
        self.name = name
        self.setup = {}
        self.restore = None
        self.restore_every = 0
        self.iterates_finite = None
        self.out_tensor = None
        self.graph = 0        # steps per captured graph replay in the timed region
        self.cpu = None       # CpuLeg or None
        self.extra = {}       # roofline extras (e.g. a gather-aware bound)
        self.keep = []        # device tensors to free afterwards
        self.digest = None    # fingerprint of the generated inputs


def _digest(*arrays):
    """SHA-256 (first 16 hex digits) of the generator's arrays, in order: a
    fingerprint of the inputs a run used."""
    import numpy as np
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).view(np.uint8).reshape(-1))
    return h.hexdigest()[:16]


def _to_dev(torch, a):
    return torch.from_numpy(a).cuda()


def _csr_from_coo(w, sp, torch, coo):
    d_row, d_col, d_val = (_to_dev(torch, a) for a in (coo.row, coo.col, coo.val))
    torch.cuda.synchronize()
    t1 = time.time()
    rp, ci, vv = sp.csr_build_from_coo(coo.m, coo.n, d_row, d_col, d_val)
    torch.cuda.synchronize()
    w.setup["csr_build_from_coo_ms"] = (time.time() - t1) * 1e3
    return rp, ci, vv


def prepare(name, args, opts):
    import numpy as np
    import torch

    import gen
    import spmm_csr_spmv_amd as sp

    base, N = parse_workload(name)
    w = Workload(name)
    t0 = time.time()
    if base == "bsr_blocks":
        b = gen.block_sparse_bsr(seed=0)
        N = 512
        Bh = gen.bf16_matrix(b.kb * b.bs, N, seed=0)
        d_brow, d_bcol = _to_dev(torch, b.brow_ptr), _to_dev(torch, b.bcol)
        d_bval = _to_dev(torch, b.bval.view(np.int16))
        d_B = _to_dev(torch, Bh.view(np.int16))
        C = torch.empty(b.mb * b.bs, N, device="cuda")
        w.setup["generate_s"] = time.time() - t0
        w.digest = _digest(b.brow_ptr, b.bcol, b.bval, Bh)

        def step():
            sp.bsr_spmm(b.mb, b.kb, b.bs, d_brow, d_bcol, d_bval, d_B, 1.0, 0.0, C)

        w.step, w.out_tensor, w.graph = step, C, 20
        w.flops = bsr_flops(b.nnzb, b.bs, N)
        w.nbytes = bsr_bytes(b.mb, b.kb, b.bs, b.nnzb, N)
        w.launches = 1
        w.dtype = "bf16 in / f32 acc"
        w.config = dict(workload=name, M=b.mb * b.bs, K=b.kb * b.bs, block=b.bs, nnz_blocks=b.nnzb, N=N)
        w.bound, w.peak, w.unit = "mfma", PEAK_BF16_TFLOPS, "TFLOP/s"
        if not args.no_cpu_baseline:
            import oracle
            rp, col, v64 = oracle.bsr_to_csr(b.mb, b.bs, b.brow_ptr, b.bcol, b.bval)
            hi = _sample_rows(rp, 2 * N, args.cpu_sample_gflop * 1e9)
            w.cpu = CpuLeg([(rp, hi, lambda lo, h: oracle.spmm_bf16(rp, col, v64, Bh, rows=np.arange(lo, h)))],
                           2 * int(rp[hi]) * N, bsr_bytes(b.mb, b.kb, b.bs, b.nnzb, N) * int(rp[hi]) / max(1, int(rp[-1])),
                           "rows [0, %d) of %d of C = A B over the expanded bf16 blocks (fp64 accumulation)"
                           % (hi, rp.size - 1))
        return w
    if base == "bsr_spmv":
        bs = 64
        coo = gen.block_sparse_coo(seed=0)
        w.setup["generate_s"] = time.time() - t0
        w.digest = _digest(coo.row, coo.col, coo.val)
        m, n = coo.m, coo.n
        rp, ci, vv = _csr_from_coo(w, sp, torch, coo)
        t1 = time.time()
        brp, bcol, bval, fill = sp.csr_to_bsr(m, n, rp, ci, vv, bs, min_fill=0.5)
        torch.cuda.synchronize()
        w.setup["csr_to_bsr_ms"] = (time.time() - t1) * 1e3
        nnzb = bcol.numel()
        x = _to_dev(torch, gen.dense_vector(n, 0, 1))
        y = torch.zeros(m, device="cuda")

        def step():
            sp.bsr_spmv(m, n, bs, brp, bcol, bval, 1.0, x, 0.0, y)

        w.step, w.out_tensor, w.graph = step, y, 20
        w.flops = 2 * nnzb * bs * bs
        w.nbytes = bsr_spmv_bytes(m, n, bs, nnzb)
        # the BCSR page's two thread mappings (section 2.1 whole blocks, 2.2
        # whole columns), at 64 x 64 and at 4 x 4 blocks of the same matrix
        # (section 3 compares them): mean kernel time of 20 graph-free launches
        cmp = {}
        b4 = sp.csr_to_bsr(m, n, rp, ci, vv, 4)
        for name_b, (bsx, arr) in () if args.counter_run else (("64x64", (64, (brp, bcol, bval))), ("4x4", (4, b4[:3]))):
            for strat, rw in (("whole_blocks", False), ("rows", True)):
                for _ in range(3):
                    sp.bsr_spmv(m, n, bsx, *arr, 1.0, x, 0.0, y, rowwise=rw)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(20):
                    sp.bsr_spmv(m, n, bsx, *arr, 1.0, x, 0.0, y, rowwise=rw)
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / 20
                nb = arr[1].numel()
                cmp["%s_%s" % (name_b, strat)] = dict(
                    ms=round(ms, 5), gflops=round(2 * nb * bsx * bsx / (ms * 1e-3) / 1e9, 1),
                    gbs=round(bsr_spmv_bytes(m, n, bsx, nb) / (ms * 1e-3) / 1e9, 1))
        del b4
        w.launches = 1
        w.dtype = "f32"
        w.config = dict(workload=name, M=m, K=n, block=bs, nnz=coo.nnz, nnz_blocks=nnzb, fill_ratio=fill,
                        strategies=cmp)
        w.bound, w.peak, w.unit = "hbm", PEAK_HBM_GBS, "GB/s"
        if not args.no_cpu_baseline:
            import oracle
            h_brp, h_bcol, h_bval, h_x = (t.cpu().numpy() for t in (brp, bcol, bval, x))
            w.cpu = CpuLeg([(np.array([0, m], np.int64), 1,
                             lambda lo, h: oracle.bsr_spmv(m, n, bs, h_brp, h_bcol, h_bval, h_x))],
                           w.flops, w.nbytes, "full passes of y = A x over the 64 x 64-block BSR (fp64 accumulation, "
                                              "one call per pass)", max_threads=1)
        del rp, ci, vv
        return w
    if base == "spmm_clustered":
        coo = gen.clustered_coo(seed=0)
        w.setup["generate_s"] = time.time() - t0
        w.digest = _digest(coo.row, coo.col, coo.val)
        m, n, nnz = coo.m, coo.n, coo.nnz
        rp, ci, vv = _csr_from_coo(w, sp, torch, coo)
        t1 = time.time()
        wp, wc, wv, fill = sp.csr_to_wcsr(m, n, rp, ci, vv, pad=8)
        torch.cuda.synchronize()
        w.setup["csr_to_wcsr_ms"] = (time.time() - t1) * 1e3
        total_cols = wc.numel()
        B = _to_dev(torch, gen.dense_matrix(n, N, 0))
        C = torch.empty(m, N, device="cuda")

        def step():
            sp.wcsr_spmm(m, n, wp, wc, wv, 1.0, B, 0.0, C)

        w.step, w.out_tensor, w.graph = step, C, 20
        w.flops = 2 * nnz * N
        w.nbytes = spmm_bytes(m, n, nnz, N)
        w.launches = 1
        w.dtype = "f32"
        w.config = dict(workload=name, M=m, K=n, nnz=nnz, N=N, window=64, compressed_columns=total_cols,
                        window_fill=round(fill, 4), mfma_flops=2 * total_cols * 64 * N,
                        wcsr_bytes=4 * total_cols * 64 + 4 * total_cols + 4 * total_cols * N + 4 * m * N)
        w.bound, w.peak, w.unit = "hbm", PEAK_HBM_GBS, "GB/s"
        # the CSR SpMM on the same matrix, for comparison
        if not args.counter_run:
            plan_c = sp.Plan(m, n, rp, ci, vv, max_N=N)
            for _ in range(3):
                sp.spmm(plan_c, 1.0, B, 0.0, C)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                sp.spmm(plan_c, 1.0, B, 0.0, C)
            e1.record()
            torch.cuda.synchronize()
            w.config["csr_spmm_ms_same_matrix"] = round(e0.elapsed_time(e1) / 10, 5)
            del plan_c
        if not args.no_cpu_baseline:
            import oracle
            h_rp, h_ci, h_vv = (t.cpu().numpy() for t in (rp, ci, vv))
            Bh = B.cpu().numpy()
            hi = _sample_rows(h_rp, 2 * N, args.cpu_sample_gflop * 1e9)
            w.cpu = CpuLeg([(h_rp, hi, lambda lo, h: oracle.spmm(h_rp, h_ci, h_vv, Bh, rows=np.arange(lo, h)))],
                           2 * int(h_rp[hi]) * N, spmm_bytes(m, n, nnz, N) * int(h_rp[hi]) / max(1, nnz),
                           "rows [0, %d) of %d of C = A B over the CSR (fp64 accumulation)" % (hi, m))
        w.keep = [rp, ci, vv, wp, wc, wv]
        return w

    if base == "spmm_skewed":
        coo = gen.skewed_windows_coo(seed=0)
        w.setup["generate_s"] = time.time() - t0
        w.digest = _digest(coo.row, coo.col, coo.val)
        m, n, nnz = coo.m, coo.n, coo.nnz
        rp, ci, vv = _csr_from_coo(w, sp, torch, coo)
        del coo
        t1 = time.time()
        wp, wc, wv, fill = sp.csr_to_wcsr(m, n, rp, ci, vv, pad=8)
        torch.cuda.synchronize()
        w.setup["csr_to_wcsr_ms"] = (time.time() - t1) * 1e3
        total_cols = wc.numel()
        T = SKEWED_TASK_COLS
        t1 = time.time()
        tasks = sp.wcsr_tasks(m, wp, total_cols, task_cols=T)
        w.setup["wcsr_tasks_ms"] = (time.time() - t1) * 1e3
        B = _to_dev(torch, gen.dense_matrix(n, N, 0))
        C = torch.empty(m, N, device="cuda")
        work = torch.empty(max(tasks.workspace_bytes(N), 1), dtype=torch.uint8, device="cuda")

        def step():
            sp.wcsr_spmm_tasks(m, n, tasks, wc, wv, 1.0, B, 0.0, C, work=work)

        w.step, w.out_tensor, w.graph = step, C, 20
        w.flops = 2 * nnz * N
        w.nbytes = spmm_bytes(m, n, nnz, N)
        w.launches = 1  # one library call: the task kernel and the partial sums
        w.dtype = "f32"
        widths = (wp[1:] - wp[:-1]).cpu().numpy()
        w.config = dict(workload=name, M=m, K=n, nnz=nnz, N=N, window=64, compressed_columns=total_cols,
                        window_fill=round(fill, 4), widest_window=int(widths.max()),
                        median_window=float(np.median(widths)), task_cols=T, tasks=tasks.ntasks,
                        partial_slots=tasks.nslots, partial_bytes=2 * tasks.workspace_bytes(N),
                        mfma_flops=2 * total_cols * 64 * N,
                        wcsr_bytes=4 * total_cols * 64 + 4 * total_cols + 4 * total_cols * N + 4 * m * N)
        w.bound, w.peak, w.unit = "hbm", PEAK_HBM_GBS, "GB/s"
        # the same product with one workgroup per window, and through the CSR
        if not args.counter_run:
            def ms_of(fn, reps=10):
                for _ in range(2):
                    fn()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    fn()
                e1.record()
                torch.cuda.synchronize()
                return round(e0.elapsed_time(e1) / reps, 5)

            w.config["one_workgroup_per_window_ms"] = ms_of(lambda: sp.wcsr_spmm(m, n, wp, wc, wv, 1.0, B, 0.0, C))
            # the same call with other task widths (tables built here, widest first)
            widths = {}
            for Tw in (512, 1024, 2048, 4096):
                tw = sp.wcsr_tasks(m, wp, total_cols, task_cols=Tw)
                ww = torch.empty(max(tw.workspace_bytes(N), 1), dtype=torch.uint8, device="cuda")
                widths[str(Tw)] = dict(ms=ms_of(lambda: sp.wcsr_spmm_tasks(m, n, tw, wc, wv, 1.0, B, 0.0, C, work=ww)),
                                       tasks=tw.ntasks, partial_slots=tw.nslots)
                del tw, ww
            w.config["task_widths"] = widths
            plan_c = sp.Plan(m, n, rp, ci, vv, max_N=N)
            w.config["csr_spmm_ms_same_matrix"] = ms_of(lambda: sp.spmm(plan_c, 1.0, B, 0.0, C))
            del plan_c
        if not args.no_cpu_baseline:
            import oracle
            h_rp, h_ci, h_vv = (t.cpu().numpy() for t in (rp, ci, vv))
            Bh = B.cpu().numpy()
            hi = _sample_rows(h_rp, 2 * N, args.cpu_sample_gflop * 1e9)
            w.cpu = CpuLeg([(h_rp, hi, lambda lo, h: oracle.spmm(h_rp, h_ci, h_vv, Bh, rows=np.arange(lo, h)))],
                           2 * int(h_rp[hi]) * N, spmm_bytes(m, n, nnz, N) * int(h_rp[hi]) / max(1, nnz),
                           "rows [0, %d) of %d of C = A B over the CSR (fp64 accumulation)" % (hi, m))
        w.keep = [rp, ci, vv, wp, wc, wv, tasks.table, work]
        return w

    # CSR workloads through a plan
    coo = {"spmv_uniform": lambda: gen.uniform_rows_coo(seed=0),
           "spmv_powerlaw": lambda: gen.powerlaw_coo(seed=0),
           "stencil27": lambda: gen.stencil27_coo(seed=0),
           "spmm_lognormal": lambda: gen.lognormal_coo(seed=0)}[base]()
    w.setup["generate_s"] = time.time() - t0
    w.digest = _digest(coo.row, coo.col, coo.val)
    m, n, nnz = coo.m, coo.n, coo.nnz
    rp, ci, vv = _csr_from_coo(w, sp, torch, coo)
    del coo
    csc = None
    if base == "stencil27":
        t1 = time.time()
        csc = sp.csr_to_csc(m, n, rp, ci, vv)
        torch.cuda.synchronize()
        w.setup["csr_to_csc_ms"] = (time.time() - t1) * 1e3
    N = N if base == "spmm_lognormal" else 1
    tune = None
    if args.autotune and base != "spmm_lognormal":
        x_t = _to_dev(torch, gen.dense_vector(n, 0, 1))
        t1 = time.time()
        best, ms, best_opts = sp.autotune_spmv(m, n, rp, ci, vv, x_t, reps=10)
        w.setup["autotune_ms"] = (time.time() - t1) * 1e3
        tune = dict(candidates=[dict(c) for c in sp.DEFAULT_CANDIDATES], ms_per_call=[round(t, 5) for t in ms],
                    best=best)
        del x_t
    t1 = time.time()
    if tune is not None:
        plan = sp.Plan(m, n, rp, ci, vv, csc=csc, max_N=N, tuned=True)
    else:
        plan = sp.Plan(m, n, rp, ci, vv, csc=csc, max_N=N, **opts)
    torch.cuda.synchronize()
    w.setup["plan_ms"] = (time.time() - t1) * 1e3
    prof = plan.profile()
    x = _to_dev(torch, gen.dense_vector(n, 0, 1))
    y = torch.zeros(m, device="cuda")
    w.config = dict(workload=name, M=m, K=n, nnz=nnz, row_len_mean=round(prof["mean"], 3), p95=prof["p95"],
                    p99=prof["p99"], max_row=prof["max_len"],
                    bins=dict(group_tasks=prof["group_tasks"], wave_rows=prof["wave_rows"],
                              block_rows=prof["block_rows"], split_rows=prof["split_rows"],
                              split_segments=prof["split_segments"]),
                    path="x-window stream" if prof["x_window_bits"] else
                    ("column-panel stream" if prof["col_panels"] else
                     ("SELL-C-sigma" if prof["sell_slots"] else "row bins")))
    if opts:
        w.config["plan_options"] = opts
    if tune is not None:
        w.config["autotune"] = tune
        w.config["col_panels"] = prof["col_panels"]
    if base == "spmv_powerlaw" and not args.counter_run and not opts and tune is None:
        # the entry-balanced one-kernel stream against the binned dispatcher and
        # the other paths on this matrix (mean of 20 graph-free calls each)
        w.config["strategies"] = compare_spmv_paths(sp, torch, m, n, rp, ci, vv, x_dev=_to_dev(torch, gen.dense_vector(n, 0, 1)))
    w.bound, w.peak, w.unit = "hbm", PEAK_HBM_GBS, "GB/s"
    w.dtype = "f32"
    want_cpu = not args.no_cpu_baseline
    if want_cpu:
        import oracle
        h_rp, h_ci, h_vv = (t.cpu().numpy() for t in (rp, ci, vv))
    if base == "stencil27":
        u = _to_dev(torch, gen.dense_vector(m, 0, 2))
        v = _to_dev(torch, gen.dense_vector(n, 0, 3))
        u0, v0 = u.clone(), v.clone()
        rng = np.random.default_rng(5)
        ab = rng.uniform(0.5, 2.0, size=(1 << 16, 2)).astype(np.float32)
        it = [0]

        def step():
            a, bt = ab[it[0] % ab.shape[0]]
            it[0] += 1
            sp.spmv(plan, 1.0, v, -float(a), u)
            sp.spmv_t(plan, 1.0, u, -float(bt), v)

        def restore():
            u.copy_(u0)
            v.copy_(v0)

        w.step, w.restore = step, restore
        w.graph = 0  # its alpha/beta change every step and the iterates are put back every 8 steps
        w.flops = 2 * spmv_flops(m, nnz, True)
        w.nbytes = 2 * spmv_bytes(m, n, nnz, True)  # per step (two launches)
        w.launches = 2
        w.config["step"] = "u <- A v - alpha u ; v <- A^T u - beta v"
        # the LSMR page's section 4 account: values and indices of the CSR + CSC pair
        w.config["dual_storage_bytes"] = dual_storage_bytes(m, n, nnz)
        # the iterates grow by about |A| per step and pass the fp32 range
        # after some 20 steps: put u, v back every 8 steps (inside the
        # wall-clock region, outside the per-step events)
        w.restore_every = 8
        w.config["restore_every"] = 8
        w.iterates_finite = lambda: bool(torch.isfinite(u).all().item() and torch.isfinite(v).all().item())
        if want_cpu:
            h_cp, h_ri, h_cv = (t.cpu().numpy() for t in csc)
            hu, hv = u0.cpu().numpy(), v0.cpu().numpy()
            w.cpu = CpuLeg([(h_rp, m, lambda lo, h: oracle.spmv(h_rp, h_ci, h_vv, hv, 1.0, -1.25, hu,
                                                                rows=np.arange(lo, h))),
                            (h_cp, n, lambda lo, h: oracle.spmv(h_cp, h_ri, h_cv, hu, 1.0, -0.75, hv,
                                                                rows=np.arange(lo, h)))],
                           w.flops, w.nbytes, "full operator pairs u <- A v - a u, v <- A^T u - b v over the CSR "
                                              "and the CSC (fp64 accumulation)")
    elif base == "spmm_lognormal":
        Bh = gen.dense_matrix(n, N, 0)
        B = _to_dev(torch, Bh)
        C = torch.empty(m, N, device="cuda")

        def step():
            sp.spmm(plan, 1.0, B, 0.0, C)

        w.step, w.out_tensor, w.graph = step, C, 20
        w.flops = 2 * nnz * N
        w.nbytes = spmm_bytes(m, n, nnz, N)
        w.launches = 1
        w.config["N"] = N
        # a row-by-row SpMM reads every entry's B row segment (at least a line)
        w.extra["gather_bound_bytes"] = spmm_gather_bytes(m, nnz, N)
        if want_cpu:
            hi = _sample_rows(h_rp, 2 * N, args.cpu_sample_gflop * 1e9)
            w.cpu = CpuLeg([(h_rp, hi, lambda lo, h: oracle.spmm(h_rp, h_ci, h_vv, Bh, rows=np.arange(lo, h)))],
                           2 * int(h_rp[hi]) * N, spmm_bytes(m, n, nnz, N) * int(h_rp[hi]) / max(1, nnz),
                           "rows [0, %d) of %d of C = A B (fp64 accumulation)" % (hi, m))
    else:
        def step():
            sp.spmv(plan, 1.0, x, 0.0, y)

        w.step, w.out_tensor = step, y
        w.flops = spmv_flops(m, nnz)
        w.nbytes = spmv_bytes(m, n, nnz)
        w.launches = 1
        w.graph = 20  # (the stencil pair below stays graph-free)
        if want_cpu:
            hx = x.cpu().numpy()
            # the 4096-row matrix is too small to split among threads
            w.cpu = CpuLeg([(h_rp, m, lambda lo, h: oracle.spmv(h_rp, h_ci, h_vv, hx, rows=np.arange(lo, h)))],
                           w.flops, w.nbytes, "full passes of y = A x over the same %s matrix (fp64 accumulation)"
                           % base, max_threads=1 if base == "spmv_uniform" else None)
        if base == "spmv_powerlaw" and args.gather_probe:
            w.probe = (ci, nnz, n)
    w.keep = [plan, rp, ci, vv, csc]
    return w


# --------------------------------------------------------------------------
# Traffic between the L2s and memory, from rocprofv3 counters
# --------------------------------------------------------------------------
# Every read that misses an XCD's L2 goes to the memory side (the MALL, then
# HBM) as one request of 32, 64 or 128 bytes, counted by size; writes leave as
# 32- or 64-byte requests.  So the bytes are the request counts times their
# sizes, with no scale factor.  (FETCH_SIZE is not used: its expression takes
# every request that is neither a 32-byte one nor a TCC_BUBBLE as 64 bytes,
# and on this chip the 128-byte requests are counted apart, so it reads half
# of a streaming kernel's bytes.)  A 256 MiB device copy is profiled the same
# way as a check of the method.  The MALL sits on the memory side of these
# counters, so the bytes are what the XCDs move, wherever in memory it is
# served from.
COUNTER_PASSES = (
    ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum"),
    ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_EA0_RDREQ_DRAM_sum", "TCC_EA0_WRREQ_DRAM_sum"),
    ("TCC_HIT_sum", "TCC_MISS_sum", "TCC_BUBBLE_sum"),
)
COUNTER_STEPS, COUNTER_WARMUP = 5, 1


def _child_args(name):
    """bench.py arguments of one counter run; a workload name may carry plan
    options after a '+', separated by ':' (spmv_powerlaw+col_panels=8:wave_min=64)."""
    if name == "copy":
        return ["--copy-calibration"]
    name, _, opts = name.partition("+")
    base, N = parse_workload(name)
    a = ["--config", base] + (["--N", str(N)] if N is not None else [])
    a += ["--options", opts.replace(":", ",")] if opts else []
    return a + ["--counter-run", "--steps", str(COUNTER_STEPS), "--warmup", str(COUNTER_WARMUP)]


def _rocprof(prof_args, name, outdir):
    """One rocprofv3 run over a child bench.py (started from /tmp, the program
    itself right after '--'); returns the child's last stdout line."""
    import subprocess
    cmd = ["timeout", "-s", "KILL", "240", "rocprofv3"] + prof_args + [
        "--output-format", "csv", "-d", outdir, "-o", "run", "--", sys.executable, os.path.join(HERE, "bench.py")
    ] + _child_args(name)
    env = dict(os.environ, TMPDIR="/tmp")
    r = subprocess.run(cmd, cwd="/tmp", env=env, capture_output=True, text=True)
    # rocprofv3 may end with SIGSEGV after the program finished and wrote its results
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    if r.returncode not in (0, 139, -11) or not lines:
        raise RuntimeError("%s failed (%d): %s" % (" ".join(cmd), r.returncode, (r.stderr or "")[-2000:]))
    shown = ["rocprofv3"] + prof_args + ["--output-format", "csv", "-d", "<out>", "-o", "run", "--", "python3",
                                          "<repo>/bench.py"] + _child_args(name)
    return json.loads(lines[-1]), " ".join(shown)


def _csv_rows(outdir, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(outdir, "**", "*" + suffix), recursive=True))
    if not files:
        raise RuntimeError("no %s under %s" % (suffix, outdir))
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _short_kernel(name):
    """'void spx::(anonymous namespace)::bsr_spmm_dma<256>(int const*, ...)' -> 'bsr_spmm_dma<256>'"""
    head = name.replace("(anonymous namespace)::", "").split("(")[0].strip()
    if head.startswith("void "):
        head = head[5:]
    lt = head.find("<")
    base, targs = (head, "") if lt < 0 else (head[:lt], head[lt:])
    return base.split("::")[-1] + targs


def _dispatches(rows):
    """[(dispatch id, kernel name, {counter: value})] of one counter pass, in
    dispatch order."""
    out = {}
    for r in rows:
        d = int(r["Dispatch_Id"])
        out.setdefault(d, (r["Kernel_Name"], {}))[1][r["Counter_Name"]] = float(r["Counter_Value"])
    return [(d, k, v) for d, (k, v) in sorted(out.items())]


def _call_dispatches(disp, calls):
    """The dispatches of the last `calls` library calls of a counter run: the
    timed steps come last, each call dispatching each of its kernels once, so
    walking back from the end until a kernel repeats gives one call's kernels."""
    lib = [x for x in disp if "spx::" in x[1]]
    names = []
    for _, k, _ in reversed(lib):
        if k in names:
            break
        names.append(k)
    tail = lib[-calls * len(names):]
    if len(tail) != calls * len(names) or any(k not in names for _, k, _ in tail):
        raise RuntimeError("the last %d calls do not repeat the kernels %s" % (calls, names))
    return names[::-1], tail


def _request_bytes(c):
    """Read and write bytes of one dispatch's (or one launch's) counters."""
    n = c["TCC_EA0_RDREQ_sum"]
    n32, n64, n128 = c["TCC_EA0_RDREQ_32B_sum"], c["TCC_EA0_RDREQ_64B_sum"], c["TCC_EA0_RDREQ_128B_sum"]
    other = max(0.0, n - n32 - n64 - n128)
    read = 32 * n32 + 64 * (n64 + other) + 128 * n128
    w, w64 = c["TCC_EA0_WRREQ_sum"], c["TCC_EA0_WRREQ_64B_sum"]
    write = 32 * (w - w64) + 64 * w64
    return read, write, other


def collect_traffic(names_arg, out, summarize_only=False):
    """Runs the counter passes (and a kernel trace) of the copy check and of
    each workload, keeping the raw CSVs, the child's record and the commands
    under out/raw, then writes the summaries from them."""
    names = ALL_WORKLOADS if names_arg == "all" else names_arg.split(",")
    out = os.path.abspath(out)  # the profiler runs from /tmp
    raw = os.path.join(out, "raw")
    os.makedirs(raw, exist_ok=True)
    if not summarize_only:
        for name in ["copy"] + names:
            cmds = []
            for i, ctrs in enumerate(COUNTER_PASSES):
                rec, shown = _rocprof(["--pmc"] + list(ctrs), name, os.path.join(raw, "%s_p%d" % (name, i)))
                cmds.append(shown)
                log("counters", name, "pass", i, "done")
            if name != "copy":
                rec, shown = _rocprof(["--kernel-trace", "--stats"], name, os.path.join(raw, "%s_kt" % name))
                cmds.append(shown)
                log("kernel trace", name, "done")
            with open(os.path.join(raw, "%s_run.json" % name), "w") as f:
                json.dump(dict(record=rec, commands=cmds), f)
    summarize_traffic(names, out)


def _pass_counters(raw, name, calls):
    """Per-launch counter values over the last `calls` calls, and the call's
    kernels."""
    total, kernels, by_kernel = {}, None, {}
    for i in range(len(COUNTER_PASSES)):
        disp = _dispatches(_csv_rows(os.path.join(raw, "%s_p%d" % (name, i)), "counter_collection.csv"))
        if calls is None:  # the copy check: the run's last dispatch is its last copy
            names, tail = [disp[-1][1]], [disp[-1]]
            n = 1
        else:
            names, tail = _call_dispatches(disp, calls)
            n = calls
        if kernels is not None and names != kernels:
            raise RuntimeError("passes disagree on the call's kernels: %s / %s" % (kernels, names))
        kernels = names
        for _, kn, v in tail:
            for c, x in v.items():
                total[c] = total.get(c, 0.0) + x / n
                by_kernel.setdefault(kn, {})[c] = by_kernel.get(kn, {}).get(c, 0.0) + x / n
    return kernels, total, by_kernel


def summarize_traffic(names, out):
    raw = os.path.join(out, "raw")
    with open(os.path.join(raw, "copy_run.json")) as f:
        run = json.load(f)
    rec = run["record"]
    kernels, c, _ = _pass_counters(raw, "copy", None)
    rd, wr, _ = _request_bytes(c)
    check = dict(kernel=_short_kernel(kernels[0]), bytes_read=rec["copy_bytes_read"],
                 bytes_written=rec["copy_bytes_written"], counted_read=int(rd), counted_write=int(wr),
                 read_ratio=round(rd / rec["copy_bytes_read"], 4), write_ratio=round(wr / rec["copy_bytes_written"], 4),
                 requests_128B_share=round(c["TCC_EA0_RDREQ_128B_sum"] / c["TCC_EA0_RDREQ_sum"], 4),
                 commands=run["commands"])
    with open(os.path.join(out, "traffic_copy_check.json"), "w") as f:
        json.dump(check, f, indent=1)

    for name in names:
        with open(os.path.join(raw, "%s_run.json" % name)) as f:
            run = json.load(f)
        rec, cmds = run["record"], run["commands"]
        calls = (COUNTER_WARMUP + COUNTER_STEPS) * rec.get("launches_per_step", 1)
        call, per_launch, by_kernel = _pass_counters(raw, name, calls)
        rd, wr, other = _request_bytes(per_launch)
        split = {}
        for k in call:
            krd, kwr, _ = _request_bytes(by_kernel[k])
            kh, km = by_kernel[k]["TCC_HIT_sum"], by_kernel[k]["TCC_MISS_sum"]
            split[_short_kernel(k)] = dict(read_bytes=int(krd), write_bytes=int(kwr),
                                           l2_hit_rate=round(kh / max(1.0, kh + km), 4))
        fetch_equiv = (128 * per_launch["TCC_BUBBLE_sum"] + 64 * (per_launch["TCC_EA0_RDREQ_sum"] -
                       per_launch["TCC_BUBBLE_sum"] - per_launch["TCC_EA0_RDREQ_32B_sum"]) +
                       32 * per_launch["TCC_EA0_RDREQ_32B_sum"])
        hits, miss = per_launch["TCC_HIT_sum"], per_launch["TCC_MISS_sum"]
        roof = rec.get("roofline", {})
        t = dict(workload=name, kernels=[_short_kernel(k) for k in call], kernel_names=call,
                 kernel_fingerprint=kernel_fingerprint(name), launches=calls,
                 read_bytes_per_launch=int(rd), write_bytes_per_launch=int(wr), bytes_per_launch=int(rd + wr),
                 algorithmic_bytes_per_launch=roof.get("algorithmic_bytes_per_launch"),
                 requests_per_launch={k.replace("TCC_", "").replace("_sum", ""): round(v, 1)
                                      for k, v in sorted(per_launch.items())},
                 read_requests_unsized_per_launch=round(other, 1),
                 fetch_size_bytes_per_launch=int(fetch_equiv),
                 l2_hit_rate=round(hits / max(1.0, hits + miss), 4), per_kernel=split,
                 method="read = 32 x RDREQ_32B + 64 x RDREQ_64B + 128 x RDREQ_128B, write = 32 x (WRREQ - "
                        "WRREQ_64B) + 64 x WRREQ_64B (TCC_EA0 counters summed over the L2 channels), per launch "
                        "over the dispatches of the last %d calls; no scale factor (copy check: read x%.4f, "
                        "write x%.4f of a 256 MiB copy)" % (calls, check["read_ratio"], check["write_ratio"]),
                 commands=cmds,
                 note="run from /tmp with TMPDIR=/tmp; <repo> is the repository root; one launch = one library "
                      "call = one dispatch of each kernel listed")
        with open(os.path.join(out, "traffic_%s.json" % name), "w") as f:
            json.dump(t, f, indent=1)
        kt = _csv_rows(os.path.join(raw, "%s_kt" % name), "kernel_stats.csv")
        _kernel_summary(out, name, t, kt, rec, cmds[-1])
        log("traffic", name, "%.1f MB read + %.1f MB written per launch" % (rd / 1e6, wr / 1e6))


def _kernel_summary(out, name, t, kt, rec, kt_cmd):
    roof = rec.get("roofline", {})
    rows = sorted(kt, key=lambda r: -float(r["TotalDurationNs"]))
    main = re.sub(r"[^A-Za-z0-9_]", "", "_".join(k.split("<")[0] for k in t["kernels"][:2]))
    lines = ["# %s on %s" % (", ".join(t["kernels"]), name), "",
             "Written by `python3 <repo>/bench.py --collect-traffic %s --traffic-out <dir>` (`<repo>` is the "
             "repository root), which runs each rocprofv3 pass below as a child process from /tmp with "
             "TMPDIR=/tmp, and `traffic_%s.json` beside this file." % (name, name), "",
             "Kernel trace:", "",
             "```", kt_cmd, "```", "",
             "| kernel | calls | total us | average us | % |", "|---|---|---|---|---|"]
    for r in rows[:12]:
        lines.append("| %s | %s | %.1f | %.2f | %.1f |" % (
            _short_kernel(r["Name"])[:70], r["Calls"], float(r["TotalDurationNs"]) / 1e3, float(r["AverageNs"]) / 1e3,
            float(r["Percentage"])))
    lines += ["", "The same run's events (bench.py, plain launches, per launch): %.2f us; algorithmic bytes per "
              "launch %s." % (
        1e3 * roof.get("kernel_ms", float("nan")), roof.get("algorithmic_bytes_per_launch")), "",
        "Traffic between the L2s and memory per launch (counter passes below, averaged over the last %d "
        "launches):" % t["launches"], "",
        "| quantity | value |", "|---|---|",
        "| read bytes | %d |" % t["read_bytes_per_launch"],
        "| write bytes | %d |" % t["write_bytes_per_launch"],
        "| total / algorithmic | %.3f |" % (t["bytes_per_launch"] / max(1, t["algorithmic_bytes_per_launch"] or 1)),
        "| L2 hit rate | %.3f |" % t["l2_hit_rate"],
        "| FETCH_SIZE (as ROCm defines it), bytes | %d |" % t["fetch_size_bytes_per_launch"]]
    for k, v in t["requests_per_launch"].items():
        lines.append("| %s | %.0f |" % (k, v))
    if len(t["per_kernel"]) > 1:
        lines += ["", "| kernel | read bytes | write bytes | L2 hit rate |", "|---|---|---|---|"]
        for k, v in t["per_kernel"].items():
            lines.append("| %s | %d | %d | %.3f |" % (k, v["read_bytes"], v["write_bytes"], v["l2_hit_rate"]))
    lines += ["", "Counter passes:", "", "```"] + t["commands"][:-1] + ["```", "",
              "Method: " + t["method"] + ".", ""]
    with open(os.path.join(out, "%s_%s.md" % (main, name)), "w") as f:
        f.write("\n".join(lines))


# --------------------------------------------------------------------------
# GPU measurement
# --------------------------------------------------------------------------
def copy_rate_gbs():
    """A plain 256 MiB device copy, read + write bytes over its time."""
    import numpy as np
    import torch
    ref = torch.ones(64 << 20, device="cuda")
    dst = torch.empty_like(ref)
    dst.copy_(ref)
    t = []
    for _ in range(5):
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        dst.copy_(ref)
        a1.record()
        torch.cuda.synchronize()
        t.append(a0.elapsed_time(a1))
    del ref, dst
    return 2 * (64 << 20) * 4 / (float(np.median(t)) * 1e-3) / 1e9


def warm_library():
    """One tiny conversion, plan and product, so that the one-time loading of
    the library's code objects (and of its static device arrays) is not
    counted in the first workload's setup times."""
    import numpy as np
    import torch

    import spmm_csr_spmv_amd as sp
    row = torch.tensor([0, 1, 2, 2], dtype=torch.int32, device="cuda")
    col = torch.tensor([1, 0, 2, 0], dtype=torch.int32, device="cuda")
    val = torch.ones(4, device="cuda")
    rp, ci, vv = sp.csr_build_from_coo(3, 3, row, col, val)
    csc = sp.csr_to_csc(3, 3, rp, ci, vv)
    plan = sp.Plan(3, 3, rp, ci, vv, csc=csc)
    y = torch.empty(3, device="cuda")
    sp.spmv(plan, 1.0, torch.ones(3, device="cuda"), 0.0, y)
    torch.cuda.synchronize()
    assert np.allclose(y.cpu().numpy(), [1.0, 1.0, 2.0])
    del plan


def gather_probe(col, nnz, n):
    """Stream rate and gather rate over the matrix's own column array (see
    csrc/probe.hip): times of 3 runs each, medians."""
    import ctypes

    import numpy as np
    import torch
    from spmm_csr_spmv_amd import build as b
    if not os.path.exists(b.PROBE_LIB):
        raise ImportError("%s is not built" % b.PROBE_LIB)
    L = ctypes.CDLL(b.PROBE_LIB)
    L.spx_probe_out_bytes.restype = ctypes.c_int64
    L.spx_probe_entries.restype = ctypes.c_int64
    L.spx_probe_entries.argtypes = [ctypes.c_int64]
    L.spx_probe_gather.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                   ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    bits = max(1, (n - 1).bit_length())
    x = torch.ones(1 << bits, device="cuda")
    val = torch.ones(nnz, device="cuda")
    out = torch.empty(L.spx_probe_out_bytes() // 4, device="cuda")
    s = torch.cuda.current_stream()
    cases = {"stream_only": (0xFFFFFFFF, 0), "gather_x": ((1 << bits) - 1, 1),
             "gather_2MiB_slice": ((1 << 19) - 1, 1), "gather_16KiB": ((1 << 12) - 1, 1)}
    res = {}
    for key, (mask, mode) in cases.items():
        ts = []
        for _ in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            rc = L.spx_probe_gather(ctypes.c_void_p(col.data_ptr()), ctypes.c_void_p(val.data_ptr()), nnz,
                                    ctypes.c_void_p(x.data_ptr()), mask & 0xFFFFFFFF, mode,
                                    ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(s.cuda_stream))
            e1.record(s)
            if rc != 0:
                raise RuntimeError("spx_probe_gather failed: %d" % rc)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        res[key + "_ms"] = round(float(np.median(ts[1:])), 5)
    entries = int(L.spx_probe_entries(nnz))
    res["entries"] = entries
    res["stream_gbs"] = round(8 * entries / (res["stream_only_ms"] * 1e-3) / 1e9, 1)
    for key in ("gather_x", "gather_2MiB_slice", "gather_16KiB"):
        res[key + "_gps"] = round(entries / (res[key + "_ms"] * 1e-3) / 1e9, 1)  # G gathers / s
    del x, val, out
    return res


def feed_probe():
    """Rates at which the memory side fills LDS through global_load_lds (see
    csrc/probe.hip): a buffer resident in an XCD's L2, a 64 MiB buffer read
    many times per launch and once per launch (held by the MALL between
    launches), and a 1 GiB one (HBM).  Medians of 3 timed launches."""
    import ctypes

    import numpy as np
    import torch
    from spmm_csr_spmv_amd import build as b
    if not os.path.exists(b.PROBE_LIB):
        raise ImportError("%s is not built" % b.PROBE_LIB)
    L = ctypes.CDLL(b.PROBE_LIB)
    L.spx_feed_probe_waves.restype = ctypes.c_int64
    L.spx_probe_feed.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p,
                                 ctypes.c_void_p]
    waves = int(L.spx_feed_probe_waves())
    src = torch.ones(1 << 28, device="cuda")  # 1 GiB
    out = torch.empty(512 * 256, device="cuda")
    s = torch.cuda.current_stream()
    cases = {"l2_2MiB_tbs": (2048, 2048, 7919), "mall_64MiB_reread_tbs": (65536, 2048, 7919),
             "mall_64MiB_once_tbs": (65536, 65536 // waves, 0), "hbm_1GiB_tbs": (1 << 20, 2048, 7919)}
    res = {}
    for key, (pieces, iters, stride) in cases.items():
        ts = []
        for _ in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            rc = L.spx_probe_feed(ctypes.c_void_p(src.data_ptr()), pieces, iters, stride,
                                  ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(s.cuda_stream))
            e1.record(s)
            if rc != 0:
                raise RuntimeError("spx_probe_feed failed: %d" % rc)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        res[key] = round(waves * iters * 1024 / (float(np.median(ts[1:])) * 1e-3) / 1e12, 2)
    del src, out
    return res


def compare_spmv_paths(sp, torch, m, n, rp, ci, vv, x_dev):
    """Call time of y = A x through each SpMV path on one matrix: the default
    plan's choice, the row bins (no SELL, no streams), the entry-balanced
    one-kernel stream (one column panel) and eight column panels."""
    paths = {"x_window_stream": dict(), "row_bins": dict(use_sell=0, col_panels=0, x_window_bits=0),
             "entry_balanced_stream": dict(use_sell=0, col_panels=1, x_window_bits=0),
             "column_panels_8": dict(use_sell=0, col_panels=8, x_window_bits=0)}
    y = torch.empty(m, device="cuda")
    out = {}
    for key, o in paths.items():
        plan = sp.Plan(m, n, rp, ci, vv, **o)
        for _ in range(3):
            sp.spmv(plan, 1.0, x_dev, 0.0, y)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            sp.spmv(plan, 1.0, x_dev, 0.0, y)
        e1.record()
        torch.cuda.synchronize()
        out[key] = dict(ms=round(e0.elapsed_time(e1) / 20, 5), options=o)
        del plan
    return out


def measure(w, args, stream):
    """Warm-up, then exactly args.steps timed steps; returns the record."""
    import numpy as np
    import torch
    for _ in range(args.warmup):
        w.step()
    if w.restore:
        w.restore()
    torch.cuda.synchronize()
    # Short single-kernel steps are timed as replays of a captured HIP graph of
    # G back-to-back steps, so that the events measure the kernels and not the
    # host's launch rate; G divides the step count.
    G = args.graph_batch if args.graph_batch >= 0 else w.graph
    graph = None
    if G > 0:
        G = max(g for g in range(1, min(G, args.steps) + 1) if args.steps % g == 0)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(G):
                w.step()
        torch.cuda.synchronize()
    nrec = args.steps // G if G > 0 else args.steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(nrec)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(nrec)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(nrec):
        if w.restore_every and i > 0 and i % w.restore_every == 0:
            w.restore()
        starts[i].record(stream)
        if graph is not None:
            graph.replay()
        else:
            w.step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    r = dict(metric=METRIC, unit="GFLOP/s")
    if w.iterates_finite is not None:
        r["iterates_finite"] = w.iterates_finite()
    ev_ms = [s.elapsed_time(e) / (G if G > 0 else 1) for s, e in zip(starts, ends)]
    if graph is not None:
        # the graph's result equals an eager step's, bit for bit (deterministic kernels)
        if w.out_tensor is not None:
            got = w.out_tensor.clone()
            w.step()
            torch.cuda.synchronize()
            r["graph_replay_matches_eager"] = bool(torch.equal(got, w.out_tensor))
        r["graph_batch"] = G
    ms_per_step = elapsed * 1e3 / args.steps
    launch_ms = float(np.mean(ev_ms)) / w.launches
    r["value"] = round(w.flops / (ms_per_step * 1e-3) / 1e9, 3)
    r["ms_per_step"] = round(ms_per_step, 5)
    r["dtype"] = w.dtype
    r["config"] = w.config
    if w.digest:
        r["config"]["input_sha256"] = w.digest
    per_launch_bytes = w.nbytes / w.launches
    per_launch_flops = w.flops / w.launches
    if w.bound == "hbm":
        achieved = per_launch_bytes / (launch_ms * 1e-3) / 1e9
    else:
        achieved = per_launch_flops / (launch_ms * 1e-3) / 1e12
    # the committed counters were taken on the default plan: not for a run
    # with other plan options or an autotuned plan
    default_plan = not (w.config.get("plan_options") or w.config.get("autotune"))
    tr = load_traffic_record(w.name) if default_plan else None
    roof = dict(bound=w.bound, achieved=round(achieved, 2), peak=w.peak, unit=w.unit, frac=round(achieved / w.peak, 4),
                traffic=None if tr is None else tr.get("bytes_per_launch"),
                kernel_ms=round(launch_ms, 5), algorithmic_bytes_per_launch=int(per_launch_bytes),
                flops_per_launch=int(per_launch_flops), event_ms_median=round(float(np.median(ev_ms)), 5),
                event_ms_min=round(float(np.min(ev_ms)), 5))
    if tr is not None:
        for k in ("read_bytes_per_launch", "write_bytes_per_launch", "l2_hit_rate", "method"):
            if k in tr:
                roof["traffic_" + k.replace("_per_launch", "")] = tr[k]
    if w.bound == "mfma":
        roof["hbm_gbs"] = round(per_launch_bytes / (launch_ms * 1e-3) / 1e9, 1)
        roof["frac_of_hbm_peak"] = round(per_launch_bytes / (launch_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    if "gather_bound_bytes" in w.extra:
        gb = w.extra["gather_bound_bytes"]
        roof["gather_bound_bytes"] = int(gb)
        roof["gather_bound_gbs"] = round(gb / (launch_ms * 1e-3) / 1e9, 1)
        roof["gather_bound_frac"] = round(gb / (launch_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    r["roofline"] = roof
    r["gflops_event"] = round(per_launch_flops / (launch_ms * 1e-3) / 1e9, 2)

    # cold-cache reps: asked for, or by default where the working set is under
    # the 256 MB MALL (so that warm numbers read part of it from there)
    cold_reps = args.cold if args.cold >= 0 else (10 if per_launch_bytes < (256 << 20) else 0)
    if cold_reps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(cold_reps)]
        # each rep: flush, one timed step (cold), then one more timed step the
        # same way (warm: what the flushed step left in the caches)
        for i in range(cold_reps):
            if w.restore:
                w.restore()  # before the flush, so the copy leaves nothing in the caches
            flush.fill_(i & 255)
            for j in (0, 2):
                ev[i][j].record(stream)
                w.step()
                ev[i][j + 1].record(stream)
        torch.cuda.synchronize()
        del flush
        cold_ms = [e[0].elapsed_time(e[1]) / w.launches for e in ev]
        single_ms = [e[2].elapsed_time(e[3]) / w.launches for e in ev]
        med = float(np.median(cold_ms))
        if w.bound == "hbm":
            cold_achieved = per_launch_bytes / (med * 1e-3) / 1e9
        else:
            cold_achieved = per_launch_flops / (med * 1e-3) / 1e12
        r["cold"] = dict(reps=cold_reps, flush_bytes=512 << 20, kernel_ms_median=round(med, 5),
                         kernel_ms_min=round(float(np.min(cold_ms)), 5), achieved=round(cold_achieved, 2),
                         unit=w.unit, frac=round(cold_achieved / w.peak, 4),
                         warm_single_ms_median=round(float(np.median(single_ms)), 5))
    r["setup"] = {k: round(v, 2) for k, v in w.setup.items()}
    if args.counter_run:
        r["launches_per_step"] = w.launches
    return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=None,
                    choices=ALL_WORKLOADS + ["spmm_lognormal", "spmm_clustered", "spmm_skewed"],
                    help="run only this workload (spmm_lognormal / spmm_clustered / spmm_skewed take --N)")
    ap.add_argument("--N", type=int, default=32, help="right-hand-side columns for --config spmm_lognormal")
    ap.add_argument("--graph-batch", type=int, default=-1,
                    help="steps per replay of a captured HIP graph in the timed region (0: one plain launch per "
                         "step; -1: 20 for workloads whose step is a single short kernel, else 0)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", type=int, default=-1, metavar="R",
                    help="after the timed region, also time R single steps each preceded by writing a 512 MiB "
                         "buffer (evicts the L2s and the 256 MB MALL): cold-cache numbers, reported under 'cold'; "
                         "-1 (default): 10 for workloads whose algorithmic bytes per launch are under 256 MiB, "
                         "else none")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="oracle time of the headline's CPU baseline (half on all threads, half on one)")
    ap.add_argument("--cpu-seconds-other", type=float, default=2.0,
                    help="oracle time of every other workload's CPU baseline")
    ap.add_argument("--cpu-sample-gflop", type=float, default=1.0,
                    help="flops of the row sample when a full oracle pass would be longer")
    ap.add_argument("--options", default="", help="plan options, e.g. group_nnz=1024,wave_min=128")
    ap.add_argument("--autotune", action="store_true",
                    help="SpMV workloads: time the default candidate plans (sp_autotune_spmv), then build the plan "
                         "from the tuning cache; the candidates' times are reported under 'autotune'")
    ap.add_argument("--no-gather-probe", dest="gather_probe", action="store_false",
                    help="skip the probes (the gather rate over the power-law matrix's columns, the LDS feed "
                         "rates beside bsr_blocks)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device copy (5 launches) to calibrate HBM byte counters")
    ap.add_argument("--counter-run", action="store_true",
                    help="the run a counter pass profiles: warm-up and timed steps as plain launches, nothing else "
                         "on the GPU but the workload's setup (no probes, comparisons or CPU baseline)")
    ap.add_argument("--collect-traffic", default=None, metavar="NAMES",
                    help="comma-separated workloads (or 'all'; plan options after '+', e.g. "
                         "spmv_powerlaw+col_panels=8): run rocprofv3 counter and kernel-trace passes over "
                         "'--counter-run' children and write traffic_<workload>.json and a kernel summary per "
                         "workload to --traffic-out")
    ap.add_argument("--traffic-out", default=None, metavar="DIR")
    ap.add_argument("--summarize-only", action="store_true",
                    help="with --collect-traffic: rewrite the summaries from DIR/raw without profiling")
    args = ap.parse_args()
    if args.collect_traffic:
        if not args.traffic_out:
            ap.error("--collect-traffic needs --traffic-out")
        collect_traffic(args.collect_traffic, args.traffic_out, args.summarize_only)
        return
    if args.counter_run:
        args.no_cpu_baseline, args.gather_probe, args.graph_batch, args.cold = True, False, 0, 0
    if args.copy_calibration:
        import torch
        n = 64 << 20  # floats: 256 MiB per buffer
        src = torch.ones(n, device="cuda")
        dst = torch.empty(n, device="cuda")
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps(dict(copy_bytes_read=4 * n, copy_bytes_written=4 * n, launches=5)))
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the sparse products here are single-GPU kernels (rows would be "
              "sharded across GPUs with x all-gathered first, which is not built); --gpus %d is not supported"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    opts = {}
    for kv in filter(None, args.options.split(",")):
        k, v = kv.split("=")
        opts[k] = int(v)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    if args.config is None:
        names = ALL_WORKLOADS
    elif args.config in ("spmm_lognormal", "spmm_clustered", "spmm_skewed"):
        names = ["%s_N%d" % (args.config, args.N)]
    else:
        names = [args.config]
    copy_gbs = copy_rate_gbs()
    if not args.counter_run:  # (a counter run counts every dispatch of the call's kernels)
        warm_library()
    records = {}
    for i, name in enumerate(names):
        log("workload", name)
        w = prepare(name, args, opts if i == 0 else {})
        rec = measure(w, args, stream)
        if w.bound == "hbm":
            rec["roofline"]["measured_copy_gbs"] = round(copy_gbs, 1)
            rec["roofline"]["frac_of_copy"] = round(rec["roofline"]["achieved"] / copy_gbs, 4)
        probe = getattr(w, "probe", None)
        if probe is not None:
            p = gather_probe(*probe)
            rec["gather_probe"] = p
            # the one-pass floor: every entry's gather at the best measured rate
            # (x cut into L2-sized slices, one per XCD), against this call's time
            floor_ms = p["entries"] / (p["gather_2MiB_slice_gps"] * 1e9) * 1e3
            rec["roofline"]["measured_gather_rate"] = p["gather_2MiB_slice_gps"]
            rec["roofline"]["one_pass_gather_floor_ms"] = round(floor_ms, 5)
            rec["roofline"]["frac_of_gather_floor"] = round(floor_ms / rec["roofline"]["kernel_ms"], 4)
        if w.name == "bsr_blocks" and args.gather_probe:
            rec["feed_probe"] = feed_probe()
            tb = rec["roofline"].get("traffic")
            if tb:  # what the call moves between the L2s and memory, per second
                rec["roofline"]["traffic_tbs"] = round(tb / (rec["roofline"]["kernel_ms"] * 1e-3) / 1e12, 2)
        if w.cpu is not None:
            secs = args.cpu_seconds if i == 0 else args.cpu_seconds_other
            rec["cpu_baseline"] = cpu_baseline(w.cpu, secs)
        elif not args.no_cpu_baseline:
            rec["cpu_baseline"] = None
        records[name] = rec
        del w
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    head = records[names[0]]
    result = dict(metric=METRIC, value=head["value"], unit="GFLOP/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
                  ms_per_step=head["ms_per_step"], higher_is_better=True, scaling="weak", vs_baseline=None,
                  dtype=head["dtype"], data="synthetic (seeded generators in gen/, seed 0)", config=head["config"],
                  roofline=head["roofline"])
    for k, v in head.items():
        if k not in result and k not in ("metric", "unit"):
            result[k] = v
    if len(names) > 1:
        result["configs"] = {k: {kk: vv for kk, vv in v.items() if kk not in ("metric",)}
                             for k, v in records.items() if k != names[0]}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
