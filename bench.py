#!/usr/bin/env python3
"""Throughput of the sparse x dense products on one MI355X.

Default workload: CSR SpMV y = A x on the power-law matrix (2^22 x 2^22,
lognormal row lengths plus planted hub rows, ~46.8M entries, fp32).  One step
is one `spmv` call: every row bin of the plan (group / wave / block / split
rows and the split reduction, with the fused axpby store).  The one-time work
(COO -> CSR build, plan) is timed separately and reported under "setup".

Prints ONE JSON line.  Other workloads (--config) exist for profiling:
  spmv_uniform, spmv_powerlaw, stencil27 (u <- A v - a u, v <- A^T u - b v per
  step), spmm_lognormal (--N), bsr_blocks.
"""
import argparse
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
# Sources whose code decides the kernels each workload runs (a committed
# traffic summary is used only while these are unchanged).
_CSRC = "spmm_csr_spmv_amd/csrc/"
KERNEL_SOURCES = {
    "spmv": [_CSRC + f for f in ("spmv.hip", "pstream.hip", "xwin.hip", "seg_rows.h", "device_common.h", "internal.h",
                                 "api.cpp")],
    "spmm": [_CSRC + f for f in ("spmm.hip", "device_common.h", "internal.h", "api.cpp")],
    "bsr": [_CSRC + f for f in ("bsr.hip", "device_common.h", "internal.h")],
    "bsr_spmv": [_CSRC + f for f in ("bsr_convert.hip", "device_common.h", "internal.h")],
    "wcsr": [_CSRC + f for f in ("wcsr.hip", "device_common.h", "internal.h")],
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


def bsr_bytes(mb, kb, bs, nnzb, N, beta_nonzero=False):
    return 2 * nnzb * bs * bs + 4 * (nnzb + mb + 1) + 2 * kb * bs * N + 4 * mb * bs * N * (2 if beta_nonzero else 1)


def bsr_flops(nnzb, bs, N):
    return 2 * nnzb * bs * bs * N


def bsr_spmv_bytes(m, n, bs, nnzb, beta_nonzero=False):
    """BSR SpMV with fp32 blocks: every stored block (4 bs^2 B), block column
    indices and block row pointer, x and y once."""
    mb = (m + bs - 1) // bs
    return 4 * nnzb * bs * bs + 4 * (nnzb + mb + 1) + 4 * n + 4 * m + (4 * m if beta_nonzero else 0)


def csr_storage_bytes(m, nnz, val_bytes=8, idx_bytes=4):
    """Bytes of a CSR (values, column indices, row pointer of m+1 entries)."""
    return nnz * (val_bytes + idx_bytes) + (m + 1) * idx_bytes


def coo_storage_bytes(nnz, val_bytes=8, idx_bytes=4):
    return nnz * (val_bytes + 2 * idx_bytes)


def dual_storage_bytes(m, n, nnz):
    """CSR + CSC of an fp32/int32 matrix (LSMR page, section 4)."""
    return 2 * (8 * nnz + 4 * (m + n + 2))


def block_index_bytes_per_value(bs, idx_bytes=4):
    return idx_bytes / float(bs * bs)


def kernel_family(workload):
    if workload == "bsr_spmv":
        return "bsr_spmv"
    if workload.startswith("spmm_clustered"):
        return "wcsr"
    return "bsr" if workload.startswith("bsr") else ("spmm" if workload.startswith("spmm") else "spmv")


def kernel_fingerprint(workload):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel_family(workload)]:
        with open(os.path.join(HERE, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload, launches_bytes):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernels (same fingerprint); else None."""
    path = os.path.join(HERE, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_fingerprint") != kernel_fingerprint(workload):
        return None
    return t.get("bytes_per_launch")


# --------------------------------------------------------------------------
def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="spmv_powerlaw",
                    choices=["spmv_uniform", "spmv_powerlaw", "stencil27", "spmm_lognormal", "bsr_blocks", "bsr_spmv",
                             "spmm_clustered"])
    ap.add_argument("--N", type=int, default=32, help="right-hand-side columns for spmm_lognormal")
    ap.add_argument("--graph-batch", type=int, default=-1,
                    help="steps per replay of a captured HIP graph in the timed region (0: one plain launch per "
                         "step; -1: up to 20 for workloads whose step is a single short kernel, else 0)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", type=int, default=0, metavar="R",
                    help="after the timed region, also time R single steps each preceded by writing a 512 MiB "
                         "buffer (evicts the L2s and the 256 MB MALL): cold-cache numbers, reported under 'cold'")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--options", default="", help="plan options, e.g. group_nnz=1024,wave_min=128")
    ap.add_argument("--autotune", action="store_true",
                    help="SpMV workloads: time the default candidate plans (sp_autotune_spmv), then build the plan "
                         "from the tuning cache; the candidates' times are reported under 'autotune'")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device copy (5 launches) to calibrate HBM byte counters")
    args = ap.parse_args()
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

    import numpy as np
    import torch

    import gen
    import spmm_csr_spmv_amd as sp

    opts = {}
    for kv in filter(None, args.options.split(",")):
        k, v = kv.split("=")
        opts[k] = int(v)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    setup = {}
    cfg = args.config
    result = dict(metric="SpMV/SpMM GFLOP/s + achieved HBM GB/s vs MI355X peak (fp32), 1 GPU", unit="GFLOP/s",
                  n_gpus=1, steps=args.steps, warmup=args.warmup, higher_is_better=True, scaling="weak",
                  vs_baseline=None, data="synthetic (seeded generators in gen/, seed 0)")

    t0 = time.time()
    if cfg == "bsr_blocks":
        b = gen.block_sparse_bsr(seed=0)
        N = 512
        Bh = gen.bf16_matrix(b.kb * b.bs, N, seed=0)
        d_brow, d_bcol = torch.from_numpy(b.brow_ptr).cuda(), torch.from_numpy(b.bcol).cuda()
        d_bval = torch.from_numpy(b.bval.view(np.int16)).cuda()
        d_B = torch.from_numpy(Bh.view(np.int16)).cuda()
        C = torch.empty(b.mb * b.bs, N, device="cuda")
        setup["generate_s"] = time.time() - t0

        def step():
            sp.bsr_spmm(b.mb, b.kb, b.bs, d_brow, d_bcol, d_bval, d_B, 1.0, 0.0, C)

        out_tensor = C

        flops = bsr_flops(b.nnzb, b.bs, N)
        nbytes = bsr_bytes(b.mb, b.kb, b.bs, b.nnzb, N)
        launches = 1
        dtype = "bf16 in / f32 acc"
        config = dict(workload=cfg, M=b.mb * b.bs, K=b.kb * b.bs, block=b.bs, nnz_blocks=b.nnzb, N=N)
        bound, peak, unit = "mfma", PEAK_BF16_TFLOPS, "TFLOP/s"
        cpu_leg = None
    elif cfg == "bsr_spmv":
        bs = 64
        coo = gen.block_sparse_coo(seed=0)
        setup["generate_s"] = time.time() - t0
        m, n = coo.m, coo.n
        d_row, d_col, d_val = (torch.from_numpy(a).cuda() for a in (coo.row, coo.col, coo.val))
        torch.cuda.synchronize()
        t1 = time.time()
        rp, ci, vv = sp.csr_build_from_coo(m, n, d_row, d_col, d_val)
        torch.cuda.synchronize()
        setup["csr_build_from_coo_ms"] = (time.time() - t1) * 1e3
        del d_row, d_col, d_val
        t1 = time.time()
        brp, bcol, bval, fill = sp.csr_to_bsr(m, n, rp, ci, vv, bs, min_fill=0.5)
        torch.cuda.synchronize()
        setup["csr_to_bsr_ms"] = (time.time() - t1) * 1e3
        nnzb = bcol.numel()
        x = torch.from_numpy(gen.dense_vector(n, 0, 1)).cuda()
        y = torch.zeros(m, device="cuda")

        def step():
            sp.bsr_spmv(m, n, bs, brp, bcol, bval, 1.0, x, 0.0, y)

        out_tensor = y

        flops = 2 * nnzb * bs * bs
        nbytes = bsr_spmv_bytes(m, n, bs, nnzb)
        launches = 1
        dtype = "f32"
        config = dict(workload=cfg, M=m, K=n, block=bs, nnz=coo.nnz, nnz_blocks=nnzb, fill_ratio=fill)
        bound, peak, unit = "hbm", PEAK_HBM_GBS, "GB/s"
        h_brp, h_bcol, h_bval, h_x = (t.cpu().numpy() for t in (brp, bcol, bval, x))

        def cpu_call():
            import oracle
            oracle.bsr_spmv(m, n, bs, h_brp, h_bcol, h_bval, h_x)

        cpu_leg = (cpu_call, flops, "full passes of y = A x over the same 64 x 64-block BSR (fp32 blocks, fp64 "
                                    "accumulation, single-threaded C loop)")
    elif cfg == "spmm_clustered":
        coo = gen.clustered_coo(seed=0)
        setup["generate_s"] = time.time() - t0
        m, n, nnz = coo.m, coo.n, coo.nnz
        N = args.N
        d_row, d_col, d_val = (torch.from_numpy(a).cuda() for a in (coo.row, coo.col, coo.val))
        torch.cuda.synchronize()
        t1 = time.time()
        rp, ci, vv = sp.csr_build_from_coo(m, n, d_row, d_col, d_val)
        torch.cuda.synchronize()
        setup["csr_build_from_coo_ms"] = (time.time() - t1) * 1e3
        del d_row, d_col, d_val
        t1 = time.time()
        wp, wc, wv, fill = sp.csr_to_wcsr(m, n, rp, ci, vv, pad=8)
        torch.cuda.synchronize()
        setup["csr_to_wcsr_ms"] = (time.time() - t1) * 1e3
        total_cols = wc.numel()
        B = torch.from_numpy(gen.dense_matrix(n, N, 0)).cuda()
        C = torch.empty(m, N, device="cuda")

        def step():
            sp.wcsr_spmm(m, n, wp, wc, wv, 1.0, B, 0.0, C)

        out_tensor = C
        flops = 2 * nnz * N
        nbytes = spmm_bytes(m, n, nnz, N)
        launches = 1
        dtype = "f32"
        config = dict(workload=cfg, M=m, K=n, nnz=nnz, N=N, window=64, compressed_columns=total_cols,
                      window_fill=round(fill, 4),
                      mfma_flops=2 * total_cols * 64 * N,
                      wcsr_bytes=4 * total_cols * 64 + 4 * total_cols + 4 * total_cols * N + 4 * m * N)
        bound, peak, unit = "hbm", PEAK_HBM_GBS, "GB/s"
        # the CSR SpMM on the same matrix, for comparison
        plan_c = sp.Plan(m, n, rp, ci, vv, max_N=N)
        for _ in range(3):
            sp.spmm(plan_c, 1.0, B, 0.0, C)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            sp.spmm(plan_c, 1.0, B, 0.0, C)
        e1.record(stream)
        torch.cuda.synchronize()
        config["csr_spmm_ms_same_matrix"] = round(e0.elapsed_time(e1) / 10, 5)
        del plan_c
        cpu_leg = None
    else:
        coo = {"spmv_uniform": lambda: gen.uniform_rows_coo(seed=0),
               "spmv_powerlaw": lambda: gen.powerlaw_coo(seed=0),
               "stencil27": lambda: gen.stencil27_coo(seed=0),
               "spmm_lognormal": lambda: gen.lognormal_coo(seed=0)}[cfg]()
        setup["generate_s"] = time.time() - t0
        m, n, nnz = coo.m, coo.n, coo.nnz
        d_row, d_col, d_val = (torch.from_numpy(a).cuda() for a in (coo.row, coo.col, coo.val))
        torch.cuda.synchronize()
        t1 = time.time()
        rp, ci, vv = sp.csr_build_from_coo(m, n, d_row, d_col, d_val)
        torch.cuda.synchronize()
        setup["csr_build_from_coo_ms"] = (time.time() - t1) * 1e3
        del d_row, d_col, d_val
        csc = None
        if cfg == "stencil27":
            t1 = time.time()
            csc = sp.csr_to_csc(m, n, rp, ci, vv)
            torch.cuda.synchronize()
            setup["csr_to_csc_ms"] = (time.time() - t1) * 1e3
        N = args.N if cfg == "spmm_lognormal" else 1
        tune = None
        if args.autotune and cfg != "spmm_lognormal":
            x_t = torch.from_numpy(gen.dense_vector(n, 0, 1)).cuda()
            t1 = time.time()
            best, ms, best_opts = sp.autotune_spmv(m, n, rp, ci, vv, x_t, reps=10)
            setup["autotune_ms"] = (time.time() - t1) * 1e3
            tune = dict(candidates=[dict(c) for c in sp.DEFAULT_CANDIDATES], ms_per_call=[round(t, 5) for t in ms],
                        best=best)
            del x_t
        t1 = time.time()
        if tune is not None:
            plan = sp.Plan(m, n, rp, ci, vv, csc=csc, max_N=N, tuned=True)
        else:
            plan = sp.Plan(m, n, rp, ci, vv, csc=csc, max_N=N, **opts)
        torch.cuda.synchronize()
        setup["plan_ms"] = (time.time() - t1) * 1e3
        prof = plan.profile()
        x = torch.from_numpy(gen.dense_vector(n, 0, 1)).cuda()
        y = torch.zeros(m, device="cuda")
        config = dict(workload=cfg, M=m, K=n, nnz=nnz, row_len_mean=round(prof["mean"], 3), p95=prof["p95"],
                      p99=prof["p99"], max_row=prof["max_len"],
                      bins=dict(group_tasks=prof["group_tasks"], wave_rows=prof["wave_rows"],
                                block_rows=prof["block_rows"], split_rows=prof["split_rows"],
                                split_segments=prof["split_segments"]),
                      path="x-window stream" if prof["x_window_bits"] else
                      ("column-panel stream" if prof["col_panels"] else
                       ("SELL-C-sigma" if prof["sell_slots"] else "row bins")))
        if opts:
            config["plan_options"] = opts
        if tune is not None:
            result["autotune"] = tune
            config["col_panels"] = prof["col_panels"]
        bound, peak, unit = "hbm", PEAK_HBM_GBS, "GB/s"
        dtype = "f32"
        if cfg == "stencil27":
            u = torch.from_numpy(gen.dense_vector(m, 0, 2)).cuda()
            v = torch.from_numpy(gen.dense_vector(n, 0, 3)).cuda()
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

            flops = 2 * spmv_flops(m, nnz, True)
            nbytes = 2 * spmv_bytes(m, n, nnz, True)  # per step (two launches)
            launches = 2
            config["step"] = "u <- A v - alpha u ; v <- A^T u - beta v"
            # the iterates grow by about |A| per step and pass the fp32 range
            # after some 20 steps: put u, v back every 8 steps (inside the
            # wall-clock region, outside the per-step events)
            restore_every = 8
            config["restore_every"] = restore_every

            def iterates_finite():
                return bool(torch.isfinite(u).all().item() and torch.isfinite(v).all().item())
        elif cfg == "spmm_lognormal":
            B = torch.from_numpy(gen.dense_matrix(n, N, 0)).cuda()
            C = torch.empty(m, N, device="cuda")

            def step():
                sp.spmm(plan, 1.0, B, 0.0, C)

            out_tensor = C

            flops = 2 * nnz * N
            nbytes = spmm_bytes(m, n, nnz, N)
            launches = 1
            config["N"] = N
        else:
            def step():
                sp.spmv(plan, 1.0, x, 0.0, y)

            out_tensor = y

            flops = spmv_flops(m, nnz)
            nbytes = spmv_bytes(m, n, nnz)
            launches = 1
        cpu_leg = None
        if cfg in ("spmv_powerlaw", "spmv_uniform"):
            h_rp, h_ci, h_vv, h_x = (t.cpu().numpy() for t in (rp, ci, vv, x))

            def cpu_call():
                import oracle
                oracle.spmv(h_rp, h_ci, h_vv, h_x)

            cpu_leg = (cpu_call, spmv_flops(m, nnz), "full passes of y = A x over the same %s matrix (fp64 "
                                                     "accumulation, single-threaded C loop)" % cfg)

    restore_fn = locals().get("restore")
    restore_every = locals().get("restore_every", 0)
    # ---------------- warmup + timed region
    for _ in range(args.warmup):
        step()
    if restore_fn:
        restore_fn()
    torch.cuda.synchronize()
    # Short single-kernel steps are timed as replays of a captured HIP graph of
    # G back-to-back steps, so that the events measure the kernels and not the
    # host's launch rate; G divides the step count.
    G = args.graph_batch
    if G < 0:
        G = 20 if cfg in ("spmv_uniform", "bsr_spmv", "bsr_blocks") else 0
    if G > 0:
        G = max(g for g in range(1, min(G, args.steps) + 1) if args.steps % g == 0)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(G):
                step()
        torch.cuda.synchronize()
    nrec = args.steps // G if G > 0 else args.steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(nrec)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(nrec)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(nrec):
        if restore_every and i > 0 and i % restore_every == 0:
            restore_fn()
        starts[i].record(stream)
        if G > 0:
            graph.replay()
        else:
            step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    finite = locals().get("iterates_finite")
    if finite is not None:
        result["iterates_finite"] = finite()
    ev_ms = [s.elapsed_time(e) / (G if G > 0 else 1) for s, e in zip(starts, ends)]
    if G > 0:
        # the graph's result equals an eager step's, bit for bit (deterministic kernels)
        out = locals().get("out_tensor")
        if out is not None:
            got = out.clone()
            step()
            torch.cuda.synchronize()
            result["graph_replay_matches_eager"] = bool(torch.equal(got, out))
        result["graph_batch"] = G
    ms_per_step = elapsed * 1e3 / args.steps
    launch_ms = float(np.mean(ev_ms)) / launches
    step_flops_s = flops / (ms_per_step * 1e-3)
    result["value"] = round(step_flops_s / 1e9, 3)
    result["ms_per_step"] = round(ms_per_step, 5)
    result["dtype"] = dtype
    result["config"] = config
    per_launch_bytes = nbytes / launches
    per_launch_flops = flops / launches
    if bound == "hbm":
        achieved = per_launch_bytes / (launch_ms * 1e-3) / 1e9
    else:
        achieved = per_launch_flops / (launch_ms * 1e-3) / 1e12
    traffic = load_traffic(cfg + ("_N%d" % N if cfg in ("spmm_lognormal", "spmm_clustered") else ""), per_launch_bytes)
    result["roofline"] = dict(bound=bound, achieved=round(achieved, 2), peak=peak, unit=unit,
                              frac=round(achieved / peak, 4), traffic=traffic,
                              kernel_ms=round(launch_ms, 5), algorithmic_bytes_per_launch=int(per_launch_bytes),
                              flops_per_launch=int(per_launch_flops), event_ms_median=round(float(np.median(ev_ms)), 5))
    if bound == "mfma":
        result["roofline"]["hbm_gbs"] = round(per_launch_bytes / (launch_ms * 1e-3) / 1e9, 1)
    result["roofline"]["event_ms_min"] = round(float(np.min(ev_ms)), 5)
    # the copy rate this GPU measures now (outside the timed region): a plain
    # 256 MiB device copy, read + write bytes over its time, as a reference
    # beside the 8 TB/s spec (algorithmic bytes can exceed what a kernel
    # moves, so the fraction can pass 1)
    if bound == "hbm":
        ref = torch.ones(64 << 20, device="cuda")
        dst = torch.empty_like(ref)
        dst.copy_(ref)
        t = []
        for _ in range(5):
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            dst.copy_(ref)
            a1.record(stream)
            torch.cuda.synchronize()
            t.append(a0.elapsed_time(a1))
        del ref, dst
        copy_gbs = 2 * (64 << 20) * 4 / (float(np.median(t)) * 1e-3) / 1e9
        result["roofline"]["measured_copy_gbs"] = round(copy_gbs, 1)
        result["roofline"]["frac_of_copy"] = round(achieved / copy_gbs, 4)
    result["gflops_event"] = round(per_launch_flops / (launch_ms * 1e-3) / 1e9, 2)

    # ---------------- cold-cache steps (outside the timed region, on request)
    if args.cold > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.cold)]
        # each rep: flush, one timed step (cold), then one more timed step the
        # same way (warm: what the flushed step left in the caches), so that
        # the difference is the caches' and not the single launch's
        for i in range(args.cold):
            if restore_fn:
                restore_fn()  # before the flush, so the copy leaves nothing in the caches
            flush.fill_(i & 255)
            for j in (0, 2):
                ev[i][j].record(stream)
                step()
                ev[i][j + 1].record(stream)
        torch.cuda.synchronize()
        del flush
        cold_ms = [e[0].elapsed_time(e[1]) / launches for e in ev]
        single_ms = [e[2].elapsed_time(e[3]) / launches for e in ev]
        med = float(np.median(cold_ms))
        if bound == "hbm":
            cold_achieved = per_launch_bytes / (med * 1e-3) / 1e9
        else:
            cold_achieved = per_launch_flops / (med * 1e-3) / 1e12
        result["cold"] = dict(reps=args.cold, flush_bytes=512 << 20, kernel_ms_median=round(med, 5),
                              kernel_ms_min=round(float(np.min(cold_ms)), 5), achieved=round(cold_achieved, 2),
                              unit=unit, frac=round(cold_achieved / peak, 4),
                              warm_single_ms_median=round(float(np.median(single_ms)), 5))
    result["setup"] = {k: round(v, 2) for k, v in setup.items()}

    # ---------------- CPU baseline: the oracle on the host cores
    if not args.no_cpu_baseline and cpu_leg is not None:
        cpu_call, cpu_flops, cpu_desc = cpu_leg
        reps, t_cpu = 0, 0.0
        t0 = time.perf_counter()
        while t_cpu < args.cpu_seconds and reps < 1000:
            cpu_call()
            reps += 1
            t_cpu = time.perf_counter() - t0
        per = t_cpu / reps
        result["cpu_baseline"] = dict(value=round(cpu_flops / per / 1e9, 4), unit="GFLOP/s", cores=1, kind="oracle",
                                      sample="%d %s, %.1f s" % (reps, cpu_desc, t_cpu))
    elif not args.no_cpu_baseline:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
