"""ctypes binding of libspmm_csr_spmv.so -- argument marshalling only.

Every function here has the name of the C entry point it calls and does no
arithmetic of its own: it checks dtypes/devices, allocates outputs and
workspaces with torch (PyTorch is the device-memory and stream provider),
passes raw device pointers and the current torch HIP stream, and raises
SparseError on a non-zero status.

Streams: a call given `stream=` enqueues its kernels there and allocates its
outputs and workspaces on that stream (torch's caching allocator then does not
hand the memory to other streams' work before the call's kernels are done); a
plan's workspace used on another stream is marked with record_stream.
"""
import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspmm_csr_spmv.so")

SP_OK = 0
STATUS = {0: "SP_OK", 1: "SP_ERR_NULL", 2: "SP_ERR_SIZE", 3: "SP_ERR_INDEX", 4: "SP_ERR_WORKSPACE",
          5: "SP_ERR_UNSUPPORTED", 6: "SP_ERR_HIP", 7: "SP_ERR_STATE", 8: "SP_ERR_FILL"}

# Names declared in include/spmm_csr_spmv.h.
EXPORTS = ("sp_status_string", "sp_version", "csr_build_from_coo_bufsize", "csr_build_from_coo",
           "csr_to_csc_bufsize", "csr_to_csc", "sp_plan_options_default", "sp_plan_create",
           "sp_plan_workspace_size", "sp_plan_bind", "sp_plan_profile", "sp_plan_destroy", "spmv", "spmv_t", "spmm",
           "csr_to_bsr_bufsize", "csr_to_bsr_analyze", "csr_to_bsr_fill", "bsr_spmv", "bsr_spmm_bufsize", "bsr_spmm",
           "sp_plan_dispatch_key", "sp_tune_cache_store", "sp_tune_cache_lookup", "sp_tune_cache_clear",
           "sp_tune_cache_size", "sp_autotune_workspace_size", "sp_autotune_spmv", "csr_to_wcsr_bufsize",
           "csr_to_wcsr_analyze", "csr_to_wcsr_fill", "wcsr_spmm", "sp_plan_view_create",
           "csr_build_from_coo_noalloc", "bsr_spmv_rowwise", "wcsr_tasks_bufsize", "wcsr_tasks_build",
           "wcsr_spmm_tasks_bufsize", "wcsr_spmm_tasks")


class SparseError(RuntimeError):
    def __init__(self, fn, code, lib=None):
        msg = lib.sp_status_string(code).decode() if lib is not None else STATUS.get(code, str(code))
        super().__init__("%s failed: %s" % (fn, msg))
        self.code = code
        self.fn = fn


class sp_plan_options(ctypes.Structure):
    _fields_ = [("group_nnz", ctypes.c_int32), ("wave_min", ctypes.c_int32), ("block_min", ctypes.c_int32),
                ("split_min", ctypes.c_int32), ("split_seg", ctypes.c_int32), ("use_sell", ctypes.c_int32),
                ("sell_sigma", ctypes.c_int32), ("xcd_remap", ctypes.c_int32), ("col_panels", ctypes.c_int32),
                ("x_window_bits", ctypes.c_int32), ("spmm_phase_bits", ctypes.c_int32)]


class sp_profile(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("nnz", ctypes.c_int64),
                ("mean", ctypes.c_double), ("var", ctypes.c_double), ("cv", ctypes.c_double),
                ("p95", ctypes.c_int64), ("p99", ctypes.c_int64), ("max_len", ctypes.c_int64),
                ("empty_rows", ctypes.c_int64),
                ("group_tasks", ctypes.c_int64), ("group_rows", ctypes.c_int64), ("group_nnz", ctypes.c_int64),
                ("wave_rows", ctypes.c_int64), ("wave_nnz", ctypes.c_int64),
                ("block_rows", ctypes.c_int64), ("block_nnz", ctypes.c_int64),
                ("split_rows", ctypes.c_int64), ("split_segments", ctypes.c_int64), ("split_nnz", ctypes.c_int64),
                ("sell_slots", ctypes.c_int64), ("col_panels", ctypes.c_int64), ("x_window_bits", ctypes.c_int64),
                ("spmm_phase_bits", ctypes.c_int64)]


class sp_dispatch_key(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("dtype", ctypes.c_int32), ("index_bits", ctypes.c_int32),
                ("transposed", ctypes.c_int32), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("nnz", ctypes.c_int64), ("N", ctypes.c_int32), ("arch", ctypes.c_int32),
                ("avg_len_q", ctypes.c_int32), ("p95_len_q", ctypes.c_int32), ("max_len_q", ctypes.c_int32),
                ("cv_q", ctypes.c_int32), ("version", ctypes.c_uint64)]


_lib = None
_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f = ctypes.c_float
_sz = ctypes.c_size_t


def lib():
    """The loaded library (loads it on first use; raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libspmm_csr_spmv.so is not built (%s); run __graft_entry__.build() or "
                              "python -m spmm_csr_spmv_amd.build" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        L.sp_status_string.argtypes = [ctypes.c_int]
        L.sp_status_string.restype = ctypes.c_char_p
        L.sp_version.restype = ctypes.c_int
        L.csr_build_from_coo_bufsize.argtypes = [_i64, _i64, _i64, ctypes.POINTER(_sz)]
        L.csr_build_from_coo.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p, _sz, _p]
        L.csr_build_from_coo_noalloc.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p]
        L.csr_to_csc_bufsize.argtypes = [_i64, _i64, _i64, ctypes.POINTER(_sz)]
        L.csr_to_csc.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p, _sz, _p]
        L.sp_plan_options_default.argtypes = [ctypes.POINTER(sp_plan_options)]
        L.sp_plan_create.argtypes = [ctypes.POINTER(_p), _i64, _i64, _i64, _p, _p, _p, _p, _p, _p,
                                     ctypes.POINTER(sp_plan_options), _p]
        L.sp_plan_workspace_size.argtypes = [_p, _i32, ctypes.POINTER(_sz)]
        L.sp_plan_bind.argtypes = [_p, _p, _sz, _i32, _p]
        L.sp_plan_profile.argtypes = [_p, _i32, ctypes.POINTER(sp_profile)]
        L.sp_plan_destroy.argtypes = [_p]
        L.sp_plan_view_create.argtypes = [_p, ctypes.POINTER(_p)]
        L.spmv.argtypes = [_p, _f, _p, _f, _p, _p]
        L.spmv_t.argtypes = [_p, _f, _p, _f, _p, _p]
        L.spmm.argtypes = [_p, _i32, _f, _p, _i64, _f, _p, _i64, _p]
        L.csr_to_bsr_bufsize.argtypes = [_i64, _i64, _i64, _i32, ctypes.POINTER(_sz)]
        L.csr_to_bsr_analyze.argtypes = [_i64, _i64, _i64, _p, _p, _i32, ctypes.c_double, _p,
                                         ctypes.POINTER(_i64), ctypes.POINTER(ctypes.c_double), _p, _sz, _p]
        L.csr_to_bsr_fill.argtypes = [_i64, _i64, _i64, _p, _p, _p, _i32, _p, _i64, _p, _p, _i32, _p]
        L.bsr_spmv.argtypes = [_i64, _i64, _i32, _i64, _p, _p, _p, _f, _p, _f, _p, _p]
        L.bsr_spmv_rowwise.argtypes = [_i64, _i64, _i32, _i64, _p, _p, _p, _f, _p, _f, _p, _p]
        L.bsr_spmm_bufsize.argtypes = [_i64, _i64, _i32, _i64, _i32, ctypes.POINTER(_sz)]
        L.csr_to_wcsr_bufsize.argtypes = [_i64, _i64, _i64, ctypes.POINTER(_sz)]
        L.csr_to_wcsr_analyze.argtypes = [_i64, _i64, _i64, _p, _p, _i32, _p, ctypes.POINTER(_i64),
                                          ctypes.POINTER(ctypes.c_double), _p, _sz, _p]
        L.csr_to_wcsr_fill.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _i64, _p, _p, _p]
        L.wcsr_spmm.argtypes = [_i64, _i64, _p, _p, _p, _i32, _f, _p, _i64, _f, _p, _i64, _p]
        L.wcsr_tasks_bufsize.argtypes = [_i64, _i64, _i32, ctypes.POINTER(_sz)]
        L.wcsr_tasks_build.argtypes = [_i64, _p, _i64, _i32, _p, _sz, ctypes.POINTER(_i64), ctypes.POINTER(_i64), _p]
        L.wcsr_spmm_tasks_bufsize.argtypes = [_i64, _i32, ctypes.POINTER(_sz)]
        L.wcsr_spmm_tasks.argtypes = [_i64, _i64, _p, _i64, _i64, _p, _p, _i32, _f, _p, _i64, _f, _p, _i64, _p, _sz,
                                      _p]
        _key = ctypes.POINTER(sp_dispatch_key)
        _opt = ctypes.POINTER(sp_plan_options)
        L.sp_plan_dispatch_key.argtypes = [_p, _i32, _i32, ctypes.c_uint64, _key]
        L.sp_tune_cache_store.argtypes = [_key, _opt]
        L.sp_tune_cache_lookup.argtypes = [_key, _opt, ctypes.POINTER(_i32)]
        L.sp_tune_cache_clear.argtypes = []
        L.sp_tune_cache_size.argtypes = [ctypes.POINTER(_i64)]
        L.sp_autotune_workspace_size.argtypes = [_i64, _i64, _i64, _p, _p, _p, _opt, _i32, ctypes.POINTER(_sz), _p]
        L.sp_autotune_spmv.argtypes = [_i64, _i64, _i64, _p, _p, _p, _opt, _i32, _p, _p, _i32, ctypes.c_uint64, _p,
                                       _sz, ctypes.POINTER(_i32), ctypes.POINTER(_f), _p]
        L.bsr_spmm.argtypes = [_i64, _i64, _i32, _i64, _p, _p, _p, _i32, _p, _i64, _f, _f, _p, _i64, _p, _sz, _p]
        for name in EXPORTS:
            if name not in ("sp_status_string", "sp_version"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(fn, code):
    if code != SP_OK:
        raise SparseError(fn, code, lib())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _dev(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise TypeError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise TypeError("%s must be contiguous" % name)
    return t


def status_string(code):
    return lib().sp_status_string(code).decode()


def sp_version():
    return lib().sp_version()


def _on(stream):
    """Allocation context: torch allocations inside it belong to `stream`."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _used_on(t, stream):
    """Marks a tensor allocated on another stream as in use on `stream`."""
    if stream is not None and t is not None:
        t.record_stream(stream)


# ---------------------------------------------------------------- conversions
def csr_build_from_coo(m, n, coo_row, coo_col, coo_val, stream=None):
    """COO (device int32/int32/float32, any order) -> (row_ptr, col_idx, val) on the device."""
    L = lib()
    _dev(coo_row, torch.int32, "coo_row"), _dev(coo_col, torch.int32, "coo_col"), _dev(coo_val, torch.float32, "coo_val")
    nnz = coo_row.numel()
    dev = coo_row.device
    size = _sz()
    _check("csr_build_from_coo_bufsize", L.csr_build_from_coo_bufsize(m, n, nnz, ctypes.byref(size)))
    with _on(stream):
        work = _workspace(size.value, dev)
        row_ptr = torch.empty(m + 1, dtype=torch.int32, device=dev)
        col_idx = torch.empty(nnz, dtype=torch.int32, device=dev)
        val = torch.empty(nnz, dtype=torch.float32, device=dev)
    _check("csr_build_from_coo",
           L.csr_build_from_coo(m, n, nnz, _ptr(coo_row), _ptr(coo_col), _ptr(coo_val), _ptr(row_ptr), _ptr(col_idx),
                                _ptr(val), _ptr(work), size.value, _stream(stream)))
    return row_ptr, col_idx, val


def csr_build_from_coo_noalloc(m, n, coo_row, coo_col, coo_val, stream=None):
    """COO -> CSR like csr_build_from_coo, the library's static per-GPU scratch
    instead of a workspace (the outputs are still allocated here)."""
    L = lib()
    _dev(coo_row, torch.int32, "coo_row"), _dev(coo_col, torch.int32, "coo_col"), _dev(coo_val, torch.float32, "coo_val")
    nnz = coo_row.numel()
    dev = coo_row.device
    with _on(stream):
        row_ptr = torch.empty(m + 1, dtype=torch.int32, device=dev)
        col_idx = torch.empty(nnz, dtype=torch.int32, device=dev)
        val = torch.empty(nnz, dtype=torch.float32, device=dev)
    _check("csr_build_from_coo_noalloc",
           L.csr_build_from_coo_noalloc(m, n, nnz, _ptr(coo_row), _ptr(coo_col), _ptr(coo_val), _ptr(row_ptr),
                                        _ptr(col_idx), _ptr(val), _stream(stream)))
    return row_ptr, col_idx, val


def csr_to_csc(m, n, row_ptr, col_idx, val, stream=None):
    """CSR of an m x n matrix -> (col_ptr, row_idx, cval), the CSR of its transpose."""
    L = lib()
    _dev(row_ptr, torch.int32, "row_ptr"), _dev(col_idx, torch.int32, "col_idx"), _dev(val, torch.float32, "val")
    nnz = col_idx.numel()
    dev = row_ptr.device
    size = _sz()
    _check("csr_to_csc_bufsize", L.csr_to_csc_bufsize(m, n, nnz, ctypes.byref(size)))
    with _on(stream):
        work = _workspace(size.value, dev)
        col_ptr = torch.empty(n + 1, dtype=torch.int32, device=dev)
        row_idx = torch.empty(nnz, dtype=torch.int32, device=dev)
        cval = torch.empty(nnz, dtype=torch.float32, device=dev)
    _check("csr_to_csc", L.csr_to_csc(m, n, nnz, _ptr(row_ptr), _ptr(col_idx), _ptr(val), _ptr(col_ptr),
                                      _ptr(row_idx), _ptr(cval), _ptr(work), size.value, _stream(stream)))
    return col_ptr, row_idx, cval


def csr_to_bsr(m, n, row_ptr, col_idx, val, bs, min_fill=0.0, out="f32", stream=None):
    """CSR (rows sorted by column) -> BSR with bs x bs blocks: (brow_ptr, bcol, blocks, fill).
    blocks is float32 [nnzb, bs, bs] (out="f32") or bf16 bit patterns as int16 (out="bf16").
    Raises SparseError with code SP_ERR_FILL when the fill ratio is below min_fill."""
    L = lib()
    _dev(row_ptr, torch.int32, "row_ptr"), _dev(col_idx, torch.int32, "col_idx"), _dev(val, torch.float32, "val")
    nnz = col_idx.numel()
    dev = row_ptr.device
    size = _sz()
    _check("csr_to_bsr_bufsize", L.csr_to_bsr_bufsize(m, n, nnz, bs, ctypes.byref(size)))
    mb = (m + bs - 1) // bs
    with _on(stream):
        work = _workspace(size.value, dev)
        brow_ptr = torch.empty(mb + 1, dtype=torch.int32, device=dev)
    nnzb, fill = _i64(), ctypes.c_double()
    _check("csr_to_bsr_analyze",
           L.csr_to_bsr_analyze(m, n, nnz, _ptr(row_ptr), _ptr(col_idx), bs, float(min_fill), _ptr(brow_ptr),
                                ctypes.byref(nnzb), ctypes.byref(fill), _ptr(work), size.value, _stream(stream)))
    with _on(stream):
        bcol = torch.empty(nnzb.value, dtype=torch.int32, device=dev)
        bval = torch.empty((nnzb.value, bs, bs), dtype=torch.int16 if out == "bf16" else torch.float32, device=dev)
    _check("csr_to_bsr_fill",
           L.csr_to_bsr_fill(m, n, nnz, _ptr(row_ptr), _ptr(col_idx), _ptr(val), bs, _ptr(brow_ptr), nnzb.value,
                             _ptr(bcol), _ptr(bval), 1 if out == "bf16" else 0, _stream(stream)))
    return brow_ptr, bcol, bval, fill.value


def csr_to_wcsr(m, n, row_ptr, col_idx, val, pad=8, stream=None):
    """CSR (rows sorted by column) -> windowed rows of 64: (window_ptr, window_col,
    values float32 [total_cols, 64], fill)."""
    L = lib()
    _dev(row_ptr, torch.int32, "row_ptr"), _dev(col_idx, torch.int32, "col_idx"), _dev(val, torch.float32, "val")
    nnz = col_idx.numel()
    dev = row_ptr.device
    size = _sz()
    _check("csr_to_wcsr_bufsize", L.csr_to_wcsr_bufsize(m, n, nnz, ctypes.byref(size)))
    with _on(stream):
        work = _workspace(size.value, dev)
        window_ptr = torch.empty((m + 63) // 64 + 1, dtype=torch.int32, device=dev)
    total, fill = _i64(), ctypes.c_double()
    _check("csr_to_wcsr_analyze",
           L.csr_to_wcsr_analyze(m, n, nnz, _ptr(row_ptr), _ptr(col_idx), int(pad), _ptr(window_ptr),
                                 ctypes.byref(total), ctypes.byref(fill), _ptr(work), size.value, _stream(stream)))
    with _on(stream):
        window_col = torch.empty(total.value, dtype=torch.int32, device=dev)
        values = torch.empty((total.value, 64), dtype=torch.float32, device=dev)
    _check("csr_to_wcsr_fill",
           L.csr_to_wcsr_fill(m, n, nnz, _ptr(row_ptr), _ptr(col_idx), _ptr(val), _ptr(window_ptr), total.value,
                              _ptr(window_col), _ptr(values), _stream(stream)))
    return window_ptr, window_col, values, fill.value


def wcsr_spmm(m, n, window_ptr, window_col, values, alpha, B, beta, C, stream=None):
    """C = alpha * A B + beta * C (in place on C) with A in windowed rows; B n x N, C m x N."""
    _dev(window_ptr, torch.int32, "window_ptr"), _dev(window_col, torch.int32, "window_col")
    _dev(values, torch.float32, "values"), _dev(B, torch.float32, "B"), _dev(C, torch.float32, "C")
    N = B.shape[1]
    if B.shape[0] != n or C.shape[0] != m or C.shape[1] != N:
        raise ValueError("shape mismatch")
    _check("wcsr_spmm", lib().wcsr_spmm(m, n, _ptr(window_ptr), _ptr(window_col), _ptr(values), N, float(alpha),
                                        _ptr(B), N, float(beta), _ptr(C), N, _stream(stream)))
    return C


class WcsrTasks:
    """Task table of a windowed matrix (windows of more than task_cols compressed
    columns cut into tasks of task_cols); built once, read-only afterwards."""

    def __init__(self, m, table, ntasks, nslots, task_cols):
        self.m, self.table, self.ntasks, self.nslots, self.task_cols = m, table, ntasks, nslots, task_cols

    def workspace_bytes(self, N):
        size = _sz()
        _check("wcsr_spmm_tasks_bufsize", lib().wcsr_spmm_tasks_bufsize(self.nslots, int(N), ctypes.byref(size)))
        return size.value


def wcsr_tasks(m, window_ptr, total_cols, task_cols=2048, stream=None):
    """Builds the task table of a WCSR matrix (synchronises once)."""
    L = lib()
    _dev(window_ptr, torch.int32, "window_ptr")
    size = _sz()
    _check("wcsr_tasks_bufsize", L.wcsr_tasks_bufsize(m, int(total_cols), int(task_cols), ctypes.byref(size)))
    with _on(stream):
        table = _workspace(size.value, window_ptr.device)
    ntasks, nslots = _i64(), _i64()
    _check("wcsr_tasks_build",
           L.wcsr_tasks_build(m, _ptr(window_ptr), int(total_cols), int(task_cols), _ptr(table), size.value,
                              ctypes.byref(ntasks), ctypes.byref(nslots), _stream(stream)))
    return WcsrTasks(m, table, ntasks.value, nslots.value, int(task_cols))


def wcsr_spmm_tasks(m, n, tasks, window_col, values, alpha, B, beta, C, work=None, stream=None):
    """C = alpha * A B + beta * C over a task table from wcsr_tasks; `work` is a uint8
    device tensor of at least tasks.workspace_bytes(N) bytes (allocated when None)."""
    _dev(window_col, torch.int32, "window_col"), _dev(values, torch.float32, "values")
    _dev(B, torch.float32, "B"), _dev(C, torch.float32, "C")
    N = B.shape[1]
    if B.shape[0] != n or C.shape[0] != m or C.shape[1] != N or tasks.m != m:
        raise ValueError("shape mismatch")
    need = tasks.workspace_bytes(N)
    if work is None:
        with _on(stream):
            work = _workspace(need, C.device)
    elif work.numel() * work.element_size() < need:
        raise ValueError("workspace of %d bytes, %d needed" % (work.numel() * work.element_size(), need))
    _check("wcsr_spmm_tasks",
           lib().wcsr_spmm_tasks(m, n, _ptr(tasks.table), tasks.ntasks, tasks.nslots, _ptr(window_col),
                                 _ptr(values), N, float(alpha), _ptr(B), N, float(beta), _ptr(C), N, _ptr(work),
                                 need, _stream(stream)))
    _used_on(tasks.table, stream)  # the table may have been allocated on another stream
    return C


# ---------------------------------------------------------------- plan
def plan_options(**kw):
    o = sp_plan_options()
    _check("sp_plan_options_default", lib().sp_plan_options_default(ctypes.byref(o)))
    for k, v in kw.items():
        if not hasattr(o, k):
            raise KeyError(k)
        setattr(o, k, int(v))
    return o


class Plan:
    """sp_plan of an m x n CSR matrix (and of its CSC when given), bound to a
    torch-allocated workspace.  Holds references to the arrays it points to."""

    def __init__(self, m, n, row_ptr, col_idx, val, csc=None, max_N=1, stream=None, tuned=False, **options):
        """tuned=True passes no options: the library uses the tuning cache's
        options for this matrix's dispatch key if it holds any, else the defaults."""
        L = lib()
        self._arrays = (row_ptr, col_idx, val) + (tuple(csc) if csc is not None else ())
        _dev(row_ptr, torch.int32, "row_ptr"), _dev(col_idx, torch.int32, "col_idx"), _dev(val, torch.float32, "val")
        cp, ri, cv = csc if csc is not None else (None, None, None)
        self.m, self.n, self.nnz = m, n, col_idx.numel()
        if tuned and options:
            raise ValueError("tuned=True takes no explicit options")
        self.opt = None if tuned else plan_options(**options)
        h = ctypes.c_void_p()
        _check("sp_plan_create",
               L.sp_plan_create(ctypes.byref(h), m, n, self.nnz, _ptr(row_ptr), _ptr(col_idx), _ptr(val),
                                _ptr(cp) if cp is not None else None, _ptr(ri) if ri is not None else None,
                                _ptr(cv) if cv is not None else None,
                                ctypes.byref(self.opt) if self.opt is not None else None, _stream(stream)))
        self.handle = h
        self.max_N = int(max_N)
        size = _sz()
        _check("sp_plan_workspace_size", L.sp_plan_workspace_size(h, self.max_N, ctypes.byref(size)))
        self.workspace_bytes = size.value
        self.stream = stream
        with _on(stream):
            self.work = _workspace(size.value, row_ptr.device)
        _check("sp_plan_bind", L.sp_plan_bind(h, _ptr(self.work), size.value, self.max_N, _stream(stream)))

    def view(self, max_N=None, stream=None):
        """A PlanView of this plan (its own per-call scratch; see PlanView)."""
        return PlanView(self, self.max_N if max_N is None else max_N, stream=stream)

    def dispatch_key(self, transposed=False, N=1, version=0):
        k = sp_dispatch_key()
        _check("sp_plan_dispatch_key", lib().sp_plan_dispatch_key(self.handle, 1 if transposed else 0, int(N),
                                                                  int(version), ctypes.byref(k)))
        return k

    def profile(self, transposed=False):
        p = sp_profile()
        _check("sp_plan_profile", lib().sp_plan_profile(self.handle, 1 if transposed else 0, ctypes.byref(p)))
        return {k: getattr(p, k) for k, _ in sp_profile._fields_}

    def destroy(self):
        """Frees the plan; SparseError (SP_ERR_STATE) while views of it are alive."""
        if self.handle is not None and self.handle.value:
            _check("sp_plan_destroy", lib().sp_plan_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


class PlanView:
    """sp_plan_view_create + sp_plan_bind: a handle that reads the bound tables of
    `plan` and owns only a per-call scratch (allocated here on `stream`), so that
    products on different views, or on the plan and its views, can run at the
    same time on different streams.  Accepted wherever a Plan is."""

    def __init__(self, plan, max_N=1, stream=None):
        L = lib()
        h = ctypes.c_void_p()
        _check("sp_plan_view_create", L.sp_plan_view_create(plan.handle, ctypes.byref(h)))
        self.handle = h
        self.base = plan  # keeps the plan (and its arrays) alive while the view exists
        self.m, self.n, self.nnz, self.max_N = plan.m, plan.n, plan.nnz, int(max_N)
        size = _sz()
        _check("sp_plan_workspace_size", L.sp_plan_workspace_size(h, self.max_N, ctypes.byref(size)))
        self.workspace_bytes = size.value
        self.stream = stream
        with _on(stream):
            self.work = _workspace(size.value, plan.work.device)
        _check("sp_plan_bind", L.sp_plan_bind(h, _ptr(self.work), size.value, self.max_N, _stream(stream)))

    def profile(self, transposed=False):
        return Plan.profile(self, transposed)

    def destroy(self):
        if self.handle is not None and self.handle.value:
            lib().sp_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def _plan_used_on(plan, stream):
    """The plan's (or view's) workspace, and a view's base workspace, are in use on `stream`."""
    if stream is None:
        return
    if plan.stream is not stream:
        _used_on(plan.work, stream)
    base = getattr(plan, "base", None)
    if base is not None and base.stream is not stream:
        _used_on(base.work, stream)


def sp_plan_create(m, n, row_ptr, col_idx, val, csc=None, max_N=1, **options):
    return Plan(m, n, row_ptr, col_idx, val, csc=csc, max_N=max_N, **options)


# ---------------------------------------------------------------- tuning cache, autotune
# The candidates timed by autotune_spmv when none are given: the row bins
# alone, SELL-C-sigma, the 8-panel stream, the x-window stream (2^15 columns).
DEFAULT_CANDIDATES = (dict(use_sell=0, col_panels=0, x_window_bits=0), dict(use_sell=1, col_panels=0, x_window_bits=0),
                      dict(use_sell=0, col_panels=8, x_window_bits=0), dict(use_sell=0, col_panels=0, x_window_bits=15))


def options_dict(o):
    return {k: getattr(o, k) for k, _ in sp_plan_options._fields_}


def tune_cache_store(key, **options):
    _check("sp_tune_cache_store", lib().sp_tune_cache_store(ctypes.byref(key), ctypes.byref(plan_options(**options))))


def tune_cache_lookup(key):
    """The cached options (dict) for key, or None."""
    o, found = sp_plan_options(), _i32()
    _check("sp_tune_cache_lookup", lib().sp_tune_cache_lookup(ctypes.byref(key), ctypes.byref(o), ctypes.byref(found)))
    return options_dict(o) if found.value else None


def tune_cache_clear():
    _check("sp_tune_cache_clear", lib().sp_tune_cache_clear())


def tune_cache_size():
    n = _i64()
    _check("sp_tune_cache_size", lib().sp_tune_cache_size(ctypes.byref(n)))
    return n.value


def autotune_spmv(m, n, row_ptr, col_idx, val, x, candidates=None, reps=20, version=0, stream=None):
    """Times spmv under each candidate option set (dicts of plan options), caches
    the fastest under the matrix's dispatch key; returns (best index, ms per call
    for each candidate, best options as a dict)."""
    L = lib()
    _dev(row_ptr, torch.int32, "row_ptr"), _dev(col_idx, torch.int32, "col_idx"), _dev(val, torch.float32, "val")
    _dev(x, torch.float32, "x")
    cands = list(candidates) if candidates is not None else list(DEFAULT_CANDIDATES)
    arr = (sp_plan_options * len(cands))(*[plan_options(**c) for c in cands])
    nnz = col_idx.numel()
    size = _sz()
    _check("sp_autotune_workspace_size",
           L.sp_autotune_workspace_size(m, n, nnz, _ptr(row_ptr), _ptr(col_idx), _ptr(val), arr, len(cands),
                                        ctypes.byref(size), _stream(stream)))
    with _on(stream):
        work = _workspace(size.value, row_ptr.device)
        y = torch.empty(m, dtype=torch.float32, device=row_ptr.device)
    best = _i32()
    ms = (_f * len(cands))()
    _check("sp_autotune_spmv",
           L.sp_autotune_spmv(m, n, nnz, _ptr(row_ptr), _ptr(col_idx), _ptr(val), arr, len(cands), _ptr(x), _ptr(y),
                              int(reps), int(version), _ptr(work), size.value, ctypes.byref(best), ms,
                              _stream(stream)))
    return best.value, list(ms), options_dict(arr[best.value])


# ---------------------------------------------------------------- products
def spmv(plan, alpha, x, beta, y, stream=None):
    """y = alpha * A x + beta * y (in place on y)."""
    _dev(x, torch.float32, "x"), _dev(y, torch.float32, "y")
    if x.numel() != plan.n or y.numel() != plan.m:
        raise ValueError("x must have n entries and y m entries")
    _plan_used_on(plan, stream)
    _check("spmv", lib().spmv(plan.handle, float(alpha), _ptr(x), float(beta), _ptr(y), _stream(stream)))
    return y


def spmv_t(plan, alpha, u, beta, z, stream=None):
    """z = alpha * A^T u + beta * z (in place on z), through the plan's CSC."""
    _dev(u, torch.float32, "u"), _dev(z, torch.float32, "z")
    if u.numel() != plan.m or z.numel() != plan.n:
        raise ValueError("u must have m entries and z n entries")
    _plan_used_on(plan, stream)
    _check("spmv_t", lib().spmv_t(plan.handle, float(alpha), _ptr(u), float(beta), _ptr(z), _stream(stream)))
    return z


def spmm(plan, alpha, B, beta, C, stream=None):
    """C = alpha * A B + beta * C (in place on C); B is n x N, C is m x N, row-major."""
    _dev(B, torch.float32, "B"), _dev(C, torch.float32, "C")
    N = B.shape[1]
    if B.shape[0] != plan.n or C.shape[0] != plan.m or C.shape[1] != N:
        raise ValueError("shape mismatch")
    _plan_used_on(plan, stream)
    _check("spmm", lib().spmm(plan.handle, N, float(alpha), _ptr(B), N, float(beta), _ptr(C), N, _stream(stream)))
    return C


def bsr_spmv(m, n, bs, brow_ptr, bcol, bval, alpha, x, beta, y, stream=None, rowwise=False):
    """y = alpha * A x + beta * y (in place on y) with A in BSR, fp32 bs x bs blocks.
    rowwise=True calls bsr_spmv_rowwise (one lane per element row) instead."""
    _dev(brow_ptr, torch.int32, "brow_ptr"), _dev(bcol, torch.int32, "bcol"), _dev(bval, torch.float32, "bval")
    _dev(x, torch.float32, "x"), _dev(y, torch.float32, "y")
    if x.numel() != n or y.numel() != m:
        raise ValueError("x must have n entries and y m entries")
    if bs > 0 and (brow_ptr.numel() != (m + bs - 1) // bs + 1 or bval.numel() != bcol.numel() * bs * bs):
        raise ValueError("brow_ptr must have ceil(m / bs) + 1 entries and bval nnzb * bs * bs")
    fn = "bsr_spmv_rowwise" if rowwise else "bsr_spmv"
    _check(fn, getattr(lib(), fn)(m, n, bs, bcol.numel(), _ptr(brow_ptr), _ptr(bcol), _ptr(bval), float(alpha),
                                  _ptr(x), float(beta), _ptr(y), _stream(stream)))
    return y


def bsr_spmm(mb, kb, bs, brow_ptr, bcol, bval, B, alpha, beta, C, stream=None, work=None):
    """C = alpha * A B + beta * C with A in BSR (bf16 blocks as int16/uint16 bits or bfloat16),
    B bf16 (kb*bs x N), C fp32 (mb*bs x N)."""
    L = lib()
    _dev(brow_ptr, torch.int32, "brow_ptr"), _dev(bcol, torch.int32, "bcol")
    for name, t in (("bval", bval), ("B", B)):
        if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
            raise TypeError("%s must hold bf16 bit patterns" % name)
        if not t.is_cuda or not t.is_contiguous():
            raise TypeError("%s must be a contiguous device tensor" % name)
    _dev(C, torch.float32, "C")
    nnzb = bcol.numel()
    N = B.shape[1]
    if (B.dim() != 2 or C.dim() != 2 or B.shape[0] != kb * bs or tuple(C.shape) != (mb * bs, N)
            or brow_ptr.numel() != mb + 1 or bval.numel() != nnzb * bs * bs):
        raise ValueError("shape mismatch: B must be (kb*bs, N), C (mb*bs, N), brow_ptr mb + 1, bval nnzb*bs*bs")
    size = _sz()
    _check("bsr_spmm_bufsize", L.bsr_spmm_bufsize(mb, kb, bs, nnzb, N, ctypes.byref(size)))
    if size.value > 0 and work is None:
        with _on(stream):
            work = _workspace(size.value, C.device)
    wbytes = size.value if work is not None else 0
    _check("bsr_spmm", L.bsr_spmm(mb, kb, bs, nnzb, _ptr(brow_ptr), _ptr(bcol), _ptr(bval), N, _ptr(B), N,
                                  float(alpha), float(beta), _ptr(C), N, _ptr(work) if work is not None else None,
                                  wbytes, _stream(stream)))
    return C
