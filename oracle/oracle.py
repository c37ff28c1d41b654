"""numpy marshalling for the C oracle (test infrastructure only).

Each wrapper allocates its outputs with numpy and calls the function of the
same name in ``oracle.c``; no arithmetic of the method is done here.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


class OracleError(RuntimeError):
    pass


def library_path():
    return _LIB


def build(force=True):
    """Compile oracle.c with gcc into liboracle.so next to it."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_d = ctypes.c_double


def _declare(lib):
    lib.oracle_coo_to_csr.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _p, _p]
    lib.oracle_coo_to_csr.restype = ctypes.c_int
    lib.oracle_csr_to_csc.argtypes = [_i64, _i64, _p, _p, _p, _p, _p, _p]
    lib.oracle_csr_to_csc.restype = ctypes.c_int
    lib.oracle_spmv.argtypes = [_i64, _p, _p, _p, _p, _d, _d, _p, _p, _i64, _p, _p]
    lib.oracle_spmv.restype = None
    lib.oracle_spmv_t_scatter.argtypes = [_i64, _i64, _p, _p, _p, _p, _d, _d, _p, _p, _p]
    lib.oracle_spmv_t_scatter.restype = None
    lib.oracle_spmm.argtypes = [_i64, _p, _p, _p, _i64, _p, _i64, _d, _d, _p, _i64, _p, _i64, _p, _p]
    lib.oracle_spmm.restype = None
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = _d
    lib.oracle_bsr_to_csr.argtypes = [_i64, _i64, _p, _p, _p, _p, _p, _p]
    lib.oracle_bsr_to_csr.restype = ctypes.c_int
    lib.oracle_spmm_bf16.argtypes = [_i64, _p, _p, _p, _i64, _p, _i64, _d, _d, _p, _i64, _p, _i64, _p, _p]
    lib.oracle_spmm_bf16.restype = None
    lib.oracle_bsr_spmm_direct.argtypes = [_i64, _i64, _p, _p, _p, _i64, _p, _i64, _d, _d, _p, _i64, _p,
                                           _i64, _p]
    lib.oracle_bsr_spmm_direct.restype = None
    lib.oracle_csr_to_bsr_count.argtypes = [_i64, _i64, _p, _p, _i64, _p]
    lib.oracle_csr_to_bsr_count.restype = _i64
    lib.oracle_csr_to_bsr_fill.argtypes = [_i64, _p, _p, _p, _i64, _p, _p, _p]
    lib.oracle_csr_to_bsr_fill.restype = None
    lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.oracle_bsr_spmv.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _d, _d, _p, _p, _p]
    lib.oracle_bsr_spmv.restype = None
    lib.oracle_csr_to_wcsr_count.argtypes = [_i64, _i64, _p, _p, _i64, _i64, _p]
    lib.oracle_csr_to_wcsr_count.restype = _i64
    lib.oracle_csr_to_wcsr_fill.argtypes = [_i64, _p, _p, _p, _i64, _p, _p, _p]
    lib.oracle_csr_to_wcsr_fill.restype = None
    lib.oracle_wcsr_tasks.argtypes = [_i64, _p, _i64, _p, _p, ctypes.POINTER(_i64)]
    lib.oracle_wcsr_tasks.restype = _i64
    lib.oracle_wcsr_spmm.argtypes = [_i64, _i64, _p, _p, _p, _i64, _p, _i64, _d, _d, _p, _i64, _p, _p]
    lib.oracle_wcsr_spmm.restype = None
    lib.oracle_row_profile.argtypes = [_i64, _p, _p]
    lib.oracle_row_profile.restype = None
    lib.oracle_sell_build.argtypes = [_i64, _p, _p, _p, _i64, _i64, _p, _p, _p, _p, _p]
    lib.oracle_sell_build.restype = _i64
    lib.oracle_sell_spmv.argtypes = [_i64, _i64, _p, _p, _p, _p, _p, _p, _d, _p]
    lib.oracle_sell_spmv.restype = None


def _c(a, dtype):
    """Contiguous array of the given dtype (a copy only when needed)."""
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _rows(rows):
    if rows is None:
        return None, 0
    r = _c(rows, np.int64)
    return r, r.size


def coo_to_csr(m, n, row, col, val):
    """COO (any order) -> CSR (row_ptr int32[m+1], col int32[nnz], val float32[nnz])."""
    lib = _load()
    row, col, val = _c(row, np.int32), _c(col, np.int32), _c(val, np.float32)
    nnz = row.size
    if col.size != nnz or val.size != nnz:
        raise OracleError("COO arrays differ in length")
    row_ptr = np.empty(m + 1, np.int32)
    col_out = np.empty(nnz, np.int32)
    val_out = np.empty(nnz, np.float32)
    rc = lib.oracle_coo_to_csr(m, n, nnz, _ptr(row), _ptr(col), _ptr(val), _ptr(row_ptr), _ptr(col_out),
                               _ptr(val_out))
    if rc != 0:
        raise OracleError("oracle_coo_to_csr failed with code %d" % rc)
    return row_ptr, col_out, val_out


def csr_to_csc(m, n, row_ptr, col, val):
    """CSR (m x n) -> CSC = CSR of the transpose (col_ptr[n+1], row_idx[nnz], val[nnz])."""
    lib = _load()
    row_ptr, col, val = _c(row_ptr, np.int32), _c(col, np.int32), _c(val, np.float32)
    nnz = int(row_ptr[m])
    col_ptr = np.empty(n + 1, np.int32)
    row_idx = np.empty(nnz, np.int32)
    val_out = np.empty(nnz, np.float32)
    rc = lib.oracle_csr_to_csc(m, n, _ptr(row_ptr), _ptr(col), _ptr(val), _ptr(col_ptr), _ptr(row_idx),
                               _ptr(val_out))
    if rc != 0:
        raise OracleError("oracle_csr_to_csc failed with code %d" % rc)
    return col_ptr, row_idx, val_out


def spmv(row_ptr, col, val, x, alpha=1.0, beta=0.0, y=None, rows=None):
    """fp64 y = alpha*A*x + beta*y for all rows (or the listed rows); returns (y, scale)."""
    lib = _load()
    m = row_ptr.size - 1
    row_ptr, col, val, x = _c(row_ptr, np.int32), _c(col, np.int32), _c(val, np.float32), _c(x, np.float32)
    y_in = _c(y, np.float32) if (beta != 0.0) else None
    r, nr = _rows(rows)
    cnt = nr if rows is not None else m
    out = np.empty(cnt, np.float64)
    scale = np.empty(cnt, np.float64)
    lib.oracle_spmv(m, _ptr(row_ptr), _ptr(col), _ptr(val), _ptr(x), float(alpha), float(beta), _ptr(y_in),
                    _ptr(r), nr, _ptr(out), _ptr(scale))
    return out, scale


def spmv_t_scatter(m, n, row_ptr, col, val, u, alpha=1.0, beta=0.0, z=None):
    """fp64 z = alpha*A^T*u + beta*z by scattering CSR entries (independent route)."""
    lib = _load()
    row_ptr, col, val, u = _c(row_ptr, np.int32), _c(col, np.int32), _c(val, np.float32), _c(u, np.float32)
    z_in = _c(z, np.float32) if beta != 0.0 else None
    out = np.empty(n, np.float64)
    scale = np.empty(n, np.float64)
    lib.oracle_spmv_t_scatter(m, n, _ptr(row_ptr), _ptr(col), _ptr(val), _ptr(u), float(alpha), float(beta),
                              _ptr(z_in), _ptr(out), _ptr(scale))
    return out, scale


def spmm(row_ptr, col, val, B, alpha=1.0, beta=0.0, C=None, rows=None):
    """fp64 C = alpha*A*B + beta*C (B K x N row-major); returns (C rows, scale) as [rows, N]."""
    lib = _load()
    m = row_ptr.size - 1
    row_ptr, col, val = _c(row_ptr, np.int32), _c(col, np.int32), _c(val, np.float32)
    B = _c(B, np.float32)
    N = B.shape[1]
    C_in = _c(C, np.float32) if beta != 0.0 else None
    r, nr = _rows(rows)
    cnt = nr if rows is not None else m
    out = np.empty((cnt, N), np.float64)
    scale = np.empty((cnt, N), np.float64)
    lib.oracle_spmm(m, _ptr(row_ptr), _ptr(col), _ptr(val), N, _ptr(B), N, float(alpha), float(beta),
                    _ptr(C_in), N, _ptr(r), nr, _ptr(out), _ptr(scale))
    return out, scale


def bf16_to_float64(h):
    """Exact bf16 (uint16 bit patterns) -> float64, element by element through the C oracle."""
    lib = _load()
    h = np.asarray(h, dtype=np.uint16)
    flat = h.ravel()
    out = np.fromiter((lib.oracle_bf16_to_double(int(v)) for v in flat), dtype=np.float64, count=flat.size)
    return out.reshape(h.shape)


def bsr_to_csr(mb, bs, brow_ptr, bcol, bval):
    """Expand BSR (row-major bf16 blocks) to CSR with fp64 values, zeros kept."""
    lib = _load()
    brow_ptr, bcol = _c(brow_ptr, np.int32), _c(bcol, np.int32)
    bval = _c(bval, np.uint16)
    nnzb = int(brow_ptr[mb])
    nnz = nnzb * bs * bs
    row_ptr = np.empty(mb * bs + 1, np.int32)
    col = np.empty(nnz, np.int32)
    val = np.empty(nnz, np.float64)
    lib.oracle_bsr_to_csr(mb, bs, _ptr(brow_ptr), _ptr(bcol), _ptr(bval), _ptr(row_ptr), _ptr(col), _ptr(val))
    return row_ptr, col, val


def spmm_bf16(row_ptr, col, val64, B, alpha=1.0, beta=0.0, C=None, rows=None):
    """fp64 SpMM over a CSR with fp64 values and a bf16 (uint16) right-hand side."""
    lib = _load()
    m = row_ptr.size - 1
    row_ptr, col, val64 = _c(row_ptr, np.int32), _c(col, np.int32), _c(val64, np.float64)
    B = _c(B, np.uint16)
    N = B.shape[1]
    C_in = _c(C, np.float32) if beta != 0.0 else None
    r, nr = _rows(rows)
    cnt = nr if rows is not None else m
    out = np.empty((cnt, N), np.float64)
    scale = np.empty((cnt, N), np.float64)
    lib.oracle_spmm_bf16(m, _ptr(row_ptr), _ptr(col), _ptr(val64), N, _ptr(B), N, float(alpha), float(beta),
                         _ptr(C_in), N, _ptr(r), nr, _ptr(out), _ptr(scale))
    return out, scale


def bsr_spmm_direct(mb, bs, brow_ptr, bcol, bval, B, alpha=1.0, beta=0.0, C=None, rows=None):
    """fp64 BSR SpMM by a direct block loop (second route)."""
    lib = _load()
    brow_ptr, bcol, bval = _c(brow_ptr, np.int32), _c(bcol, np.int32), _c(bval, np.uint16)
    B = _c(B, np.uint16)
    N = B.shape[1]
    C_in = _c(C, np.float32) if beta != 0.0 else None
    r, nr = _rows(rows)
    cnt = nr if rows is not None else mb * bs
    out = np.empty((cnt, N), np.float64)
    lib.oracle_bsr_spmm_direct(mb, bs, _ptr(brow_ptr), _ptr(bcol), _ptr(bval), N, _ptr(B), N, float(alpha),
                               float(beta), _ptr(C_in), N, _ptr(r), nr, _ptr(out))
    return out


def csr_to_bsr(m, n, row_ptr, col, val, bs, out="f32"):
    """CSR -> BSR with bs x bs blocks: (brow_ptr int32[mb+1], bcol int32[nnzb],
    blocks float32[nnzb, bs, bs] (out="f32") or their bf16 bit patterns
    uint16[nnzb, bs, bs] (out="bf16"))."""
    lib = _load()
    row_ptr, col, val = _c(row_ptr, np.int32), _c(col, np.int32), _c(val, np.float32)
    mb = (m + bs - 1) // bs
    brow_ptr = np.empty(mb + 1, np.int32)
    nnzb = lib.oracle_csr_to_bsr_count(m, n, _ptr(row_ptr), _ptr(col), bs, _ptr(brow_ptr))
    bcol = np.empty(nnzb, np.int32)
    bval = np.empty((nnzb, bs, bs), np.float32)
    lib.oracle_csr_to_bsr_fill(m, _ptr(row_ptr), _ptr(col), _ptr(val), bs, _ptr(brow_ptr), _ptr(bcol), _ptr(bval))
    if out == "bf16":
        bval = f32_to_bf16(bval)
    return brow_ptr, bcol, bval


def f32_to_bf16(a):
    """float32 -> bf16 bit patterns (uint16), element by element through the C oracle."""
    lib = _load()
    a = np.asarray(a, dtype=np.float32)
    flat = a.ravel()
    out = np.fromiter((lib.oracle_f32_to_bf16(float(v)) for v in flat), dtype=np.uint16, count=flat.size)
    return out.reshape(a.shape)


def bsr_spmv(m, n, bs, brow_ptr, bcol, bval, x, alpha=1.0, beta=0.0, y=None):
    """fp64 BSR SpMV with fp32 blocks over element rows < m and columns < n: (y, scale)."""
    lib = _load()
    brow_ptr, bcol, bval = _c(brow_ptr, np.int32), _c(bcol, np.int32), _c(bval, np.float32)
    x = _c(x, np.float32)
    y_in = _c(y, np.float32) if beta != 0.0 else None
    out = np.empty(m, np.float64)
    scale = np.empty(m, np.float64)
    lib.oracle_bsr_spmv(m, n, bs, _ptr(brow_ptr), _ptr(bcol), _ptr(bval), _ptr(x), float(alpha), float(beta),
                        _ptr(y_in), _ptr(out), _ptr(scale))
    return out, scale


def csr_to_wcsr(m, n, row_ptr, col, val, H, pad):
    """CSR -> WCSR with windows of H rows: (window_ptr int32[nw+1], window_col int32[total]
    (-1 = padding), values float32[total, H] (compressed column major))."""
    lib = _load()
    row_ptr, col, val = _c(row_ptr, np.int32), _c(col, np.int32), _c(val, np.float32)
    nw = (m + H - 1) // H
    window_ptr = np.empty(nw + 1, np.int32)
    total = lib.oracle_csr_to_wcsr_count(m, n, _ptr(row_ptr), _ptr(col), H, pad, _ptr(window_ptr))
    window_col = np.empty(total, np.int32)
    values = np.empty((total, H), np.float32)
    lib.oracle_csr_to_wcsr_fill(m, _ptr(row_ptr), _ptr(col), _ptr(val), H, _ptr(window_ptr), _ptr(window_col),
                                _ptr(values))
    return window_ptr, window_col, values


def wcsr_tasks(window_ptr, task_cols):
    """Task split of the windows: (tasks int32[T, 4] = {window, first column, end
    column, slot or -1}, winfo int32[nw, 2] = {first slot or -1, tasks}, slots)."""
    lib = _load()
    window_ptr = _c(window_ptr, np.int32)
    nw = window_ptr.size - 1
    slots = ctypes.c_int64()
    T = lib.oracle_wcsr_tasks(nw, _ptr(window_ptr), int(task_cols), None, None, ctypes.byref(slots))
    tasks = np.empty((T, 4), np.int32)
    winfo = np.empty((nw, 2), np.int32)
    lib.oracle_wcsr_tasks(nw, _ptr(window_ptr), int(task_cols), _ptr(tasks), _ptr(winfo), ctypes.byref(slots))
    return tasks, winfo, slots.value


def wcsr_spmm(m, H, window_ptr, window_col, values, B, alpha=1.0, beta=0.0, C=None):
    """fp64 SpMM over the WCSR layout: (C, scale)."""
    lib = _load()
    window_ptr, window_col, values = _c(window_ptr, np.int32), _c(window_col, np.int32), _c(values, np.float32)
    B = _c(B, np.float32)
    N = B.shape[1]
    C_in = _c(C, np.float32) if beta != 0.0 else None
    out = np.empty((m, N), np.float64)
    scale = np.empty((m, N), np.float64)
    lib.oracle_wcsr_spmm(m, H, _ptr(window_ptr), _ptr(window_col), _ptr(values), N, _ptr(B), N, float(alpha),
                         float(beta), _ptr(C_in), N, _ptr(out), _ptr(scale))
    return out, scale


def row_profile(row_ptr):
    """Row-length profile: dict(mean, var, cv, p95, p99, max, empty)."""
    lib = _load()
    row_ptr = _c(row_ptr, np.int32)
    out = np.zeros(7, np.float64)
    lib.oracle_row_profile(row_ptr.size - 1, _ptr(row_ptr), _ptr(out))
    keys = ("mean", "var", "cv", "p95", "p99", "max", "empty")
    return {k: (float(v) if i < 3 else int(v)) for i, (k, v) in enumerate(zip(keys, out))}


def sell_build(row_ptr, col, val, C, sigma):
    """SELL-C-sigma layout: dict(perm, slice_ptr, slice_len, col, val, slots)."""
    lib = _load()
    m = row_ptr.size - 1
    row_ptr, col, val = _c(row_ptr, np.int32), _c(col, np.int32), _c(val, np.float32)
    nslices = (m + C - 1) // C
    perm = np.empty(m, np.int32)
    slice_ptr = np.empty(nslices + 1, np.int64)
    slice_len = np.empty(m, np.int32)
    slots = lib.oracle_sell_build(m, _ptr(row_ptr), _ptr(col), _ptr(val), C, sigma, _ptr(perm), _ptr(slice_ptr),
                                  _ptr(slice_len), None, None)
    col_out = np.empty(max(slots, 1), np.int32)
    val_out = np.empty(max(slots, 1), np.float32)
    lib.oracle_sell_build(m, _ptr(row_ptr), _ptr(col), _ptr(val), C, sigma, _ptr(perm), _ptr(slice_ptr),
                          _ptr(slice_len), _ptr(col_out), _ptr(val_out))
    return dict(perm=perm, slice_ptr=slice_ptr, slice_len=slice_len, col=col_out[:slots], val=val_out[:slots],
                slots=int(slots))


def sell_spmv(sell, C, x, alpha=1.0):
    """fp64 y = alpha*A*x through a SELL layout produced by sell_build."""
    lib = _load()
    m = sell["perm"].size
    x = _c(x, np.float32)
    y = np.empty(m, np.float64)
    col = _c(sell["col"], np.int32)
    val = _c(sell["val"], np.float32)
    lib.oracle_sell_spmv(m, C, _ptr(sell["perm"]), _ptr(sell["slice_ptr"]), _ptr(sell["slice_len"]), _ptr(col),
                         _ptr(val), _ptr(x), float(alpha), _ptr(y))
    return y
