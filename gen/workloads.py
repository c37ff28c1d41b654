"""Workload recipes.  See the package docstring: random draws only.

Each function documents the distribution it draws.  The five named workloads
(`CONFIGS`) are:

  spmv_uniform    4096 x 4096, row lengths uniform in [1, 16], distinct sorted
                  columns, values in U[-1, 1]; delivered as shuffled COO.
  spmv_powerlaw   2^22 x 2^22, row lengths floor(exp(1.6 + 1.3 Z)) clipped to
                  200000 plus four planted hub rows of 60k/100k/150k/200k
                  entries; columns uniform with replacement, then sorted and
                  de-duplicated; values in U[-1, 1].
  stencil27       27-point stencil on a 160^3 grid (rows r = (i*160+j)*160+k,
                  neighbours in lexicographic (di, dj, dk) order, truncated at
                  the faces), values N(0, 1).
  spmm_lognormal  2^20 x 2^20, row lengths floor(exp(2.5 + Z)), distinct sorted
                  uniform columns, values U[-1, 1]; dense B is K x N, U[-1, 1].
  bsr_blocks      16384 x 16384 in 64 x 64 blocks, 10 % of the 256 x 256 block
                  positions (6554) drawn without replacement, every block dense
                  with N(0, 0.02) values rounded to bf16; B is 16384 x 512 bf16
                  drawn N(0, 1).
  spmm_clustered  2^20 x 2^20, rows in windows of 64 that draw their columns
                  from a per-window pool of 128 distinct uniform columns, row
                  lengths floor(exp(2.5 + Z)) clipped to 128, values U[-1, 1]
                  (the workload of the windowed SpMM); B as spmm_lognormal.
  bsr_spmv        the bsr_blocks block positions as an fp32 COO (every element
                  of every block, N(0, 0.02)), converted on the GPU to 64 x 64
                  BSR; x in U[-1, 1].
"""
from dataclasses import dataclass

import numpy as np


@dataclass
class Coo:
    m: int
    n: int
    row: np.ndarray  # int32
    col: np.ndarray  # int32
    val: np.ndarray  # float32

    @property
    def nnz(self):
        return int(self.row.size)


@dataclass
class Bsr:
    mb: int          # block rows
    kb: int          # block columns
    bs: int          # block edge
    brow_ptr: np.ndarray  # int32 [mb + 1]
    bcol: np.ndarray      # int32 [nnzb]
    bval: np.ndarray      # uint16 bf16 bits [nnzb, bs, bs], row-major blocks

    @property
    def nnzb(self):
        return int(self.bcol.size)


def _rng(seed, stream=0):
    # One independent PCG64 stream per (seed, stream) pair.
    return np.random.Generator(np.random.PCG64([int(seed), int(stream)]))


def f32_to_bf16_bits(a):
    """Round float32 to bf16 with round-to-nearest-even on the bit pattern.

    Inputs must be finite (the generators never draw inf/NaN).
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def dense_vector(n, seed, stream=1, low=-1.0, high=1.0):
    """float32 vector with entries U[low, high)."""
    return _rng(seed, stream).uniform(low, high, size=n).astype(np.float32)


def dense_matrix(rows, cols, seed, stream=2, low=-1.0, high=1.0):
    """float32 row-major matrix with entries U[low, high)."""
    return _rng(seed, stream).uniform(low, high, size=(rows, cols)).astype(np.float32)


def shuffle_coo(coo, seed, stream=9):
    """The same triples in a seeded random order."""
    p = _rng(seed, stream).permutation(coo.nnz)
    return Coo(coo.m, coo.n, coo.row[p].copy(), coo.col[p].copy(), coo.val[p].copy())


def _triples_from_lengths(rng, m, n, lens, distinct, chunk_rows=1 << 20):
    """Row-major triples: row i gets lens[i] uniform columns in [0, n).

    distinct=True draws until every row's columns are distinct (re-drawing the
    rows that had a collision); distinct=False draws with replacement and then
    drops repeated columns (so rows can come out shorter).  Columns of a row are
    returned in increasing order.  Done in chunks of rows to bound memory.
    """
    rows_out, cols_out = [], []
    lens = np.asarray(lens, dtype=np.int64)
    for r0 in range(0, m, chunk_rows):
        r1 = min(m, r0 + chunk_rows)
        ln = lens[r0:r1].copy()
        # Rows long enough that a with-replacement draw of them usually repeats a
        # column (l^2 > n/4, the birthday bound) are drawn exactly without
        # replacement one by one; rejection would rarely succeed for them.
        dense_rows = np.flatnonzero(ln * ln * 4 > n) + r0 if distinct else np.empty(0, np.int64)
        ln[dense_rows - r0] = 0
        rows = np.repeat(np.arange(r0, r1, dtype=np.int64), ln)
        cols = rng.integers(0, n, size=rows.size, dtype=np.int64)
        key = rows * n + cols
        if dense_rows.size:
            extra = [r * n + rng.choice(n, size=int(lens[r]), replace=False).astype(np.int64) for r in dense_rows]
            key = np.concatenate([key] + extra)
        key.sort()
        if distinct:
            for _ in range(1000):
                dup = np.flatnonzero(key[1:] == key[:-1]) + 1
                if dup.size == 0:
                    break
                bad_rows = np.unique(key[dup] // n)
                keep = ~np.isin(key // n, bad_rows)
                key = key[keep]
                redraw_len = lens[bad_rows].astype(np.int64)
                rr = np.repeat(bad_rows, redraw_len)
                cc = rng.integers(0, n, size=rr.size, dtype=np.int64)
                key = np.concatenate([key, rr * n + cc])
                key.sort()
            else:
                raise RuntimeError("distinct column draw did not converge")
        else:
            if key.size:
                key = key[np.concatenate(([True], key[1:] != key[:-1]))]
        rows_out.append((key // n).astype(np.int32))
        cols_out.append((key % n).astype(np.int32))
    return np.concatenate(rows_out), np.concatenate(cols_out)


def uniform_rows_coo(m=4096, n=4096, lmin=1, lmax=16, seed=0, shuffled=True):
    """Row lengths uniform in [lmin, lmax], distinct sorted columns, values U[-1,1]."""
    rng = _rng(seed, 10)
    lens = rng.integers(lmin, lmax + 1, size=m)
    row, col = _triples_from_lengths(rng, m, n, lens, distinct=True)
    val = rng.uniform(-1.0, 1.0, size=row.size).astype(np.float32)
    coo = Coo(m, n, row, col, val)
    return shuffle_coo(coo, seed) if shuffled else coo


def powerlaw_coo(m=1 << 22, n=1 << 22, mu=1.6, sigma=1.3, clip=200000,
                 hubs=(60000, 100000, 150000, 200000), seed=0, shuffled=False):
    """Lognormal row lengths floor(exp(mu + sigma Z)) clipped to `clip`, plus
    planted hub rows at seeded positions; columns uniform with replacement,
    sorted and de-duplicated; values U[-1, 1]."""
    rng = _rng(seed, 20)
    z = rng.standard_normal(m)
    lens = np.minimum(clip, np.floor(np.exp(mu + sigma * z))).astype(np.int64)
    hubs = [h for h in hubs if h <= n]
    if hubs:
        pos = rng.choice(m, size=len(hubs), replace=False)
        lens[pos] = hubs
    row, col = _triples_from_lengths(rng, m, n, lens, distinct=False)
    val = rng.uniform(-1.0, 1.0, size=row.size).astype(np.float32)
    coo = Coo(m, n, row, col, val)
    return shuffle_coo(coo, seed) if shuffled else coo


def stencil27_coo(g=160, seed=0, shuffled=False):
    """27-point stencil on a g^3 grid; values N(0, 1) (so A != A^T)."""
    m = g * g * g
    r = np.arange(m, dtype=np.int64)
    i, j, k = r // (g * g), (r // g) % g, r % g
    cols = np.full((m, 27), -1, dtype=np.int64)
    t = 0
    for di in (-1, 0, 1):
        for dj in (-1, 0, 1):
            for dk in (-1, 0, 1):
                ok = (i + di >= 0) & (i + di < g) & (j + dj >= 0) & (j + dj < g) & (k + dk >= 0) & (k + dk < g)
                cols[:, t] = np.where(ok, r + (di * g + dj) * g + dk, -1)
                t += 1
    rows = np.repeat(np.arange(m, dtype=np.int32), 27).reshape(m, 27)
    keep = cols >= 0
    row = rows[keep]
    col = cols[keep].astype(np.int32)
    del cols, rows, keep
    val = _rng(seed, 30).standard_normal(row.size, dtype=np.float32)
    coo = Coo(m, m, row, col, val)
    return shuffle_coo(coo, seed) if shuffled else coo


def lognormal_coo(m=1 << 20, n=1 << 20, mu=2.5, sigma=1.0, seed=0, shuffled=False):
    """Row lengths floor(exp(mu + sigma Z)), distinct sorted uniform columns, values U[-1,1]."""
    rng = _rng(seed, 40)
    z = rng.standard_normal(m)
    lens = np.minimum(n, np.floor(np.exp(mu + sigma * z))).astype(np.int64)
    row, col = _triples_from_lengths(rng, m, n, lens, distinct=True)
    val = rng.uniform(-1.0, 1.0, size=row.size).astype(np.float32)
    coo = Coo(m, n, row, col, val)
    return shuffle_coo(coo, seed) if shuffled else coo


def block_sparse_bsr(mb=256, kb=256, bs=64, density=0.1, std=0.02, seed=0):
    """round(density*mb*kb) block positions without replacement, sorted by
    (block row, block column); dense blocks with N(0, std) values as bf16."""
    rng = _rng(seed, 50)
    nblocks = int(round(density * mb * kb))
    pos = np.sort(rng.choice(mb * kb, size=nblocks, replace=False))
    brow = (pos // kb).astype(np.int64)
    bcol = (pos % kb).astype(np.int32)
    counts = np.bincount(brow, minlength=mb)
    brow_ptr = np.zeros(mb + 1, np.int64)
    brow_ptr[1:] = np.cumsum(counts)
    vals = rng.normal(0.0, std, size=(nblocks, bs, bs)).astype(np.float32)
    return Bsr(mb, kb, bs, brow_ptr.astype(np.int32), bcol, f32_to_bf16_bits(vals).reshape(nblocks, bs, bs))


def block_sparse_coo(mb=256, kb=256, bs=64, density=0.1, std=0.02, seed=0):
    """The block positions of block_sparse_bsr (same draw), every element of
    every block present, values N(0, std) in fp32; COO ordered by block, then
    row-major inside the block."""
    rng = _rng(seed, 50)
    nblocks = int(round(density * mb * kb))
    pos = np.sort(rng.choice(mb * kb, size=nblocks, replace=False))
    brow = (pos // kb).astype(np.int64)
    bcol = (pos % kb).astype(np.int64)
    r_in = np.repeat(np.arange(bs, dtype=np.int64), bs)
    c_in = np.tile(np.arange(bs, dtype=np.int64), bs)
    row = (brow[:, None] * bs + r_in[None, :]).reshape(-1).astype(np.int32)
    col = (bcol[:, None] * bs + c_in[None, :]).reshape(-1).astype(np.int32)
    val = _rng(seed, 52).normal(0.0, std, size=row.size).astype(np.float32)
    return Coo(mb * bs, kb * bs, row, col, val)


def clustered_coo(m=1 << 20, n=1 << 20, H=64, pool=128, mu=2.5, sigma=1.0, seed=0, batch=1 << 14):
    """Rows in windows of H; window w draws a pool of `pool` distinct columns
    uniformly from [0, n); a row's length is floor(exp(mu + sigma Z)) clipped
    to [0, pool] (the lognormal of spmm_lognormal) and its columns are that
    many distinct members of its window's pool; values U[-1, 1]."""
    rng = _rng(seed, 70)
    nw = (m + H - 1) // H
    lens = np.minimum(np.floor(np.exp(mu + sigma * rng.standard_normal(m))), pool).astype(np.int64)
    rows, cols = [], []
    for r0 in range(0, m, batch):
        r1 = min(m, r0 + batch)
        w0, w1 = r0 // H, (r1 + H - 1) // H
        pools = np.sort(np.stack([rng.choice(n, size=pool, replace=False) for _ in range(w0, w1)]), axis=1)
        keys = rng.random((r1 - r0, pool), dtype=np.float32)
        pick = np.argsort(keys, axis=1)                       # a random order of the pool per row
        take = np.arange(pool)[None, :] < lens[r0:r1, None]   # the first l of it
        rr = np.broadcast_to(np.arange(r0, r1)[:, None], pick.shape)[take]
        cc = pools[(rr // H) - w0, pick[take]]
        rows.append(rr.astype(np.int32))
        cols.append(cc.astype(np.int32))
    row = np.concatenate(rows) if rows else np.zeros(0, np.int32)
    col = np.concatenate(cols) if cols else np.zeros(0, np.int32)
    val = _rng(seed, 71).uniform(-1.0, 1.0, size=row.size).astype(np.float32)
    return Coo(m, n, row, col, val)


def skewed_windows_coo(m=1 << 20, n=1 << 20, H=64, pool_median=64, pool_sigma=1.5, pool_max=16384,
                       frac=(0.05, 0.3), seed=0):
    """Windows of H rows whose column pools vary widely in size: window w
    draws P_w = floor(pool_median * exp(pool_sigma Z)) clipped to [1,
    pool_max] columns uniformly from [0, n) (with replacement, duplicates
    dropped, so at most P_w distinct); every row of the window draws a rate
    f in U[frac) and keeps each pool column with probability f; values
    U[-1, 1].  Rows come out sorted by column."""
    rng = _rng(seed, 80)
    nw = (m + H - 1) // H
    sizes = np.clip(np.floor(pool_median * np.exp(pool_sigma * rng.standard_normal(nw))), 1, pool_max)
    rows, cols = [], []
    for w in range(nw):
        r0, r1 = w * H, min(m, w * H + H)
        pool = np.unique(rng.integers(0, n, size=int(sizes[w])))
        f = rng.uniform(frac[0], frac[1], size=r1 - r0)
        keep = rng.random((r1 - r0, pool.size)) < f[:, None]
        rr, pp = np.nonzero(keep)
        rows.append((rr + r0).astype(np.int32))
        cols.append(pool[pp].astype(np.int32))
    row = np.concatenate(rows) if rows else np.zeros(0, np.int32)
    col = np.concatenate(cols) if cols else np.zeros(0, np.int32)
    val = _rng(seed, 81).uniform(-1.0, 1.0, size=row.size).astype(np.float32)
    return Coo(m, n, row, col, val)


def bf16_matrix(rows, cols, seed, stream=51, std=1.0):
    """bf16 (uint16 bits) matrix with N(0, std) entries."""
    a = _rng(seed, stream).normal(0.0, std, size=(rows, cols)).astype(np.float32)
    return f32_to_bf16_bits(a).reshape(rows, cols)


def ragged_coo(m, n, seed, max_len=40, empty_frac=0.2, long_rows=(), dup_frac=0.0, shuffled=True):
    """Small irregular matrices for parity cases: row lengths uniform in
    [1, max_len] with a fraction of empty rows, optional long rows of the given
    lengths at seeded positions, optional duplicated entries (same row and
    column, different values)."""
    rng = _rng(seed, 60)
    lens = rng.integers(1, max_len + 1, size=m)
    lens[rng.random(m) < empty_frac] = 0
    long_rows = [min(int(L), n) for L in long_rows]
    if long_rows and m:
        pos = rng.choice(m, size=min(len(long_rows), m), replace=False)
        lens[pos] = long_rows[:pos.size]
    lens = np.minimum(lens, n)
    row, col = _triples_from_lengths(rng, m, n, lens, distinct=True)
    if dup_frac > 0 and row.size:
        d = rng.random(row.size) < dup_frac
        row = np.concatenate([row, row[d]])
        col = np.concatenate([col, col[d]])
    val = rng.uniform(-1.0, 1.0, size=row.size).astype(np.float32)
    coo = Coo(m, n, row.astype(np.int32), col.astype(np.int32), val)
    return shuffle_coo(coo, seed) if shuffled else coo


CONFIGS = {
    "spmv_uniform": dict(kind="spmv", build=lambda seed=0: uniform_rows_coo(seed=seed)),
    "spmv_powerlaw": dict(kind="spmv", build=lambda seed=0: powerlaw_coo(seed=seed)),
    "stencil27": dict(kind="pair", build=lambda seed=0: stencil27_coo(seed=seed)),
    "spmm_lognormal": dict(kind="spmm", build=lambda seed=0: lognormal_coo(seed=seed)),
    "bsr_blocks": dict(kind="bsr", build=lambda seed=0: block_sparse_bsr(seed=seed)),
}
