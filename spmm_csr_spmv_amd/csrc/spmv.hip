// CSR SpMV  y = alpha * A x + beta * y  for gfx950.
//
// One launch serves every row bin of a plan (「通用稀疏矩阵乘法CUDA算子实现」 §2:
// the parallel grain must follow the row length, §4: the bins come from a
// cached profile).  The grid is the concatenation
//     [split segments | block rows | wave rows (4 per workgroup) | groups]
// so the longest tasks are dispatched first, and the bin of a workgroup is a
// uniform branch on blockIdx.  The same kernel computes A^T u on the CSC
// (「CUDA LSMR 专栏（二）」 §2, §4: the CSC arrays are the CSR of A^T).
//
// Every bin streams values and column indices with 16-byte loads, gathers x,
// and fuses the axpby epilogue y = alpha*acc + beta*y into its single store
// (「CUDA LSMR 专栏（二）」 §5.2); beta == 0 never reads y.
#include "device_common.h"

namespace spx {

namespace {

// Products val[q] * x[idx[q]] for q in [b, e).  Lane `lane` of `stride`
// lanes owns the 4-entry chunks starting at (b & ~3) + 4*lane + 4*stride*k.
// Chunks are taken U at a time: the U column/value loads (16-byte loads for
// full chunks, guarded scalar loads at the ragged ends) are all issued before
// the gathers of x, and all gathers before any product, so every lane keeps
// up to 8U independent memory requests in flight.  `emit(q, prod)` receives
// each valid product; slots outside [b, e) are never read nor multiplied.
template <int U, class Emit>
__device__ __forceinline__ void stream_products(const int32_t* __restrict__ idx, const float* __restrict__ val,
                                                const float* __restrict__ x, int b, int e, int lane, int stride,
                                                Emit emit) {
    const int base = b & ~3;
    for (int v0 = base + 4 * lane; v0 < e; v0 += 4 * stride * U) {
        int c[U][4];
        float a[U][4];
        bool ok[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + 4 * stride * u;
            if (v >= b && v + 4 <= e) {
                const int4 ci = ldg4_nt(idx + v);
                const float4 ai = ldg4_nt(val + v);
                c[u][0] = ci.x; c[u][1] = ci.y; c[u][2] = ci.z; c[u][3] = ci.w;
                a[u][0] = ai.x; a[u][1] = ai.y; a[u][2] = ai.z; a[u][3] = ai.w;
#pragma unroll
                for (int j = 0; j < 4; ++j) ok[u][j] = true;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int q = v + j;
                    ok[u][j] = q >= b && q < e;
                    c[u][j] = ok[u][j] ? idx[q] : 0;
                    a[u][j] = ok[u][j] ? val[q] : 0.0f;
                }
            }
        }
        float xv[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) xv[u][j] = ok[u][j] ? x[c[u][j]] : 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + 4 * stride * u;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (ok[u][j]) emit(v + j, a[u][j] * xv[u][j]);
        }
    }
}

__device__ __forceinline__ void store_axpby(float* __restrict__ y, int row, float acc, float alpha, float beta) {
    float o = alpha * acc;
    if (beta != 0.0f) o = fmaf(beta, y[row], o);
    y[row] = o;
}

// Row sums of R consecutive rows whose E products sit in LDS (prod[0..E)),
// with row i covering prod[rs[i] .. rs[i+1]) (rs in LDS, rs[R] = E).
// The products are split evenly: thread t reads chunk [tC, tC + C) with
// C = ceil(E / 256), whatever the row lengths.  Thread t owns the rows that
// start in [tC, (t+1)C) (thread 255 also owns rows starting later, i.e. empty
// rows at the end).  A thread first stores in head[t] the part of its chunk
// that belongs to a row started in an earlier chunk; after a barrier, each
// owner adds its own part and then head[t+1], head[t+2], ... for a row that
// runs past its chunk.  The order of additions is fixed by E and rs, so the
// result is reproducible bit for bit.  out(i, sum) is called once per row.
template <class Out>
__device__ __forceinline__ void balanced_row_sums(const float* prod, int E, const int* rs, int R, float* head,
                                                  Out out) {
    const int t = threadIdx.x;
    const int C = E > 0 ? (E + kBlock - 1) / kBlock : 1;
    const int lo_s = t * C;
    const int hi_s = t == kBlock - 1 ? 0x7fffffff : lo_s + C;
    const int c0 = min(lo_s, E), c1 = min(lo_s + C, E);
    int lo = 0, hi = R;  // first row starting at or after lo_s
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (rs[mid] < lo_s) lo = mid + 1; else hi = mid;
    }
    const int first = lo;
    const int head_end = first < R ? min(c1, rs[first]) : c1;
    float h = 0.0f;
    for (int k = c0; k < head_end; ++k) h += prod[k];
    head[t] = h;
    __syncthreads();
    for (int i = first; i < R && rs[i] < hi_s; ++i) {
        const int beg = rs[i], end = rs[i + 1];
        float s = 0.0f;
        for (int k = beg; k < min(end, c1); ++k) s += prod[k];
        if (end > c1) {
            const int last_chunk = (end - 1) / C;
            for (int tt = t + 1; tt <= last_chunk; ++tt) s += head[tt];
        }
        out(i, s);
    }
}

// ---- group: consecutive short rows staged through LDS --------------------
// LDS: products [group_cap] | row starts [257] | heads [256]
__device__ void group_task(const int4 t, const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
                           const float* __restrict__ val, const float* __restrict__ x, float alpha, float beta,
                           float* __restrict__ y, float* lds, int group_cap) {
    const int r0 = t.x, r1 = t.y, b = t.z, e = t.w;
    const int R = r1 - r0;
    const int tid = threadIdx.x;
    int* rs = reinterpret_cast<int*>(lds + group_cap);
    float* head = lds + group_cap + (kGroupMaxRows + 1);
    for (int i = tid; i <= R; i += kBlock) rs[i] = ptr[r0 + i] - b;
    stream_products<kGroupMaxNnz / (4 * kBlock)>(idx, val, x, b, e, tid, kBlock,
                                                  [&](int q, float p) { lds[q - b] = p; });
    __syncthreads();
    balanced_row_sums(lds, e - b, rs, R, head, [&](int i, float s) { store_axpby(y, r0 + i, s, alpha, beta); });
}

// Exclusive prefix sum of one int per thread over the 256-thread workgroup
// (Hillis-Steele in LDS, sh: 256 ints); *total receives the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* sh, int* total) {
    const int tid = threadIdx.x;
    sh[tid] = v;
    __syncthreads();
    for (int off = 1; off < kBlock; off <<= 1) {
        const int add = tid >= off ? sh[tid - off] : 0;
        __syncthreads();
        sh[tid] += add;
        __syncthreads();
    }
    const int incl = sh[tid];
    *total = sh[kBlock - 1];
    __syncthreads();
    return incl - v;
}

// ---- column panels -----------------------------------------------------------
// For matrices whose columns scatter over an x much larger than one XCD's L2,
// the columns are cut into P panels of width W and panel p is served only by
// XCD p (workgroup id mod 8 = XCD): every gather of x then falls in a W-float
// slice that stays in that XCD's L2.  Each group's entries are copied once, at
// bind time, in (panel, row, column) order inside the group's own range
// [nz_begin, nz_end) of the copy; poff[p * rows + r] is the offset of row r's
// first entry inside the block of panel p of its group (16 bits: a panel group
// holds at most 1024 rows and P * 2048 entries, well below 65536) and
// pstart[g * (P + 1) + p] the offset of panel p inside group g, so a
// row's panel entries need no search.  Panel groups are their own grouping
// (larger than the LDS-staged groups: each (group, panel) block is sized to
// fill the LDS of one workgroup about half way).  The panel
// kernel writes ypart[p * rows + r] = sum of row r over panel p; the bins
// kernel then forms y = alpha * (ypart[0] + ... + ypart[P-1]) + beta * y in
// that fixed order.

// One workgroup per panel group: builds the panel-major copy, the row offsets
// and the block starts.  Runs once per bind; reads the columns from global
// memory.  flag[0] is raised when a panel block exceeds `cap` entries (the
// LDS capacity of the panel kernel); the plan then does not use panels.
__global__ __launch_bounds__(kBlock) void panel_build_kernel(
    const int4* __restrict__ gtasks, int rows, const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
    const float* __restrict__ val, int P, int W, int cap, int32_t* __restrict__ pcol, float* __restrict__ pval,
    int32_t* __restrict__ pstart, uint16_t* __restrict__ poff, int32_t* __restrict__ flag) {
    __shared__ int rowoff[8][kBlock];
    __shared__ int scan[kBlock];
    __shared__ int pst[9];
    __shared__ int carry[8];
    const int4 t = gtasks[blockIdx.x];
    const int r0 = t.x, R = t.y - t.x, b = t.z, E = t.w - t.z;
    const int tid = threadIdx.x;
    if (tid < 8) carry[tid] = 0;
    // pass 1: entries per panel -> block starts (exclusive over panels)
    int tot[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) tot[p] = 0;
    for (int q = tid; q < E; q += kBlock) {
        const int p = idx[b + q] / W;
#pragma unroll
        for (int k = 0; k < 8; ++k) tot[k] += (k == p);
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        if (p < P) {  // P is uniform: every thread takes the same branches
            int total;
            block_exclusive_scan(tot[p], scan, &total);
            if (tid == 0) pst[p] = total;
            __syncthreads();
        }
    }
    if (tid == 0) {
        int s = 0;
        for (int p = 0; p < P; ++p) {
            const int n = pst[p];
            if (n > cap) atomicOr(flag, 1);
            pst[p] = s;
            pstart[(int64_t)blockIdx.x * (P + 1) + p] = s;
            s += n;
        }
        pst[P] = s;
        pstart[(int64_t)blockIdx.x * (P + 1) + P] = s;
    }
    __syncthreads();
    // pass 2, per chunk of 256 rows: offsets of each row inside each panel
    // block (running offsets carried across chunks), then the copy
    for (int c0 = 0; c0 < R; c0 += kBlock) {
        const int row = c0 + tid;
        const bool in = row < R;
        const int rb = in ? ptr[r0 + row] : 0, re = in ? ptr[r0 + row + 1] : 0;
        int c[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) c[p] = 0;
        for (int k = rb; k < re; ++k) {
            const int p = idx[k] / W;
#pragma unroll
            for (int q = 0; q < 8; ++q) c[q] += (q == p);
        }
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            if (p < P) {
                int total;
                const int ex = block_exclusive_scan(c[p], scan, &total);
                rowoff[p][tid] = carry[p] + ex;
                __syncthreads();
                if (tid == 0) carry[p] += total;
            }
        }
        if (in) {
            int pos[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                pos[p] = p < P ? rowoff[p][tid] : 0;
                if (p < P) poff[(int64_t)p * rows + r0 + row] = (uint16_t)min(pos[p], 65535);
                pos[p] += p < P ? b + pst[p] : 0;
            }
            for (int k = rb; k < re; ++k) {
                const int col = idx[k];
                const int p = col / W;
                int d = 0;
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    if (q == p) d = pos[q]++;
                pcol[d] = col;
                pval[d] = val[k];
            }
        }
        __syncthreads();
    }
}

// One workgroup per (group, panel); panel = workgroup id mod P, so with P = 8
// panel p runs on XCD p.  LDS: products [group_cap] | row starts [257] |
// heads [256].
__global__ __launch_bounds__(kBlock) void spmv_panel_kernel(
    const int4* __restrict__ gtasks, int rows, int P, const int32_t* __restrict__ pcol,
    const float* __restrict__ pval, const int32_t* __restrict__ pstart, const uint16_t* __restrict__ poff,
    const float* __restrict__ x, float* __restrict__ ypart, int group_cap) {
    extern __shared__ float lds[];
    int* rs = reinterpret_cast<int*>(lds + group_cap);
    float* head = lds + group_cap + (kGroupMaxRows + 1);
    const int p = blockIdx.x % P, g = blockIdx.x / P;
    const int4 t = gtasks[g];
    const int r0 = t.x, R = t.y - t.x;
    const int tid = threadIdx.x;
    const int qb = t.z + pstart[(int64_t)g * (P + 1) + p];
    const int qe = t.z + pstart[(int64_t)g * (P + 1) + p + 1];
    for (int i = tid; i < R; i += kBlock) rs[i] = poff[(int64_t)p * rows + r0 + i];
    if (tid == 0) rs[R] = qe - qb;
    stream_products<kGroupMaxNnz / (4 * kBlock)>(pcol, pval, x, qb, qe, tid, kBlock,
                                                  [&](int q, float v) { lds[q - qb] = v; });
    __syncthreads();
    float* out = ypart + (int64_t)p * rows + r0;
    balanced_row_sums(lds, qe - qb, rs, R, head, [&](int i, float s) { out[i] = s; });
}

// ---- wave: one row per wave64 ----------------------------------------------
__device__ void wave_task(const int4 t, const int32_t* __restrict__ idx, const float* __restrict__ val,
                          const float* __restrict__ x, float alpha, float beta, float* __restrict__ y, bool valid) {
    const int lane = threadIdx.x & 63;
    float s = 0.0f;
    if (valid) stream_products<4>(idx, val, x, t.y, t.z, lane, 64, [&](int, float p) { s += p; });
    s = wave_sum(s);
    if (valid && lane == 0) store_axpby(y, t.x, s, alpha, beta);
}

// Sum of a 256-thread workgroup over [b, e) (valid in thread 0).
__device__ __forceinline__ float block_reduce_range(const int32_t* __restrict__ idx, const float* __restrict__ val,
                                                    const float* __restrict__ x, int b, int e, float* lds) {
    const int tid = threadIdx.x;
    float s = 0.0f;
    stream_products<4>(idx, val, x, b, e, tid, kBlock, [&](int, float p) { s += p; });
    s = wave_sum(s);
    if ((tid & 63) == 0) lds[tid >> 6] = s;
    __syncthreads();
    float r = 0.0f;
    if (tid == 0) r = (lds[0] + lds[1]) + (lds[2] + lds[3]);
    return r;
}

// ---- block: one row per workgroup ---------------------------------------------
__device__ void block_task(const int4 t, const int32_t* __restrict__ idx, const float* __restrict__ val,
                           const float* __restrict__ x, float alpha, float beta, float* __restrict__ y, float* lds) {
    const float s = block_reduce_range(idx, val, x, t.y, t.z, lds);
    if (threadIdx.x == 0) store_axpby(y, t.x, s, alpha, beta);
}

// ---- split: one segment of a very long row per workgroup ------------------
// The segment's sum goes to partials[]; the workgroup that finishes last
// (integer arrival counter) adds the row's partials in segment order, so the
// result does not depend on arrival order.  The counter is put back to 0 by
// that last workgroup, ready for the next launch.
__device__ void split_task(const int4 t, const int4* __restrict__ split_rows, const int32_t* __restrict__ idx,
                           const float* __restrict__ val, const float* __restrict__ x, float alpha, float beta,
                           float* __restrict__ y, float* partials, int32_t* counters, float* lds) {
    const int4 sr = split_rows[t.x];  // {row, partial_base, nseg, 0}
    const float s = block_reduce_range(idx, val, x, t.z, t.w, lds);
    if (threadIdx.x == 0) {
        atomic_store_f(partials + sr.y + t.y, s);
        const int arrived = __hip_atomic_fetch_add(counters + t.x, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (arrived == sr.z - 1) {
            float acc = 0.0f;
            for (int k = 0; k < sr.z; ++k) acc += atomic_load_f(partials + sr.y + k);
            store_axpby(y, sr.x, acc, alpha, beta);
            __hip_atomic_store(counters + t.x, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

__global__ __launch_bounds__(kBlock) void spmv_bins_kernel(
    const int4* __restrict__ tasks, int n_split, int n_block, int n_wave, int n_group, int xcd_remap,
    const int4* __restrict__ split_rows, const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
    const float* __restrict__ val, const float* __restrict__ x, float alpha, float beta, float* __restrict__ y,
    float* partials, int32_t* counters, int group_cap, const float* __restrict__ ypart, int npanels, int rows) {
    extern __shared__ float lds[];
    int b = blockIdx.x;
    if (b < n_split) {
        split_task(tasks[b], split_rows, idx, val, x, alpha, beta, y, partials, counters, lds);
        return;
    }
    b -= n_split;
    if (b < n_block) {
        block_task(tasks[n_split + b], idx, val, x, alpha, beta, y, lds);
        return;
    }
    b -= n_block;
    const int n_wave_wg = (n_wave + 3) / 4;
    if (b < n_wave_wg) {
        const int w = 4 * b + (threadIdx.x >> 6);
        const bool valid = w < n_wave;
        const int4 t = valid ? tasks[n_split + n_block + w] : make_int4(0, 0, 0, 0);
        wave_task(t, idx, val, x, alpha, beta, y, valid);
        return;
    }
    b -= n_wave_wg;
    const int first = n_split + n_block + n_wave_wg;
    const int g = xcd_remap ? xcd_contiguous(blockIdx.x, first, n_group) : b;
    const int4 t = tasks[n_split + n_block + n_wave + g];
    if (npanels > 0) {
        // the group's rows were summed per column panel: add the panels in order
        for (int r = t.x + (int)threadIdx.x; r < t.y; r += kBlock) {
            float s = 0.0f;
            for (int p = 0; p < npanels; ++p) s += ypart[(int64_t)p * rows + r];
            store_axpby(y, r, s, alpha, beta);
        }
        return;
    }
    group_task(t, ptr, idx, val, x, alpha, beta, y, lds, group_cap);
}

// ---- SELL-C-sigma, C = 64: one wave per slice, one lane per row -----------
// (「通用稀疏矩阵乘法CUDA算子实现」 §1.4; the slot layout of
// 「稀疏矩阵存储格式…」 §4 with slot t of all lanes adjacent.)  Lanes whose
// row is served by another bin (length -1) do nothing; padding is skipped by
// the length test, never multiplied.
__global__ __launch_bounds__(kBlock) void spmv_sell_kernel(
    int rows, int slices, const int64_t* __restrict__ slice_ptr, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ len, const int32_t* __restrict__ col, const float* __restrict__ val,
    const float* __restrict__ x, float alpha, float beta, float* __restrict__ y) {
    const int slice = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (slice >= slices) return;
    const int lane = threadIdx.x & 63;
    const int k = slice * 64 + lane;
    if (k >= rows) return;
    const int L = len[k];
    if (L < 0) return;
    const int32_t* cp = col + slice_ptr[slice] + lane;
    const float* vp = val + slice_ptr[slice] + lane;
    float s = 0.0f;
    int t = 0;
    // 8 slots at a time: all loads, then all gathers, then the sums in slot order
    for (; t + 8 <= L; t += 8) {
        int c[8];
        float a[8], xv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            c[u] = __builtin_nontemporal_load(cp + (int64_t)(t + u) * 64);
            a[u] = __builtin_nontemporal_load(vp + (int64_t)(t + u) * 64);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) xv[u] = x[c[u]];
#pragma unroll
        for (int u = 0; u < 8; ++u) s += a[u] * xv[u];
    }
    for (; t < L; ++t) s += __builtin_nontemporal_load(vp + (int64_t)t * 64) * x[__builtin_nontemporal_load(cp + (int64_t)t * 64)];
    store_axpby(y, perm[k], s, alpha, beta);
}

// Fill the SELL slot arrays from the CSR (padding: column -1, value 0).
__global__ __launch_bounds__(kBlock) void sell_fill_kernel(
    int rows, int slices, const int64_t* __restrict__ slice_ptr, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ len, const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
    const float* __restrict__ val, int32_t* __restrict__ scol, float* __restrict__ sval) {
    const int slice = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (slice >= slices) return;
    const int lane = threadIdx.x & 63;
    const int k = slice * 64 + lane;
    const int64_t base = slice_ptr[slice];
    const int width = (int)((slice_ptr[slice + 1] - base) / 64);
    const int L = k < rows ? len[k] : -1;
    const int p0 = (k < rows && L > 0) ? ptr[perm[k]] : 0;
    for (int t = 0; t < width; ++t) {
        const int64_t q = base + (int64_t)t * 64 + lane;
        if (t < L) {
            scol[q] = idx[p0 + t];
            sval[q] = val[p0 + t];
        } else {
            scol[q] = -1;
            sval[q] = 0.0f;
        }
    }
}

}  // namespace

hipError_t launch_spmv(const DirDevice& d, float alpha, const float* x, float beta, float* y, hipStream_t s) {
    const int n_wave_wg = (d.n_wave + 3) / 4;
    const bool panels = d.npanels > 0;
    // with panels the group part of the bins launch runs over the panel groups
    const int4* tasks = panels ? d.ptasks : d.tasks;
    const int n_group = d.use_sell ? 0 : (panels ? d.n_pgroup : d.n_group);
    const int64_t grid = (int64_t)d.n_split + d.n_block + n_wave_wg + n_group;
    // products | row starts | heads (group and panel tasks)
    const size_t lds = (size_t)(kGroupMaxNnz + (kGroupMaxRows + 1) + kBlock) * sizeof(float);
    if (panels && d.n_pgroup > 0) {
        const int4* gtasks = d.ptasks + d.n_split + d.n_block + d.n_wave;
        hipLaunchKernelGGL(spmv_panel_kernel, dim3((unsigned)((int64_t)d.n_pgroup * d.npanels)), dim3(kBlock), lds,
                           s, gtasks, d.rows, d.npanels, d.pcol, d.pval, d.pstart, d.poff, x, d.ypart,
                           kGroupMaxNnz);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (grid > 0) {
        const size_t lds_bins = (size_t)(d.group_cap + (kGroupMaxRows + 1) + kBlock) * sizeof(float);
        hipLaunchKernelGGL(spmv_bins_kernel, dim3((unsigned)grid), dim3(kBlock), lds_bins, s, tasks, d.n_split,
                           d.n_block, d.n_wave, n_group, d.xcd_remap, d.split_rows, d.ptr, d.idx, d.val, x, alpha,
                           beta, y, d.partials, d.counters, d.group_cap, d.ypart, d.npanels, d.rows);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (d.use_sell && d.sell_slices > 0) {
        hipLaunchKernelGGL(spmv_sell_kernel, dim3((unsigned)((d.sell_slices + 3) / 4)), dim3(kBlock), 0, s, d.rows,
                           d.sell_slices, d.sell_slice_ptr, d.sell_perm, d.sell_len, d.sell_col, d.sell_val, x,
                           alpha, beta, y);
        return hipGetLastError();
    }
    return hipSuccess;
}

hipError_t launch_panel_build(const DirDevice& d, int32_t* flag, hipStream_t s) {
    if (d.npanels <= 0 || d.n_pgroup <= 0) return hipSuccess;
    const int4* gtasks = d.ptasks + d.n_split + d.n_block + d.n_wave;
    hipLaunchKernelGGL(panel_build_kernel, dim3((unsigned)d.n_pgroup), dim3(kBlock), 0, s, gtasks, d.rows, d.ptr,
                       d.idx, d.val, d.npanels, d.panel_width, kGroupMaxNnz, d.pcol, d.pval, d.pstart, d.poff, flag);
    return hipGetLastError();
}

hipError_t launch_sell_fill(const DirDevice& d, int64_t slots, int32_t* sell_col, float* sell_val, hipStream_t s) {
    (void)slots;
    if (d.sell_slices <= 0) return hipSuccess;
    hipLaunchKernelGGL(sell_fill_kernel, dim3((unsigned)((d.sell_slices + 3) / 4)), dim3(kBlock), 0, s, d.rows,
                       d.sell_slices, d.sell_slice_ptr, d.sell_perm, d.sell_len, d.ptr, d.idx, d.val, sell_col,
                       sell_val);
    return hipGetLastError();
}

}  // namespace spx
