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
#include <algorithm>

#include "device_common.h"

namespace spx {

namespace {

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
    float* partials, int32_t* counters, int group_cap) {
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
    group_task(t, ptr, idx, val, x, alpha, beta, y, lds, group_cap);
}

// ---- SELL-C-sigma, C = 64: one wave per slice, one lane per row -----------
// (「通用稀疏矩阵乘法CUDA算子实现」 §1.4; the slot layout of
// 「稀疏矩阵存储格式…」 §4 with slot t of all lanes adjacent.)  Lanes whose
// row is served by another bin (length -1) do nothing; padding is skipped by
// the length test, never multiplied.  Col is the column itself (int32) or,
// when every stored column lies within 32767 of its row (banded matrices),
// the offset column - row (int16), which cuts 2 of the 8 bytes per slot.
template <typename Col>
__global__ __launch_bounds__(kBlock) void spmv_sell_kernel(
    int rows, int slices, const int64_t* __restrict__ slice_ptr, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ len, const Col* __restrict__ col, const float* __restrict__ val,
    const float* __restrict__ x, float alpha, float beta, float* __restrict__ y, int xcd_remap) {
    // with xcd_remap each XCD takes one contiguous run of slices, so the x
    // lines that neighbouring rows share stay in that XCD's L2
    const int wg = xcd_remap ? xcd_contiguous(blockIdx.x, 0, gridDim.x) : blockIdx.x;
    const int slice = wg * 4 + (threadIdx.x >> 6);
    if (slice >= slices) return;
    const int lane = threadIdx.x & 63;
    const int k = slice * 64 + lane;
    if (k >= rows) return;
    const int L = len[k];
    if (L < 0) return;
    const int row = perm[k];
    const int base = sizeof(Col) == 2 ? row : 0;  // columns are stored relative to the row
    const Col* cp = col + slice_ptr[slice] + lane;
    const float* vp = val + slice_ptr[slice] + lane;
    float s = 0.0f;
    int t = 0;
    // 8 slots at a time: all loads, then all gathers, then the sums in slot order
    for (; t + 8 <= L; t += 8) {
        int c[8];
        float a[8], xv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            c[u] = base + (int)__builtin_nontemporal_load(cp + (int64_t)(t + u) * 64);
            a[u] = __builtin_nontemporal_load(vp + (int64_t)(t + u) * 64);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) xv[u] = x[c[u]];
#pragma unroll
        for (int u = 0; u < 8; ++u) s += a[u] * xv[u];
    }
    for (; t < L; ++t)
        s += __builtin_nontemporal_load(vp + (int64_t)t * 64) *
             x[base + (int)__builtin_nontemporal_load(cp + (int64_t)t * 64)];
    store_axpby(y, row, s, alpha, beta);
}

// Largest |column - row| over the entries of the SELL rows (atomic max into *out).
__global__ __launch_bounds__(kBlock) void sell_offset_kernel(int rows, int slices, const int32_t* __restrict__ perm,
                                                             const int32_t* __restrict__ len,
                                                             const int32_t* __restrict__ ptr,
                                                             const int32_t* __restrict__ idx, int32_t* out) {
    const int k = blockIdx.x * kBlock + threadIdx.x;
    int m = 0;
    if (k < rows && k < slices * 64) {
        const int L = len[k];
        if (L > 0) {
            const int row = perm[k];
            const int p0 = ptr[row];
            for (int t = 0; t < L; ++t) m = max(m, abs(idx[p0 + t] - row));
        }
    }
    for (int o = 32; o > 0; o >>= 1) m = max(m, __shfl_xor(m, o, 64));
    if ((threadIdx.x & 63) == 0 && m > 0) atomicMax(out, m);
}

// Fill the SELL slot arrays from the CSR (padding: column -1 or offset 0, value 0).
template <typename Col>
__global__ __launch_bounds__(kBlock) void sell_fill_kernel(
    int rows, int slices, const int64_t* __restrict__ slice_ptr, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ len, const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
    const float* __restrict__ val, Col* __restrict__ scol, float* __restrict__ sval) {
    const int slice = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (slice >= slices) return;
    const int lane = threadIdx.x & 63;
    const int k = slice * 64 + lane;
    const int64_t base = slice_ptr[slice];
    const int width = (int)((slice_ptr[slice + 1] - base) / 64);
    const int L = k < rows ? len[k] : -1;
    const int row = (k < rows && L > 0) ? perm[k] : 0;
    const int p0 = (k < rows && L > 0) ? ptr[row] : 0;
    const int rel = sizeof(Col) == 2 ? row : 0;
    for (int t = 0; t < width; ++t) {
        const int64_t q = base + (int64_t)t * 64 + lane;
        if (t < L) {
            scol[q] = (Col)(idx[p0 + t] - rel);
            sval[q] = val[p0 + t];
        } else {
            scol[q] = (Col)(sizeof(Col) == 2 ? 0 : -1);
            sval[q] = 0.0f;
        }
    }
}

}  // namespace

hipError_t launch_spmv(const DirDevice& d, float alpha, const float* x, float beta, float* y, hipStream_t s) {
    if (d.xw_bits > 0) return launch_spmv_xwin(d, alpha, x, beta, y, s);
    if (d.ps_P > 0) return launch_spmv_pstream(d, alpha, x, beta, y, s);
    const int n_wave_wg = (d.n_wave + 3) / 4;
    const int n_group = d.use_sell ? 0 : d.n_group;
    const int64_t grid = (int64_t)d.n_split + d.n_block + n_wave_wg + n_group;
    if (grid > 0) {
        // products | row starts | heads (group tasks)
        const size_t lds_bins = (size_t)(d.group_cap + (kGroupMaxRows + 1) + kBlock) * sizeof(float);
        hipLaunchKernelGGL(spmv_bins_kernel, dim3((unsigned)grid), dim3(kBlock), lds_bins, s, d.tasks, d.n_split,
                           d.n_block, d.n_wave, n_group, d.xcd_remap, d.split_rows, d.ptr, d.idx, d.val, x, alpha,
                           beta, y, d.partials, d.counters, d.group_cap);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (d.use_sell && d.sell_slices > 0) {
        const dim3 grid((unsigned)((d.sell_slices + 3) / 4));
        if (d.sell_narrow)
            hipLaunchKernelGGL(spmv_sell_kernel<int16_t>, grid, dim3(kBlock), 0, s, d.rows, d.sell_slices,
                               d.sell_slice_ptr, d.sell_perm, d.sell_len, reinterpret_cast<const int16_t*>(d.sell_col),
                               d.sell_val, x, alpha, beta, y, d.xcd_remap);
        else
            hipLaunchKernelGGL(spmv_sell_kernel<int32_t>, grid, dim3(kBlock), 0, s, d.rows, d.sell_slices,
                               d.sell_slice_ptr, d.sell_perm, d.sell_len, d.sell_col, d.sell_val, x, alpha, beta, y,
                               d.xcd_remap);
        return hipGetLastError();
    }
    return hipSuccess;
}

hipError_t launch_sell_offset(const DirDevice& d, int32_t* out, hipStream_t s) {
    if (d.sell_slices <= 0) return hipSuccess;
    const int64_t n = std::min<int64_t>((int64_t)d.rows, (int64_t)d.sell_slices * 64);
    hipLaunchKernelGGL(sell_offset_kernel, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, d.rows,
                       d.sell_slices, d.sell_perm, d.sell_len, d.ptr, d.idx, out);
    return hipGetLastError();
}

hipError_t launch_sell_fill(const DirDevice& d, int64_t slots, int32_t* sell_col, float* sell_val, hipStream_t s) {
    (void)slots;
    if (d.sell_slices <= 0) return hipSuccess;
    const dim3 grid((unsigned)((d.sell_slices + 3) / 4));
    if (d.sell_narrow)
        hipLaunchKernelGGL(sell_fill_kernel<int16_t>, grid, dim3(kBlock), 0, s, d.rows, d.sell_slices, d.sell_slice_ptr,
                           d.sell_perm, d.sell_len, d.ptr, d.idx, d.val, reinterpret_cast<int16_t*>(sell_col),
                           sell_val);
    else
        hipLaunchKernelGGL(sell_fill_kernel<int32_t>, grid, dim3(kBlock), 0, s, d.rows, d.sell_slices, d.sell_slice_ptr,
                           d.sell_perm, d.sell_len, d.ptr, d.idx, d.val, sell_col, sell_val);
    return hipGetLastError();
}

}  // namespace spx
