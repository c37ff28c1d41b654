// Column-panel entry stream for CSR SpMV on matrices whose columns scatter
// over an x much larger than one XCD's L2.
//
// 「通用稀疏矩阵乘法CUDA算子实现」 §2.5 names the random reads of x as the real
// cost of SpMV once x no longer fits in cache, and §2.4 asks for an entry-
// balanced split of long rows with a deterministic second stage.  Here the
// columns are cut into P panels of W = 2^cb columns and panel p is served
// only by the XCDs whose index is p mod P (workgroup id mod 8 is the XCD),
// so every gather of x falls in a W-float slice held by that XCD's L2.
//
// Layout (built once, at bind, in the plan workspace):
//   * every row with at most `S` entries contributes its panel-p entries to
//     the stream of panel p, rows ascending, columns ascending within a row;
//   * each panel's stream is cut into chunks at row boundaries, a chunk holding
//     at most kPsEntries entries (its start padded to a multiple of 4) and at
//     most 2^(32-cb) (and kPsMaxRows) rows; a chunk is {q_begin, q_end,
//     row_begin, row_end} and covers every row of [row_begin, row_end),
//     rows without panel-p entries included;
//   * an entry is one 32-bit word, column within the panel in the low cb bits
//     and row - row_begin in the high bits, plus its fp32 value;
//   * rows longer than S are cut out of the stream (they end chunks) and
//     served from the CSR in segments of split_seg entries over the whole x.
//
// spmv_pstream_kernel: one workgroup per chunk (and per split segment).  The
// chunk's entries are read with coalesced 16-byte loads (lane t of the
// workgroup holds the four runs of four entries starting at 4t, 1024 + 4t,
// 2048 + 4t, 3072 + 4t), x is gathered, and the row sums are formed by a
// segmented reduction over the 1024 runs: a suffix scan over (sum, link)
// pairs inside each wave, the same scan over the 16 wave blocks, then the run
// holding the first entry of a row writes the row's sum to LDS.  The sums are
// added in an order fixed by the layout alone, so results are reproducible
// bit for bit.  Rows of the chunk then go to ypart[p] (P > 1) or, with one
// panel, straight to y with the axpby epilogue.
//
// spmv_pstream_reduce_kernel: y = alpha * (ypart[0] + ... + ypart[P-1]) +
// beta * y for the stream rows (panel order fixed; 16-byte loads, the long
// rows skipped through a bitmask built at bind), and
// y = alpha * (sum of segment partials in segment order) + beta * y for the
// split rows.
#include <algorithm>

#include "seg_rows.h"

namespace spx {

namespace {

static_assert(kPsEntries == 4 * kPassRuns, "one pass of row sums per chunk");

struct PanelOffsets {
    int v[kXcds + 1];  // first chunk of each panel, v[P] = number of chunks
};

struct PsArgs {
    const int4* chunks;  // all panels, panel-major
    int coff[kXcds + 1]; // first chunk of each panel
    int P;               // panels (1, 2, 4 or 8)
    int G;               // XCDs per panel (8 / P)
    int cb;              // column bits: W = 1 << cb
    const uint32_t* pk;  // packed (row offset, column in panel)
    const float* pv;     // values
    float* ypart;        // [P][ystride] (P > 1)
    int64_t ystride;
    int n_split;         // split segments (first workgroups of the grid)
    int n_split_pad;     // n_split rounded up to a multiple of 8
    const int4* split_tasks;  // {partial index, 0, nz_begin, nz_end}
    const int32_t* idx;  // CSR arrays (split segments)
    const float* val;
    float* partials;
    float* y;            // output when P == 1
    float alpha, beta;
};

// Sum of val[q] * x[idx[q]] over [b, e) by the whole workgroup (valid in thread 0).
__device__ float segment_sum(const int32_t* __restrict__ idx, const float* __restrict__ val,
                             const float* __restrict__ x, int b, int e, float* red) {
    const int tid = threadIdx.x;
    float s = 0.0f;
    stream_products<4>(idx, val, x, b, e, tid, kBlock, [&](int, float p) { s += p; });
    s = wave_sum(s);
    if ((tid & 63) == 0) red[tid >> 6] = s;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(kBlock) void spmv_pstream_kernel(const PsArgs a, const float* __restrict__ x) {
    __shared__ float ysh[kPsMaxRows];
    __shared__ PassScratch sc;
    const int tid = threadIdx.x;
    int b = blockIdx.x;
    if (b < a.n_split) {
        const int4 t = a.split_tasks[b];
        const float s = segment_sum(a.idx, a.val, x, t.z, t.w, sc.agg_h);
        if (tid == 0) a.partials[t.x] = s;
        return;
    }
    if (b < a.n_split_pad) return;  // idle slots that align the chunks to XCD 0
    b -= a.n_split_pad;
    const int xcd = b & (kXcds - 1);
    const int p = xcd & (a.P - 1);
    const int i = (b >> 3) * a.G + xcd / a.P;
    const int c0 = a.coff[p];
    if (i >= a.coff[p + 1] - c0) return;
    const int4 c = a.chunks[c0 + i];
    const int qb = c.x, qe = c.y, R = c.w - c.z;
    const float* __restrict__ xp = x + ((int64_t)p << a.cb);
    const uint32_t cmask = (1u << a.cb) - 1u;

    // ---- loads: run u of this thread holds entries [qb + 1024u + 4 tid, +4)
    uint32_t pk[4][4];
    float pv[4][4];
    int nv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int q = qb + 1024 * u + 4 * tid;
        nv[u] = min(max(qe - q, 0), 4);
        if (nv[u] > 0) {
            const v4u32 k4 = __builtin_nontemporal_load(reinterpret_cast<const v4u32*>(a.pk + q));
            const v4f32 v4 = __builtin_nontemporal_load(reinterpret_cast<const v4f32*>(a.pv + q));
            pk[u][0] = k4.x; pk[u][1] = k4.y; pk[u][2] = k4.z; pk[u][3] = k4.w;
            pv[u][0] = v4.x; pv[u][1] = v4.y; pv[u][2] = v4.z; pv[u][3] = v4.w;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pk[u][j] = 0u;
                pv[u][j] = 0.0f;
            }
        }
    }
    // rows without entries in this chunk keep the zero written here
    for (int k = tid; k < R; k += kBlock) ysh[k] = 0.0f;
    __syncthreads();
    // ---- gathers of x (all issued before any product)
    float xv[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) xv[u][j] = j < nv[u] ? xp[pk[u][j] & cmask] : 0.0f;
    int ro[4][4];
    float pr[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ro[u][j] = (int)(pk[u][j] >> a.cb);
            pr[u][j] = pv[u][j] * xv[u][j];
        }
    pass_row_sums(ro, pr, nv, ysh, sc);
    __syncthreads();
    // ---- rows of the chunk: panel partials, or y itself with one panel
    const int rb = c.z;
    if (a.P == 1) {
        for (int k = tid; k < R; k += kBlock) store_axpby(a.y, rb + k, ysh[k], a.alpha, a.beta);
    } else {
        float* out = a.ypart + (int64_t)p * a.ystride + rb;
        for (int k = tid; k < R; k += kBlock) out[k] = ysh[k];
    }
}

// Four consecutive rows per thread: the P panel sums are read with 16-byte
// loads and added in panel order; rows marked in `skip` (the long rows, whose
// panel sums are never written) are left to the split part: one thread per
// long row adds its segment partials in segment order.
__global__ __launch_bounds__(kBlock) void spmv_pstream_reduce_kernel(
    int64_t rows, int n_row_blocks, int P, const float* __restrict__ ypart, int64_t ystride,
    const uint32_t* __restrict__ skip, int n_split_rows, const int4* __restrict__ split_rows,
    const float* __restrict__ partials, float alpha, float beta, float* __restrict__ y) {
    const int b = blockIdx.x;
    if (b < n_row_blocks) {
        const int64_t r0 = ((int64_t)b * kBlock + threadIdx.x) * 4;
        if (r0 >= rows) return;
        const uint32_t bits = (skip[r0 >> 5] >> (r0 & 31)) & 15u;
        if (r0 + 4 <= rows) {
            float4 s = *reinterpret_cast<const float4*>(ypart + r0);
            for (int p = 1; p < P; ++p) {
                const float4 t = *reinterpret_cast<const float4*>(ypart + (int64_t)p * ystride + r0);
                s.x += t.x;
                s.y += t.y;
                s.z += t.z;
                s.w += t.w;
            }
            const float v[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (!((bits >> j) & 1u)) store_axpby(y, (int)(r0 + j), v[j], alpha, beta);
        } else {
            for (int64_t r = r0; r < rows; ++r) {
                if ((bits >> (r - r0)) & 1u) continue;
                float t = ypart[r];
                for (int p = 1; p < P; ++p) t += ypart[(int64_t)p * ystride + r];
                store_axpby(y, (int)r, t, alpha, beta);
            }
        }
        return;
    }
    const int j = (b - n_row_blocks) * kBlock + (int)threadIdx.x;
    if (j >= n_split_rows) return;
    const int4 sr = split_rows[j];  // {row, partial_base, nseg, 0}
    float t = 0.0f;
    for (int k = 0; k < sr.z; ++k) t += partials[sr.y + k];
    store_axpby(y, sr.x, t, alpha, beta);
}

// Bind time: one workgroup per chunk writes the chunk's entries (row by row,
// from start[p * rows + r]) and zero padding up to the next multiple of 4.
__global__ __launch_bounds__(kBlock) void ps_build_kernel(
    const int4* __restrict__ chunks, int n_chunks, const PanelOffsets coff, int P, int cb,
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx, const float* __restrict__ val,
    const int32_t* __restrict__ start, int64_t rows, uint32_t* __restrict__ pk, float* __restrict__ pv) {
    const int ci = blockIdx.x;
    if (ci >= n_chunks) return;
    int p = 0;
    while (p + 1 < P && ci >= coff.v[p + 1]) ++p;
    const int4 c = chunks[ci];
    const int rb = c.z;
    for (int r = rb + (int)threadIdx.x; r < c.w; r += kBlock) {
        int s = start[(int64_t)p * rows + r];
        const uint32_t rowbits = (uint32_t)(r - rb) << cb;
        for (int k = ptr[r]; k < ptr[r + 1]; ++k) {
            const int col = idx[k];
            if ((col >> cb) == p) {
                pk[s] = rowbits | ((uint32_t)col & ((1u << cb) - 1u));
                pv[s] = val[k];
                ++s;
            }
        }
    }
    const int pad_end = (c.y + 3) & ~3;
    if ((int)threadIdx.x < pad_end - c.y) {
        pk[c.y + threadIdx.x] = 0u;
        pv[c.y + threadIdx.x] = 0.0f;
    }
}

}  // namespace

hipError_t launch_pstream_build(const DirDevice& d, const int32_t* start, hipStream_t s) {
    const int n = d.ps_coff[d.ps_P];
    if (n == 0) return hipSuccess;
    PanelOffsets coff{};
    for (int k = 0; k <= kXcds; ++k) coff.v[k] = d.ps_coff[std::min(k, (int)d.ps_P)];
    hipLaunchKernelGGL(ps_build_kernel, dim3((unsigned)n), dim3(kBlock), 0, s, d.ps_chunks, n, coff, d.ps_P,
                       d.ps_cb, d.ptr, d.idx, d.val, start, (int64_t)d.rows, d.ps_pk, d.ps_pv);
    return hipGetLastError();
}

hipError_t launch_spmv_pstream(const DirDevice& d, float alpha, const float* x, float beta, float* y,
                               hipStream_t s) {
    PsArgs a{};
    a.chunks = d.ps_chunks;
    for (int k = 0; k <= kXcds; ++k) a.coff[k] = k <= d.ps_P ? d.ps_coff[k] : d.ps_coff[d.ps_P];
    a.P = d.ps_P;
    a.G = kXcds / d.ps_P;
    a.cb = d.ps_cb;
    a.pk = d.ps_pk;
    a.pv = d.ps_pv;
    a.ypart = d.ps_ypart;
    a.ystride = d.ps_ystride;
    a.n_split = d.ps_n_split_tasks;
    a.n_split_pad = (d.ps_n_split_tasks + kXcds - 1) / kXcds * kXcds;
    a.split_tasks = d.ps_split_tasks;
    a.idx = d.idx;
    a.val = d.val;
    a.partials = d.ps_partials;
    a.y = y;
    a.alpha = alpha;
    a.beta = beta;
    int max_chunks = 0;
    for (int p = 0; p < d.ps_P; ++p) max_chunks = std::max(max_chunks, d.ps_coff[p + 1] - d.ps_coff[p]);
    const int64_t slots = (int64_t)kXcds * ((max_chunks + a.G - 1) / a.G);
    const int64_t grid = a.n_split_pad + slots;
    if (grid > 0) {
        hipLaunchKernelGGL(spmv_pstream_kernel, dim3((unsigned)grid), dim3(kBlock), 0, s, a, x);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    const int64_t n_row_blocks = d.ps_P > 1 ? ((int64_t)d.rows + 4 * kBlock - 1) / (4 * kBlock) : 0;
    const int64_t rgrid = n_row_blocks + (d.ps_n_split_rows + kBlock - 1) / kBlock;
    if (rgrid > 0) {
        hipLaunchKernelGGL(spmv_pstream_reduce_kernel, dim3((unsigned)rgrid), dim3(kBlock), 0, s, (int64_t)d.rows,
                           (int)n_row_blocks, d.ps_P, d.ps_ypart, d.ps_ystride, d.ps_skip, d.ps_n_split_rows,
                           d.ps_split_rows, d.ps_partials, alpha, beta, y);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace spx
