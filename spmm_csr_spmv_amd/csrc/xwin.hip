// x-window stream: CSR SpMV for matrices whose columns scatter over an x far
// larger than an XCD's L2, with every gather of x served from LDS.
//
// 「通用稀疏矩阵乘法CUDA算子实现」 §2.5 names the random reads of x as the real
// cost of SpMV once x no longer fits in cache, §2.1 stages data through
// shared memory, and §2.4 asks for long rows to be cut into pieces whose
// partial sums are combined in a fixed order.  On MI355X a 4-byte gather that
// misses L1 costs a whole L2 request, and the chip sustains about 220 G such
// requests per second, whereas LDS serves scattered 4-byte reads at several
// times that rate.  So x is cut into windows of W = 2^bits columns (at most
// 32768, 128 KB of LDS), the product of every entry is formed in a pass that
// holds one window of x in LDS, and the row sums are formed in a second pass
// that reads the products back in CSR order.
//
// Layout (built once, at bind, in the plan workspace):
//   * row chunks: the rows cut greedily into chunks of at most kXwChunk
//     entries and kXwMaxRows rows; a row longer than kXwChunk entries forms
//     chunks of its own (segments of kXwChunk entries) whose partial sums are
//     added in segment order at the end.  Chunks partition the CSR entries in
//     order.  Run (c, w) = the entries of chunk c in window w, CSR order,
//     padded to a multiple of 8 slots.
//   * chunk-major stream (position in the chunk's CSR order as uint16,
//     0xffff in padding; the products of a call): chunk after chunk, the
//     chunk's runs in window order.  runs[c][w] is where run (c, w) starts,
//     runs[c][nw] the chunk's end.
//   * window-major stream (column within the window as uint16, value):
//     window after window, the window's runs in chunk order.
//
// xw_products_kernel (1024 threads, one window of x in LDS): a piece is the
//   runs of one window over at most kXwPieceRuns consecutive chunks and
//   kXwPiece slots, one contiguous stretch of the window-major stream.  Each
//   thread loads its 4 groups of 8 slots (16-byte loads) before waiting for
//   anything, forms value * x[window + column], finds the group's run by a
//   branchless binary search over the piece's run table in LDS, and stores
//   the 8 products at their chunk-major place.  Every piece of window w runs
//   on XCD w mod 8, so the window's x is read from HBM once and from that
//   XCD's L2 afterwards.
// xw_rows_kernel (256 threads, two workgroups per CU, each taking every
//   grid-th chunk): the chunk's stream slice and row starts are loaded into
//   registers while the previous chunk is being summed; each product is
//   stored in LDS at its CSR position; then thread t adds the products of
//   its slice of about n/256 consecutive entries in order (rows found
//   through a bitmap of row starts and its per-word prefix counts), writes
//   the rows that start and end inside the slice, and one segmented suffix
//   scan over the 256 slices completes the rows that cross slice boundaries.
//   The order of every sum is fixed by the chunk alone, so results are
//   bitwise reproducible.
// xw_split_kernel: y = alpha * (segment partials in order) + beta * y for the
//   rows longer than a chunk.
#include <algorithm>

#include "device_common.h"

namespace spx {

namespace {

constexpr int kXwProdThreads = 1024;
constexpr int kXwWords = kXwChunk / 32;  // row-start bitmap words of a chunk
constexpr uint32_t kXwPad = 0xffffu;     // position of a padding slot
static_assert(kXwChunk % 32 == 0, "chunk bitmap in whole words");
static_assert(kXwChunk < (int)kXwPad && kXwMaxRows <= 32767, "local positions and ranks fit 16 bits");
static_assert(kXwPieceRuns <= kXwProdThreads, "one thread per run in the piece table");
static_assert(kXwMaxWindows <= 256 && kXwPieceRuns < (1 << 23), "piece descriptor packs window and run count");
constexpr int kXwProdGroups = kXwPiece / 8 / kXwProdThreads;  // groups of 8 slots per thread and piece
static_assert(kXwProdGroups * 8 * kXwProdThreads == kXwPiece, "a piece is whole groups per thread");
// registers per thread for one chunk of the row kernel
constexpr int kXwSpanLoads = (kXwChunk + 7 * kXwMaxWindows + 4 * kBlock - 1) / (4 * kBlock);
constexpr int kXwRowLoads = (kXwMaxRows + 1 + kBlock - 1) / kBlock;

// Exclusive sum over the workgroup (NT threads) of one value per thread; `tot`
// receives the wave totals.  Contains one barrier.
template <int NT>
__device__ __forceinline__ int block_exclusive_sum(int v, int* tot) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
        const int t = __shfl_up(incl, k, 64);
        if (lane >= k) incl += t;
    }
    if (lane == 63) tot[w] = incl;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int j = 0; j < NT / 64 - 1; ++j)
        if (j < w) before += tot[j];
    return before + incl - v;
}

// Rank among the chunk's non-empty rows of the row that holds local entry e.
__device__ __forceinline__ int row_rank(const uint32_t* rbits, const int16_t* wpre, int e) {
    const uint32_t m = (2u << (e & 31)) - 1u;  // bits 0..e%32
    return (int)wpre[e >> 5] + __popc(rbits[e >> 5] & m) - 1;
}

struct ChunkScratch {
    int16_t frs[kBlock + 1];  // first row (rank) of each slice, -1 if empty; [kBlock] = -1
    int16_t lrs[kBlock];      // last row of each slice
    float agg_h[4];
    int agg_m[4];
    float cf[5];
};

// Row sums of the n <= kXwChunk products in ps (CSR order), written to
// ysh[rank] for every non-empty row of the chunk.  Thread t owns entries
// [t E, t E + E), E = ceil(n / 256) rounded up to a multiple of 4.
__device__ __forceinline__ void chunk_row_sums(const float* ps, int n, const uint32_t* rbits, const int16_t* wpre,
                                               float* ysh, ChunkScratch& s) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int E = (((n + kBlock - 1) / kBlock) + 3) & ~3;
    const int e0 = min(n, tid * E), e1 = min(n, e0 + E);
    int fr = -1, lr = -1;
    float hsum = 0.0f, tsum = 0.0f;
    if (e0 < e1) {
        int r = row_rank(rbits, wpre, e0);
        fr = r;
        bool head = true;
        float acc = 0.0f;
        for (int e = e0; e < e1; e += 4) {
            // e is a multiple of 4 below n <= kXwChunk: the 16-byte read stays in ps
            const float4 v = *reinterpret_cast<const float4*>(ps + e);
            const uint32_t bw = rbits[e >> 5] >> (e & 31);
            const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (e + j < e1) {
                    if (((bw >> j) & 1u) && e + j > e0) {  // a row starts: the current one is complete here
                        if (head) {
                            hsum = acc;
                            head = false;
                        } else {
                            ysh[r] = acc;  // starts and ends inside the slice
                        }
                        ++r;
                        acc = 0.0f;
                    }
                    acc += vv[j];
                }
            }
        }
        lr = r;
        if (head) hsum = acc;
        tsum = acc;
    }
    s.frs[tid] = (int16_t)fr;
    s.lrs[tid] = (int16_t)lr;
    if (tid == 0) s.frs[kBlock] = -1;
    __syncthreads();
    // segmented suffix scan over slices: C_t = hsum_t + m_t C_{t+1}, where
    // m_t = (slice t is one row) and (slice t + 1 starts inside that row)
    const bool link = lr >= 0 && s.frs[tid + 1] == lr;
    const bool cont = tid > 0 && fr >= 0 && s.lrs[tid - 1] == fr;
    float H = hsum;
    int M = (fr == lr && link) ? 1 : 0;
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
        const float h2 = __shfl_down(H, k, 64);
        const int m2 = __shfl_down(M, k, 64);
        if (lane + k < 64 && M) {
            H += h2;
            M = m2;
        }
    }
    if (lane == 0) {
        s.agg_h[w] = H;
        s.agg_m[w] = M;
    }
    __syncthreads();
    if (tid == 0) {
        float c = 0.0f;
        s.cf[4] = 0.0f;
        for (int b = 3; b >= 0; --b) {
            c = s.agg_m[b] ? s.agg_h[b] + c : s.agg_h[b];
            s.cf[b] = c;
        }
    }
    __syncthreads();
    const float after = s.cf[w + 1];
    const float C = M ? H + after : H;
    float Cn = __shfl_down(C, 1, 64);
    if (lane == 63) Cn = after;
    if (fr >= 0) {
        if (!cont) ysh[fr] = C;                             // the slice's first row starts here
        if (lr != fr) ysh[lr] = link ? tsum + Cn : tsum;    // its last row starts inside the slice
    }
}

__global__ __launch_bounds__(kXwProdThreads) void xw_products_kernel(
    const int4* __restrict__ pieces, const int32_t* __restrict__ runs, int nw, int bits, int64_t cols,
    const float* __restrict__ x, const uint16_t* __restrict__ wcol, const float* __restrict__ wval,
    float* __restrict__ prod) {
    __shared__ __attribute__((aligned(16))) float xs[1 << kXwMaxBits];
    __shared__ int rs[kXwPieceRuns];      // chunk-major start of each run of the piece
    __shared__ int gp[kXwPieceRuns + 1];  // groups of 8 slots before each run
    __shared__ int tot[kXwProdThreads / 64];
    const int4 pc = pieces[blockIdx.x];   // {window | runs << 8, first chunk, window-major start, groups}
    if (pc.x < 0) return;                 // idle slot
    const int tid = threadIdx.x;
    const int w = pc.x & 255, nr = pc.x >> 8, ca = pc.y, src0 = pc.z, G = pc.w;  // 1 <= nr <= kXwPieceRuns
    // the piece's slots: group g = tid + 1024 u holds window-major slots src0 + 8g .. src0 + 8g + 7
    v4u32 k[kXwProdGroups];
    v4f32 a0[kXwProdGroups], a1[kXwProdGroups];
#pragma unroll
    for (int u = 0; u < kXwProdGroups; ++u) {
        const int g = tid + kXwProdThreads * u;
        if (g < G) {
            const int p = src0 + 8 * g;
            k[u] = __builtin_nontemporal_load(reinterpret_cast<const v4u32*>(wcol + p));
            a0[u] = __builtin_nontemporal_load(reinterpret_cast<const v4f32*>(wval + p));
            a1[u] = __builtin_nontemporal_load(reinterpret_cast<const v4f32*>(wval + p + 4));
        } else {
            k[u] = v4u32{0u, 0u, 0u, 0u};
            a0[u] = v4f32{0.0f, 0.0f, 0.0f, 0.0f};
            a1[u] = a0[u];
        }
    }
    int groups = 0;
    if (tid < nr) {
        const int32_t* r = runs + (int64_t)(ca + tid) * (nw + 1) + w;
        const int s = r[0];
        rs[tid] = s;
        groups = (r[1] - s) >> 3;  // runs are whole groups of 8
    }
    const int W = 1 << bits;
    const int64_t c0 = (int64_t)w << bits;
    const int nx = (int)min((int64_t)W, cols - c0);
    const float* __restrict__ xw = x + c0;
    if (nx == W && (reinterpret_cast<uintptr_t>(xw) & 15) == 0) {
        for (int j = tid; j < W / 4; j += kXwProdThreads)
            reinterpret_cast<float4*>(xs)[j] = reinterpret_cast<const float4*>(xw)[j];
    } else {
        for (int j = tid; j < nx; j += kXwProdThreads) xs[j] = xw[j];
    }
    const int ex = block_exclusive_sum<kXwProdThreads>(groups, tot);
    if (tid < nr) gp[tid] = ex;
    if (tid == nr - 1) gp[nr] = ex + groups;  // == G
    __syncthreads();  // x window and run table in LDS
    // group g lies in the last run c with gp[c] <= g (empty runs share their
    // successor's gp); every column read is below nx (padding has column 0)
#pragma unroll
    for (int u = 0; u < kXwProdGroups; ++u) {
        const int g = tid + kXwProdThreads * u;
        int lo = 0;
#pragma unroll
        for (int step = kXwPieceRuns / 2; step > 0; step >>= 1)
            if (lo + step < nr && gp[lo + step] <= g) lo += step;
        v4f32 q0, q1;
        q0.x = a0[u].x * xs[k[u].x & 0xffffu];
        q0.y = a0[u].y * xs[k[u].x >> 16];
        q0.z = a0[u].z * xs[k[u].y & 0xffffu];
        q0.w = a0[u].w * xs[k[u].y >> 16];
        q1.x = a1[u].x * xs[k[u].z & 0xffffu];
        q1.y = a1[u].y * xs[k[u].z >> 16];
        q1.z = a1[u].z * xs[k[u].w & 0xffffu];
        q1.w = a1[u].w * xs[k[u].w >> 16];
        if (g < G) {
            const int d = rs[lo] + 8 * (g - gp[lo]);
            *reinterpret_cast<v4f32*>(prod + d) = q0;
            *reinterpret_cast<v4f32*>(prod + d + 4) = q1;
        }
    }
}

struct XwRowArgs {
    const int4* chunks;
    const int2* chunk_q;
    int n_chunks;
    const float* prod;
    const uint16_t* off;
    const int32_t* ptr;
    float* partials;
    float* y;
    float alpha, beta;
};

__global__ __launch_bounds__(kBlock) void xw_rows_kernel(const XwRowArgs a) {
    __shared__ __attribute__((aligned(16))) float ps[kXwChunk];  // the chunk's products in CSR order
    __shared__ float ysh[kXwMaxRows];                            // row sums by rank of non-empty row
    __shared__ int16_t rp[kXwMaxRows + 1];                       // local row starts
    __shared__ uint32_t rbits[kXwWords];                         // bit e: entry e starts a row
    __shared__ int16_t wpre[kXwWords];                           // row starts before each word
    __shared__ int tot[4];
    __shared__ ChunkScratch sc;
    const int tid = threadIdx.x;

    // one chunk's stream slice (4 slots per load) and row starts, in registers
    v4f32 pv[kXwSpanLoads];
    uint2 po[kXwSpanLoads];
    int rpv[kXwRowLoads];
    auto fetch = [&](int ci) {
        const int4 c = a.chunks[ci];
        const int span = c.y - c.x;  // a multiple of 8
#pragma unroll
        for (int j = 0; j < kXwSpanLoads; ++j) {
            const int f = 4 * tid + 4 * kBlock * j;
            if (f < span) {
                pv[j] = __builtin_nontemporal_load(reinterpret_cast<const v4f32*>(a.prod + c.x + f));
                po[j] = *reinterpret_cast<const uint2*>(a.off + c.x + f);
            } else {
                po[j] = make_uint2(0xffffffffu, 0xffffffffu);
            }
        }
        const int R = c.w < 0 ? 0 : c.w - c.z;  // segments need no row starts
#pragma unroll
        for (int j = 0; j < kXwRowLoads; ++j) {
            const int k = tid + kBlock * j;
            rpv[j] = k <= R && c.w >= 0 ? a.ptr[c.z + k] : 0;
        }
    };

    int ci = blockIdx.x;
    if (ci < a.n_chunks) fetch(ci);
    for (; ci < a.n_chunks; ci += gridDim.x) {
        const int4 c = a.chunks[ci];  // {stream_begin, stream_end, row_begin, row_end or -(partial + 1)}
        const int2 qn = a.chunk_q[ci];
        const int rb = c.z, q0 = qn.x, n = qn.y;
        const bool seg = c.w < 0;  // a segment of one long row
        const int R = seg ? 1 : c.w - rb;
        const int nwords = (n + 31) >> 5;

        // ---- local row starts and the bitmap of row starts
#pragma unroll
        for (int j = 0; j < kXwRowLoads; ++j) {
            const int k = tid + kBlock * j;
            if (k <= R) rp[k] = (int16_t)(seg ? (k == 0 ? 0 : n) : rpv[j] - q0);
        }
        for (int k = tid; k < nwords; k += kBlock) rbits[k] = 0u;
        __syncthreads();
        for (int k = tid; k < R; k += kBlock) {
            const int b0 = rp[k];
            if (rp[k + 1] > b0) atomicOr(&rbits[b0 >> 5], 1u << (b0 & 31));
        }
        // ---- the chunk's products into CSR order; the positions are a
        // permutation of 0..n-1 plus padding, so no two stores meet
#pragma unroll
        for (int j = 0; j < kXwSpanLoads; ++j) {
            const uint32_t o0 = po[j].x & 0xffffu, o1 = po[j].x >> 16, o2 = po[j].y & 0xffffu, o3 = po[j].y >> 16;
            if (o0 != kXwPad) ps[o0] = pv[j].x;
            if (o1 != kXwPad) ps[o1] = pv[j].y;
            if (o2 != kXwPad) ps[o2] = pv[j].z;
            if (o3 != kXwPad) ps[o3] = pv[j].w;
        }
        __syncthreads();
        {  // prefix counts of row starts per bitmap word, two words per thread
            const int k0 = 2 * tid, k1 = 2 * tid + 1;
            const int t0 = k0 < nwords ? __popc(rbits[k0]) : 0;
            const int t1 = k1 < nwords ? __popc(rbits[k1]) : 0;
            const int e0 = block_exclusive_sum<kBlock>(t0 + t1, tot);
            if (k0 < nwords) wpre[k0] = (int16_t)e0;
            if (k1 < nwords) wpre[k1] = (int16_t)(e0 + t0);
        }
        __syncthreads();
        // ---- the next chunk's loads stay in flight through the row sums
        if (ci + (int)gridDim.x < a.n_chunks) fetch(ci + gridDim.x);
        chunk_row_sums(ps, n, rbits, wpre, ysh, sc);
        __syncthreads();
        // ---- outputs
        if (seg) {
            if (tid == 0) a.partials[-c.w - 1] = ysh[0];
        } else {
            for (int k = tid; k < R; k += kBlock) {
                const int b0 = rp[k];
                const float v = rp[k + 1] > b0 ? ysh[row_rank(rbits, wpre, b0)] : 0.0f;
                store_axpby(a.y, rb + k, v, a.alpha, a.beta);
            }
        }
        __syncthreads();  // LDS is reused by the next chunk
    }
}

// One thread per long row: its segment partials added in segment order.
__global__ __launch_bounds__(kBlock) void xw_split_kernel(int n_split_rows, const int4* __restrict__ split_rows,
                                                          const float* __restrict__ partials, float alpha, float beta,
                                                          float* __restrict__ y) {
    const int j = blockIdx.x * kBlock + (int)threadIdx.x;
    if (j >= n_split_rows) return;
    const int4 sr = split_rows[j];  // {row, partial_base, nseg, 0}
    float t = 0.0f;
    for (int k = 0; k < sr.z; ++k) t += partials[sr.y + k];
    store_axpby(y, sr.x, t, alpha, beta);
}

// Bind time: every stream slot starts as padding...
__global__ __launch_bounds__(kBlock) void xw_pad_kernel(int64_t total, uint16_t* __restrict__ wcol,
                                                        float* __restrict__ wval, uint16_t* __restrict__ off) {
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < total; i += (int64_t)gridDim.x * kBlock) {
        wcol[i] = 0;
        wval[i] = 0.0f;
        off[i] = (uint16_t)kXwPad;
    }
}

// ...then workgroup c writes chunk c's entries: the CSR position to the
// chunk-major slot pos[q], column and value to the window-major slot.
__global__ __launch_bounds__(kBlock) void xw_build_kernel(
    const int2* __restrict__ chunk_q, const int32_t* __restrict__ runs, const int32_t* __restrict__ wm_runs, int nw,
    int bits, const int32_t* __restrict__ idx, const float* __restrict__ val, const int32_t* __restrict__ pos,
    uint16_t* __restrict__ wcol, float* __restrict__ wval, uint16_t* __restrict__ off) {
    __shared__ int delta[kXwMaxWindows];  // window-major minus chunk-major start of each run of the chunk
    const int c = blockIdx.x;
    for (int w = threadIdx.x; w < nw; w += kBlock)
        delta[w] = wm_runs[(int64_t)c * nw + w] - runs[(int64_t)c * (nw + 1) + w];
    __syncthreads();
    const int2 qn = chunk_q[c];
    const uint32_t mask = (1u << bits) - 1u;
    for (int k = threadIdx.x; k < qn.y; k += kBlock) {
        const int q = qn.x + k;
        const int p = pos[q];
        const int col = idx[q];
        const int pw = p + delta[col >> bits];
        wcol[pw] = (uint16_t)((uint32_t)col & mask);
        wval[pw] = val[q];
        off[p] = (uint16_t)k;
    }
}

}  // namespace

hipError_t launch_xwin_build(const DirDevice& d, const int32_t* pos, hipStream_t s) {
    if (d.xw_total > 0) {
        const int64_t blocks = std::min<int64_t>((d.xw_total + kBlock - 1) / kBlock, 65536);
        hipLaunchKernelGGL(xw_pad_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, d.xw_total, d.xw_wcol,
                           d.xw_wval, d.xw_off);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (d.xw_n_chunks == 0) return hipSuccess;
    hipLaunchKernelGGL(xw_build_kernel, dim3((unsigned)d.xw_n_chunks), dim3(kBlock), 0, s, d.xw_chunk_q, d.xw_runs,
                       d.xw_wm_runs, d.xw_nw, d.xw_bits, d.idx, d.val, pos, d.xw_wcol, d.xw_wval, d.xw_off);
    return hipGetLastError();
}

hipError_t launch_spmv_xwin(const DirDevice& d, float alpha, const float* x, float beta, float* y, hipStream_t s) {
    if (d.xw_n_pieces > 0) {
        hipLaunchKernelGGL(xw_products_kernel, dim3((unsigned)d.xw_n_pieces), dim3(kXwProdThreads), 0, s,
                           d.xw_pieces, d.xw_runs, d.xw_nw, d.xw_bits, (int64_t)d.cols, x, d.xw_wcol, d.xw_wval,
                           d.xw_prod);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (d.xw_n_chunks > 0) {
        XwRowArgs a{};
        a.chunks = d.xw_chunks;
        a.chunk_q = d.xw_chunk_q;
        a.n_chunks = d.xw_n_chunks;
        a.prod = d.xw_prod;
        a.off = d.xw_off;
        a.ptr = d.ptr;
        a.partials = d.xw_partials;
        a.y = y;
        a.alpha = alpha;
        a.beta = beta;
        hipLaunchKernelGGL(xw_rows_kernel, dim3((unsigned)d.xw_row_grid), dim3(kBlock), 0, s, a);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (d.xw_n_split_rows > 0) {
        hipLaunchKernelGGL(xw_split_kernel, dim3((unsigned)((d.xw_n_split_rows + kBlock - 1) / kBlock)), dim3(kBlock),
                           0, s, d.xw_n_split_rows, d.xw_split_rows, d.xw_partials, alpha, beta, y);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace spx
