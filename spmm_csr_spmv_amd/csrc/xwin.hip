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
//   * chunk-major stream (the entry's place in the row kernel's LDS copy of
//     the chunk, as a byte offset: 4 x its position in the chunk's CSR
//     order, a padding slot pointing past the chunk; the products of a
//     call): chunk after chunk, the chunk's runs in window order.  runs[c][w] is where run (c, w) starts,
//     runs[c][nw] the chunk's end.
//   * window-major stream (column within the window as uint16, value):
//     window after window, the window's runs in chunk order.
//   * the run starts in both streams, listed in window-major order, so that
//     the runs of a piece are consecutive entries.
//
// xw_products_kernel (1024 threads, one window of x in LDS, one workgroup
//   per CU): a piece is the runs of one window over at most kXwPieceRuns
//   consecutive chunks and kXwPiece slots, one contiguous stretch of the
//   window-major stream.  The pieces of window w run on XCD w mod 8 (the
//   window's x is read from HBM once, then from that XCD's L2); each
//   workgroup takes a contiguous share of its XCD's pieces, in window order
//   (equal slot counts to within one run, or ending at a nearby window
//   boundary), and refills x only when the window changes.  Each thread holds 4 groups
//   of 8 slots of a piece in registers (16-byte loads, issued while the
//   previous piece is processed), forms value * x[window + column], finds
//   the group's run in the piece's run map in LDS (the first group of each
//   run holds the run's destination; a wave ballot finds the last run start
//   at or before the group), and stores the 8 products at their chunk-major
//   place.
// xw_rows_kernel (256 threads, two workgroups per CU, each taking every
//   grid-th chunk): the chunk's stream slice and row starts are loaded into
//   registers while the previous chunk is being scattered and summed (each
//   register is refilled as soon as its value is consumed); each product is
//   stored in LDS at its CSR position; then thread t adds the products of
//   its slice of about n/256 consecutive entries in order (rows found
//   through a bitmap of row starts and its per-word prefix counts), writes
//   the rows that start and end inside the slice, and one segmented suffix
//   scan over the 256 slices completes the rows that cross slice boundaries.
//   The order of every sum is fixed by the chunk alone, so results are
//   bitwise reproducible.  A chunk that is a segment of a row longer than a
//   chunk stores its sum as that row's partial; the workgroup that stores
//   the row's last partial (an integer arrival counter) adds the partials in
//   segment order, writes y and puts the counter back to zero, so the sum
//   does not depend on which workgroup arrives last.
#include <algorithm>
#include <type_traits>

#include "device_common.h"

namespace spx {

namespace {

constexpr int kXwProdThreads = 1024;
typedef uint32_t v2u32 __attribute__((ext_vector_type(2)));  // 4 stream positions
constexpr int kXwWords = kXwChunk / 32;  // row-start bitmap words of a chunk
constexpr int kNoRun = -2147483647 - 1;  // run map entry of a group that starts no run
constexpr uint32_t kXwSpare = 4u * kXwChunk;  // byte offset of the first spare slot past a chunk
static_assert(kXwChunk % 32 == 0, "chunk bitmap in whole words");
static_assert((kXwChunk + 64) * 4 <= 65536 && kXwMaxRows <= 32767, "LDS byte offsets and ranks fit 16 bits");
static_assert(kXwPieceRuns <= kXwProdThreads, "one thread per run in the piece table");
static_assert(kXwMaxWindows <= 256 && kXwPieceRuns < (1 << 23), "piece descriptor packs window and run count");
constexpr int kXwProdGroups = kXwPiece / 8 / kXwProdThreads;  // groups of 8 slots per thread and piece
static_assert(kXwProdGroups * 8 * kXwProdThreads == kXwPiece, "a piece is whole groups per thread");
// row kernel: threads per workgroup, and registers per thread for one chunk
constexpr int kXwRowThreads = 256;
constexpr int kXwSpanLoads = (kXwChunk + 7 * kXwMaxWindows + 4 * kXwRowThreads - 1) / (4 * kXwRowThreads);
constexpr int kXwRowLoads = (kXwMaxRows + 1 + kXwRowThreads - 1) / kXwRowThreads;
constexpr int kXwWordsPerThread = (kXwWords + kXwRowThreads - 1) / kXwRowThreads;  // prefix count

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

template <int NT>
struct ChunkScratch {
    int16_t frs[NT + 1];  // first row (rank) of each slice, -1 if empty; [NT] = -1
    int16_t lrs[NT];      // last row of each slice
    float agg_h[NT / 64];
    int agg_m[NT / 64];
    float cf[NT / 64 + 1];
};

// Row sums of the n <= kXwChunk products in ps (CSR order), written to
// ysh[rank] for every non-empty row of the chunk, by a workgroup of NT
// threads.  Thread t owns entries [t E, t E + E), E = ceil(n / NT) rounded up
// to a multiple of 4.  ysh holds kXwMaxRows rows and then one slot per lane:
// every entry stores the running sum to the row that ends before it or, when
// no row ends there, to the lane's own slot, so the loop has no branches.
// The first and last rows of a slice may continue in the neighbouring
// slices; their parts are combined by a segmented suffix scan over slices
// and written after it, over anything the loop stored for them.
template <int NT>
__device__ __forceinline__ void chunk_row_sums(const float* ps, int n, const uint32_t* rbits, const int16_t* wpre,
                                               float* ysh, ChunkScratch<NT>& s) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int E = (((n + NT - 1) / NT) + 3) & ~3;
    const int e0 = min(n, tid * E), e1 = min(n, e0 + E);
    int fr = -1, lr = -1;
    float hsum = 0.0f, tsum = 0.0f;
    if (e0 < e1) {
        const int r0 = row_rank(rbits, wpre, e0);
        // the current row's and the lane's sink slot as byte offsets in ysh
        uint32_t rb = 4u * r0;
        const uint32_t sb = 4u * (kXwMaxRows + lane);
        char* const yb = reinterpret_cast<char*>(ysh);
        float acc = 0.0f;
        // one block of nv <= 16 entries from eb: row starts at eb..eb+15
        // (bit j), without entry e0 and past nv; kTail masks the values past
        // nv (a full block reads only its own entries)
        auto block = [&](int eb, int nv, auto tail) {
            constexpr bool kTail = decltype(tail)::value;
            float4 v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[i] = *reinterpret_cast<const float4*>(ps + (kTail ? min(eb + 4 * i, kXwChunk - 4) : eb + 4 * i));
            const int wd = eb >> 5, sh = eb & 31;
            const uint32_t lo = rbits[wd], hi = rbits[min(wd + 1, kXwWords - 1)];
            uint32_t m = (lo >> sh) | (sh ? hi << (32 - sh) : 0u);
            m &= (kTail ? ((1u << nv) - 1u) : 0xffffu) & (eb == e0 ? ~1u : ~0u);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float vv[4] = {!kTail || 4 * i + 0 < nv ? v[i].x : 0.0f, !kTail || 4 * i + 1 < nv ? v[i].y : 0.0f,
                                     !kTail || 4 * i + 2 < nv ? v[i].z : 0.0f, !kTail || 4 * i + 3 < nv ? v[i].w : 0.0f};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // a row starts here: the current one is complete (kept in LDS)
                    const bool st = (m & (1u << (4 * i + j))) != 0u;
                    *reinterpret_cast<float*>(yb + (st ? rb : sb)) = acc;
                    rb += st ? 4u : 0u;
                    acc = st ? vv[j] : acc + vv[j];
                }
            }
        };
        int eb = e0;
        for (; eb + 16 <= e1; eb += 16) block(eb, 16, std::false_type{});
        if (eb < e1) block(eb, e1 - eb, std::true_type{});
        const int r = (int)(rb >> 2);
        fr = r0;
        lr = r;
        // the first row's part in this slice: stored in the loop if that row
        // ended inside the slice (its final value is written after the scan)
        hsum = r > r0 ? ysh[r0] : acc;
        tsum = acc;
    }
    s.frs[tid] = (int16_t)fr;
    s.lrs[tid] = (int16_t)lr;
    if (tid == 0) s.frs[NT] = -1;
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
        s.cf[NW] = 0.0f;
        for (int b = NW - 1; b >= 0; --b) {
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

// Loads of one piece for one thread: its groups of 8 window-major slots
// (16-byte loads) and its entry of the piece's run table.
struct PieceRegs {
    v4u32 k[kXwProdGroups];
    v4f32 a0[kXwProdGroups], a1[kXwProdGroups];
    int run_start, run_groups, run_first;  // chunk-major start, groups, groups of the piece before it
};

__device__ __forceinline__ void group_fetch(const int4& pc, int u, const uint16_t* __restrict__ wcol,
                                            const float* __restrict__ wval, PieceRegs& r) {
    const int g = threadIdx.x + kXwProdThreads * u;
    if (g < pc.w) {
        const int p = pc.z + 8 * g;
        r.k[u] = __builtin_nontemporal_load(reinterpret_cast<const v4u32*>(wcol + p));
        r.a0[u] = __builtin_nontemporal_load(reinterpret_cast<const v4f32*>(wval + p));
        r.a1[u] = __builtin_nontemporal_load(reinterpret_cast<const v4f32*>(wval + p + 4));
    } else {
        r.k[u] = v4u32{0u, 0u, 0u, 0u};
        r.a0[u] = v4f32{0.0f, 0.0f, 0.0f, 0.0f};
        r.a1[u] = r.a0[u];
    }
}

__device__ __forceinline__ void runs_fetch(const int4& pc, const int2* __restrict__ wm_tab, int n_chunks,
                                           PieceRegs& r) {
    const int tid = threadIdx.x;
    const int w = pc.x & 255, nr = pc.x >> 8, ca = pc.y;
    r.run_start = 0;
    r.run_groups = 0;
    r.run_first = 0;
    if (tid < nr) {
        // the piece's runs are consecutive in the window-major table, and so
        // are their stretches of the window-major stream (runs are whole
        // groups of 8)
        const int64_t i = (int64_t)w * n_chunks + ca + tid;
        const int2 t = wm_tab[i];
        r.run_start = t.x;
        r.run_groups = (wm_tab[i + 1].y - t.y) >> 3;
        r.run_first = (t.y - pc.z) >> 3;
    }
}

// One workgroup per CU (grid 8 x 32): workgroup b takes the pieces
// [ranges[b].x, ranges[b].y), all of XCD b mod 8 and in window order, so x is
// refilled only when the window changes; the next piece's loads are issued
// before the current piece's products are formed.
__global__ __launch_bounds__(kXwProdThreads) void xw_products_kernel(
    const int4* __restrict__ pieces, const int2* __restrict__ ranges, const int2* __restrict__ wm_tab,
    int n_chunks, int bits, int64_t cols, const float* __restrict__ x, const uint16_t* __restrict__ wcol,
    const float* __restrict__ wval, float* __restrict__ prod) {
    constexpr int kGroups = kXwProdGroups * kXwProdThreads;  // groups of 8 slots per piece
    __shared__ __attribute__((aligned(16))) float xs[1 << kXwMaxBits];
    // run map of the piece: for the first group g of each non-empty run,
    // base[g] = (chunk-major start of the run) - 8 g, so that group g' of that
    // run goes to base[g] + 8 g'; kNoRun elsewhere.  carry[b] = the base of
    // the run that holds group 64 b.
    __shared__ int base[kGroups];
    __shared__ int carry[kGroups / 64];
    const int2 rg = ranges[blockIdx.x];
    if (rg.x >= rg.y) return;
    const int tid = threadIdx.x;
    const int W = 1 << bits;
    PieceRegs cur;
    {
        const int4 p0 = pieces[rg.x];
#pragma unroll
        for (int u = 0; u < kXwProdGroups; ++u) group_fetch(p0, u, wcol, wval, cur);
        runs_fetch(p0, wm_tab, n_chunks, cur);
    }
#pragma unroll
    for (int u = 0; u < kXwProdGroups; ++u) base[tid + kXwProdThreads * u] = kNoRun;  // each thread reads and
                                                                                       // clears its own entries
    int loaded = -1;  // window held in xs
    for (int pi = rg.x; pi < rg.y; ++pi) {
        const int4 pc = pieces[pi];  // {window | runs << 8, first chunk, window-major start, groups}
        const int w = pc.x & 255, nr = pc.x >> 8, G = pc.w;  // 1 <= nr <= kXwPieceRuns
        __syncthreads();  // the previous piece is done with xs, base and carry
        if (w != loaded) {
            const int64_t c0 = (int64_t)w << bits;
            const int nx = (int)min((int64_t)W, cols - c0);
            const float* __restrict__ xw = x + c0;
            if (nx == W && (reinterpret_cast<uintptr_t>(xw) & 15) == 0) {
                for (int j = tid; j < W / 4; j += kXwProdThreads)
                    reinterpret_cast<float4*>(xs)[j] = reinterpret_cast<const float4*>(xw)[j];
            } else {
                for (int j = tid; j < nx; j += kXwProdThreads) xs[j] = xw[j];
            }
            loaded = w;
        }
        if (tid < nr && cur.run_groups > 0) {
            const int ex = cur.run_first;
            const int b0 = cur.run_start - 8 * ex;
            base[ex] = b0;
            for (int b = (ex + 63) >> 6; 64 * b < ex + cur.run_groups; ++b) carry[b] = b0;
        }
        __syncthreads();  // x window and run map in LDS
        // the next piece's loads go into the registers as they are consumed
        const bool more = pi + 1 < rg.y;
        const int4 pn = more ? pieces[pi + 1] : make_int4(0, 0, 0, 0);
        if (more) runs_fetch(pn, wm_tab, n_chunks, cur);
        // group g lies in the last run that starts at or before it: the
        // wave's 64 lanes hold one 64-group block, so that run is the last
        // marked lane up to this one, else the run that crosses into the
        // block; every column read is below the window's width (padding has
        // column 0)
        const uint64_t upto = (2ull << (tid & 63)) - 1ull;  // lanes 0 .. this lane
#pragma unroll
        for (int u = 0; u < kXwProdGroups; ++u) {
            const int g = tid + kXwProdThreads * u;
            const int mk = base[g];
            base[g] = kNoRun;  // clear for the next piece (read by no other thread)
            const uint64_t starts = __ballot(mk != kNoRun) & upto;
            const int src = starts ? 63 - __clzll(starts) : 0;
            const int from_lane = __shfl(mk, src, 64);
            const int b0 = starts ? from_lane : carry[g >> 6];
            v4f32 q0, q1;
            q0.x = cur.a0[u].x * xs[cur.k[u].x & 0xffffu];
            q0.y = cur.a0[u].y * xs[cur.k[u].x >> 16];
            q0.z = cur.a0[u].z * xs[cur.k[u].y & 0xffffu];
            q0.w = cur.a0[u].w * xs[cur.k[u].y >> 16];
            q1.x = cur.a1[u].x * xs[cur.k[u].z & 0xffffu];
            q1.y = cur.a1[u].y * xs[cur.k[u].z >> 16];
            q1.z = cur.a1[u].z * xs[cur.k[u].w & 0xffffu];
            q1.w = cur.a1[u].w * xs[cur.k[u].w >> 16];
            if (more) group_fetch(pn, u, wcol, wval, cur);
            if (g < G) {
                const int d = b0 + 8 * g;
                *reinterpret_cast<v4f32*>(prod + d) = q0;
                *reinterpret_cast<v4f32*>(prod + d + 4) = q1;
            }
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
    const int4* split_rows;  // {row, partial_base, nseg, 0} of each row longer than a chunk
    float* partials;
    int32_t* counters;       // arrival counter of each such row (zero between calls)
    float* y;
    float alpha, beta;
};

__global__ __launch_bounds__(kXwRowThreads) void xw_rows_kernel(const XwRowArgs a) {
    // the chunk's products in CSR order, then one slot per lane that takes the padding
    __shared__ __attribute__((aligned(16))) float ps[kXwChunk + 64];
    __shared__ float ysh[kXwMaxRows + 64];                       // row sums by rank of non-empty row, lane slots
    __shared__ int16_t rp[kXwMaxRows + 1];                       // local row starts
    __shared__ uint32_t rbits[kXwWords + 64];                    // bit e: entry e starts a row; lane words
    __shared__ int16_t wpre[kXwWords];                           // row starts before each word
    __shared__ int tot[kXwRowThreads / 64];
    __shared__ ChunkScratch<kXwRowThreads> sc;
    const int tid = threadIdx.x;

    // one chunk's stream slice (4 slots per load) and row starts, in registers
    v4f32 pv[kXwSpanLoads];
    uint2 po[kXwSpanLoads];
    int rpv[kXwRowLoads];
    // slot j of chunk c: stream slots 4 tid + 4 NT j .. + 3; row start k = tid + NT j
    auto fetch_slot = [&](const int4& c, int j) {
        const int f = 4 * tid + 4 * kXwRowThreads * j;
        if (f < c.y - c.x) {  // the span is a multiple of 8
            pv[j] = __builtin_nontemporal_load(reinterpret_cast<const v4f32*>(a.prod + c.x + f));
            const v2u32 o = __builtin_nontemporal_load(reinterpret_cast<const v2u32*>(a.off + c.x + f));
            po[j] = make_uint2(o.x, o.y);
        } else {
            po[j] = make_uint2(kXwSpare | (kXwSpare << 16), kXwSpare | (kXwSpare << 16));  // past the chunk
        }
    };
    auto fetch_rows = [&](const int4& c) {
        const int R = c.w < 0 ? 0 : c.w - c.z;  // segments need no row starts
#pragma unroll
        for (int j = 0; j < kXwRowLoads; ++j) {
            const int k = tid + kXwRowThreads * j;
            rpv[j] = k <= R && c.w >= 0 ? a.ptr[c.z + k] : 0;
        }
    };

    int ci = blockIdx.x;
    // chunk descriptors {stream_begin, stream_end, row_begin or long row,
    // row_end or -(partial + 1)} and {first entry, entries}, read one chunk ahead
    int4 c_next = make_int4(0, 0, 0, -1);
    int2 q_next = make_int2(0, 0);
    if (ci < a.n_chunks) {
        c_next = a.chunks[ci];
        q_next = a.chunk_q[ci];
#pragma unroll
        for (int j = 0; j < kXwSpanLoads; ++j) fetch_slot(c_next, j);
        fetch_rows(c_next);
    }
    for (; ci < a.n_chunks; ci += gridDim.x) {
        const int4 c = c_next;
        const int2 qn = q_next;
        // the next chunk's loads go into the registers as soon as they are consumed
        const bool more = ci + (int)gridDim.x < a.n_chunks;
        const int4 cn = more ? a.chunks[ci + gridDim.x] : make_int4(0, 0, 0, -1);
        if (more) q_next = a.chunk_q[ci + gridDim.x];
        c_next = cn;
        const int rb = c.z, q0 = qn.x, n = qn.y;
        const bool seg = c.w < 0;  // a segment of one long row
        const int R = seg ? 1 : c.w - rb;
        const int nwords = (n + 31) >> 5;

        // ---- local row starts and the bitmap of row starts
#pragma unroll
        for (int j = 0; j < kXwRowLoads; ++j) {
            const int k = tid + kXwRowThreads * j;
            if (k <= R) rp[k] = (int16_t)(seg ? (k == 0 ? 0 : n) : rpv[j] - q0);
        }
        if (more) fetch_rows(cn);
        for (int k = tid; k < nwords; k += kXwRowThreads) rbits[k] = 0u;
        __syncthreads();
        {  // mark the first entry of every non-empty row (reads first, then the atomics)
            int b0[kXwRowLoads], b1[kXwRowLoads];
#pragma unroll
            for (int j = 0; j < kXwRowLoads; ++j) {
                const int k = tid + kXwRowThreads * j;
                b0[j] = k < R ? rp[k] : 0;
                b1[j] = k < R ? rp[k + 1] : 0;
            }
#pragma unroll
            for (int j = 0; j < kXwRowLoads; ++j)
                atomicOr(&rbits[b1[j] > b0[j] ? b0[j] >> 5 : kXwWords + (tid & 63)], 1u << (b0[j] & 31));
        }
        // ---- the chunk's products into CSR order: the stream holds each
        // slot's byte offset in ps, a permutation of the chunk's n places
        // plus padding slots, which point to the 64 spare slots past them
        char* const psb = reinterpret_cast<char*>(ps);
        __builtin_amdgcn_s_setprio(3);  // issue the next chunk's loads ahead of the other workgroup's sums
#pragma unroll
        for (int j = 0; j < kXwSpanLoads; ++j) {
            *reinterpret_cast<float*>(psb + (po[j].x & 0xffffu)) = pv[j].x;
            *reinterpret_cast<float*>(psb + (po[j].x >> 16)) = pv[j].y;
            *reinterpret_cast<float*>(psb + (po[j].y & 0xffffu)) = pv[j].z;
            *reinterpret_cast<float*>(psb + (po[j].y >> 16)) = pv[j].w;
            if (more) fetch_slot(cn, j);
        }
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();
        {  // prefix counts of row starts per bitmap word, consecutive words per thread
            int cnt[kXwWordsPerThread], sum = 0;
#pragma unroll
            for (int j = 0; j < kXwWordsPerThread; ++j) {
                const int k = kXwWordsPerThread * tid + j;
                cnt[j] = k < nwords ? __popc(rbits[k]) : 0;
                sum += cnt[j];
            }
            int e = block_exclusive_sum<kXwRowThreads>(sum, tot);
#pragma unroll
            for (int j = 0; j < kXwWordsPerThread; ++j) {
                const int k = kXwWordsPerThread * tid + j;
                if (k < nwords) wpre[k] = (int16_t)e;
                e += cnt[j];
            }
        }
        __syncthreads();
        chunk_row_sums(ps, n, rbits, wpre, ysh, sc);
        __syncthreads();
        // ---- outputs
        if (seg) {
            if (tid == 0) {
                const int4 sr = a.split_rows[c.z];
                atomic_store_f(a.partials + (-c.w - 1), ysh[0]);
                const int arrived =
                    __hip_atomic_fetch_add(a.counters + c.z, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
                if (arrived == sr.z - 1) {
                    float t = 0.0f;
                    for (int k = 0; k < sr.z; ++k) t += atomic_load_f(a.partials + sr.y + k);
                    store_axpby(a.y, sr.x, t, a.alpha, a.beta);
                    __hip_atomic_store(a.counters + c.z, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        } else {
            float v[kXwRowLoads];
#pragma unroll
            for (int j = 0; j < kXwRowLoads; ++j) {
                const int k = tid + kXwRowThreads * j;
                const int b0 = k < R ? rp[k] : 0;
                const bool ne = k < R && rp[k + 1] > b0;
                v[j] = ne ? ysh[row_rank(rbits, wpre, b0)] : 0.0f;
            }
#pragma unroll
            for (int j = 0; j < kXwRowLoads; ++j) {
                const int k = tid + kXwRowThreads * j;
                if (k < R) store_axpby(a.y, rb + k, v[j], a.alpha, a.beta);
            }
        }
        __syncthreads();  // LDS is reused by the next chunk
    }

}

// Bind time: every stream slot starts as padding...
__global__ __launch_bounds__(kBlock) void xw_pad_kernel(int64_t total, uint16_t* __restrict__ wcol,
                                                        float* __restrict__ wval, uint16_t* __restrict__ off) {
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < total; i += (int64_t)gridDim.x * kBlock) {
        wcol[i] = 0;
        wval[i] = 0.0f;
        off[i] = (uint16_t)(4 * (kXwChunk + (int)(i & 63)));  // one of the 64 spare slots
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
        off[p] = (uint16_t)(4 * k);
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
        hipLaunchKernelGGL(xw_products_kernel, dim3((unsigned)kXwProdGrid), dim3(kXwProdThreads), 0, s,
                           d.xw_pieces, d.xw_prod_ranges, d.xw_wm_tab, d.xw_n_chunks, d.xw_bits, (int64_t)d.cols, x,
                           d.xw_wcol, d.xw_wval, d.xw_prod);
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
        a.split_rows = d.xw_split_rows;
        a.partials = d.xw_partials;
        a.counters = d.xw_counters;
        a.y = y;
        a.alpha = alpha;
        a.beta = beta;
        hipLaunchKernelGGL(xw_rows_kernel, dim3((unsigned)d.xw_row_grid), dim3(kXwRowThreads), 0, s, a);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace spx
