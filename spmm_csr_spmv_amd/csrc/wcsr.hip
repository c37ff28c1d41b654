// Windowed compressed rows (WCSR) and the windowed SpMM on MFMA.
//
// The AsyncSparse page §2.2.2: rows are grouped into windows of a fixed
// height; per window the union of its rows' column indices is kept (padding
// columns marked -1) and the values of those columns are stored densely, so
// a row of B is fetched once per window instead of once per entry.  §4: the
// B rows are gathered by all threads of the workgroup into shared memory and
// the window's dense tile is multiplied on the matrix units.
//
// Windows are 64 rows (one wave64 lane per row).  The compressed columns of a
// window are ascending and padded to a multiple of `pad`; values are stored
// column by column: values[q * 64 + r] is row r of the window at compressed
// column q.  Entries that share a position are added in CSR order in fp32,
// starting from the first.
//
// Conversion: one wave per window merges its 64 sorted rows by wave-wide
// minima of the current column (analyze counts, fill writes one compressed
// column of 64 values per round, coalesced); a window of more than 4096
// entries gets a workgroup that marks its columns in an LDS bitmap instead.
//
// SpMM: one workgroup per (window, column tile of C: 32 columns when N <= 32,
// 64 when N <= 64, else 128), one wave per 32 x 32 part of the tile.  Chunks of
// 32 compressed columns: the 32 x 64 slice of values is contiguous, the 32
// gathered B row segments are staged in LDS, and each wave runs
// v_mfma_f32_32x32x2_f32 on its 32 x 32 part of the tile (fp32 in, fp32
// accumulate: the products are the plain fp32 ones of the CSR kernels, only
// the order of the sum differs).  The next chunk is loaded into registers
// while the current one is multiplied.  wcsr_spmm_device runs one workgroup
// per window: with many windows of similar width the dispatcher balances the
// GPU and every output is written once.  For windows of very different
// widths, the task split below cuts the wide ones into tasks, as the page
// does, but adds their parts in a fixed order instead of with atomics.
#include <cstring>
#include <vector>

#include "device_common.h"

namespace spx {

namespace {

constexpr int kNoCol = 0x7fffffff;
constexpr int kWin = 64;  // window height (rows)
constexpr int kKc = 32;   // compressed columns per chunk

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int wave_min_i(int v) {
    v = min(v, __builtin_amdgcn_ds_swizzle(v, (1 << 10) | 0x1f));
    v = min(v, __builtin_amdgcn_ds_swizzle(v, (2 << 10) | 0x1f));
    v = min(v, __builtin_amdgcn_ds_swizzle(v, (4 << 10) | 0x1f));
    v = min(v, __builtin_amdgcn_ds_swizzle(v, (8 << 10) | 0x1f));
    v = min(v, __builtin_amdgcn_ds_swizzle(v, (16 << 10) | 0x1f));
    return min(v, __shfl_xor(v, 32, 64));
}

__device__ __forceinline__ int col_at(const int32_t* __restrict__ idx, int q, int qe, int n) {
    if (q >= qe) return kNoCol;
    const int c = idx[q];
    return (c >= 0 && c < n) ? c : kNoCol;
}

// A window of more than kWideEntries entries is converted by one workgroup
// of its own (wcsr_wide_kernel): the wave merge below takes one dependent
// load per compressed column, so a window of thousands of columns would hold
// the whole conversion for milliseconds.
constexpr int kWideEntries = 4096;
constexpr int kWideThreads = 1024;
constexpr int kWideBits = 19;                        // columns per pass: 2^19, a 64 KB bitmap
constexpr int kWideWords = (1 << kWideBits) / 32;
constexpr int kWideGroups = kWideWords / 8;          // set-bit counts kept per group of 8 words
constexpr int64_t kWideMaxCols = 8LL << kWideBits;   // wider matrices keep the wave merge

__device__ __forceinline__ bool wide_window(const int32_t* __restrict__ ptr, int64_t m, int64_t w, int32_t n) {
    const int64_t r0 = w * kWin, r1 = min(m, r0 + kWin);
    return (int64_t)ptr[r1] - ptr[r0] > kWideEntries && n <= kWideMaxCols;
}

// flags[0] |= 1: a column outside [0, n);  |= 2: a row not sorted by column.
// Four windows per workgroup, one per wave; wide windows are left to
// wcsr_wide_kernel.
__global__ __launch_bounds__(kBlock) void wcsr_analyze_kernel(int64_t m, int32_t n, int64_t nw, int32_t pad,
                                                              const int32_t* __restrict__ ptr,
                                                              const int32_t* __restrict__ idx,
                                                              int32_t* __restrict__ counts, int32_t* __restrict__ flags) {
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= nw || wide_window(ptr, m, w, n)) return;
    const int l = threadIdx.x & 63;
    const int64_t i = w * kWin + l;
    const bool in = i < m;
    int p = in ? ptr[i] : 0;
    const int pe = in ? ptr[i + 1] : 0;
    int bad = 0;
    for (int q = p; q < pe; ++q) {
        const int c = idx[q];
        if (c < 0 || c >= n) bad |= 1;
        if (q > p && c < idx[q - 1]) bad |= 2;
    }
    if (bad) atomicOr(flags, bad);
    int cur = col_at(idx, p, pe, n);
    int count = 0;
    while (true) {
        const int J = wave_min_i(cur);
        if (J == kNoCol) break;
        ++count;
        while (cur == J) cur = col_at(idx, ++p, pe, n);
    }
    if (l == 0) counts[w] = (count + pad - 1) / pad * pad;
}

__global__ __launch_bounds__(kBlock) void wcsr_fill_kernel(int64_t m, int32_t n, int64_t nw,
                                                           const int32_t* __restrict__ ptr,
                                                           const int32_t* __restrict__ idx,
                                                           const float* __restrict__ val,
                                                           const int32_t* __restrict__ window_ptr,
                                                           int32_t* __restrict__ window_col,
                                                           float* __restrict__ values) {
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= nw || wide_window(ptr, m, w, n)) return;
    const int l = threadIdx.x & 63;
    const int64_t i = w * kWin + l;
    const bool in = i < m;
    int p = in ? ptr[i] : 0;
    const int pe = in ? ptr[i + 1] : 0;
    int q = window_ptr[w];
    const int qend = window_ptr[w + 1];
    int cur = col_at(idx, p, pe, n);
    while (true) {
        const int J = wave_min_i(cur);
        if (J == kNoCol) break;
        float v = 0.0f;
        if (cur == J) {
            v = val[p];
            cur = col_at(idx, ++p, pe, n);
            while (cur == J) {
                v = v + val[p];
                cur = col_at(idx, ++p, pe, n);
            }
        }
        if (q < qend) {  // never past the window's range, whatever the input
            if (l == 0) window_col[q] = J;
            values[(int64_t)q * kWin + l] = v;
        }
        ++q;
    }
    for (; q < qend; ++q) {
        if (l == 0) window_col[q] = -1;
        values[(int64_t)q * kWin + l] = 0.0f;
    }
}

// Exclusive prefix sum over the 1024 threads of a workgroup; *total gets the sum.
__device__ int block_exclusive_scan(int v, int* wsum, int* total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int k = 0; k < kWideThreads / 64; ++k) {
            const int u = wsum[k];
            wsum[k] = acc;
            acc += u;
        }
        *total = acc;
    }
    __syncthreads();
    return x - v + wsum[wv];
}

// The window row holding entry e: the r with rps[r] <= e < rps[r + 1]
// (rps[0] <= e < rps[rows]).
__device__ __forceinline__ int entry_row(const int32_t* rps, int rows, int e) {
    int lo = 0, hi = rows;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (rps[mid] <= e) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Rank of column bit (k, bit) among the set bits of the bitmap.
__device__ __forceinline__ int bit_rank(const uint32_t* bm, const int32_t* gp, int k, int bit) {
    int r = gp[k >> 3];
    for (int j = k & ~7; j < k; ++j) r += __popc(bm[j]);
    return r + __popc(bm[k] & ((1u << bit) - 1u));
}

// One workgroup per wide window (the grid covers every window; the others
// exit).  Pass by pass over 2^19 columns, the window's entries set their
// column's bit in an LDS bitmap; the set bits are the window's distinct
// columns in ascending order.  Analyze: their count, rounded up to pad, and
// the same flags as wcsr_analyze_kernel.  Fill: the window's values cleared
// and its columns set to -1 first; then every set bit writes its column at
// its rank, and the first entry of each run of equal columns in a row adds
// the run in CSR order and writes the sum at that rank (the wave merge's
// values, bit for bit).
template <bool FILL>
__global__ __launch_bounds__(kWideThreads) void wcsr_wide_kernel(int64_t m, int32_t n, int32_t pad,
                                                                 const int32_t* __restrict__ ptr,
                                                                 const int32_t* __restrict__ idx,
                                                                 const float* __restrict__ val,
                                                                 int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ flags,
                                                                 const int32_t* __restrict__ window_ptr,
                                                                 int32_t* __restrict__ window_col,
                                                                 float* __restrict__ values) {
    __shared__ uint32_t bm[kWideWords];
    __shared__ int32_t gp[kWideGroups];  // set bits before each group of 8 words
    __shared__ int32_t wsum[kWideThreads / 64];
    __shared__ int32_t pass_total;
    __shared__ int32_t rps[kWin + 1];  // the window's row pointers
    const int64_t w = blockIdx.x;
    if (!wide_window(ptr, m, w, n)) return;
    const int t = threadIdx.x;
    const int64_t r0 = w * kWin;
    const int rows = (int)(min(m, r0 + kWin) - r0);
    if (t <= rows) rps[t] = ptr[r0 + t];
    int q = 0, qend = 0;
    if (FILL) {
        q = window_ptr[w];
        qend = window_ptr[w + 1];
        for (int64_t k = (int64_t)q * kWin + t; k < (int64_t)qend * kWin; k += kWideThreads) values[k] = 0.0f;
        for (int k = q + t; k < qend; k += kWideThreads) window_col[k] = -1;
    }
    __syncthreads();
    const int e0 = rps[0], e1 = rps[rows];
    int bad = 0, done = 0;
    for (int64_t base = 0; base < n; base += 1 << kWideBits) {
        const int64_t lim = min((int64_t)n, base + (1 << kWideBits));
        for (int k = t; k < kWideWords; k += kWideThreads) bm[k] = 0u;
        __syncthreads();
        for (int e = e0 + t; e < e1; e += kWideThreads) {
            const int c = idx[e];
            if (!FILL && base == 0) {
                if (c < 0 || c >= n) bad |= 1;
                if (e > rps[entry_row(rps, rows, e)] && c < idx[e - 1]) bad |= 2;
            }
            if (c >= base && c < lim) atomicOr(&bm[(c - base) >> 5], 1u << (c & 31));
        }
        __syncthreads();
        int c0 = 0, c1 = 0;  // thread t owns groups 2t and 2t + 1
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            c0 += __popc(bm[16 * t + k]);
            c1 += __popc(bm[16 * t + 8 + k]);
        }
        const int excl = block_exclusive_scan(c0 + c1, wsum, &pass_total);
        gp[2 * t] = excl;
        gp[2 * t + 1] = excl + c0;
        __syncthreads();
        if (FILL) {
            for (int k = t; k < kWideWords; k += kWideThreads) {
                uint32_t b = bm[k];
                int r = bit_rank(bm, gp, k, 0);
                while (b) {
                    const int bit = __ffs(b) - 1;
                    b &= b - 1u;
                    const int64_t qq = (int64_t)q + done + r++;
                    if (qq < qend) window_col[qq] = (int)(base + 32 * k + bit);
                }
            }
            for (int e = e0 + t; e < e1; e += kWideThreads) {
                const int c = idx[e];
                if (c < base || c >= lim) continue;
                const int r = entry_row(rps, rows, e);
                const int p0 = rps[r], p1 = rps[r + 1];
                if (e > p0 && idx[e - 1] == c) continue;
                float v = val[e];
                for (int f = e + 1; f < p1 && idx[f] == c; ++f) v = v + val[f];
                const int64_t qq = (int64_t)q + done + bit_rank(bm, gp, (int)((c - base) >> 5), c & 31);
                if (qq < qend) values[qq * kWin + r] = v;
            }
        }
        done += pass_total;
        __syncthreads();  // the next pass clears the bitmap
    }
    if (!FILL) {
        if (bad) atomicOr(flags, bad);
        if (t == 0) counts[w] = (done + pad - 1) / pad * pad;
    }
}

// One chunk of 32 compressed columns in registers.  A workgroup of 4 NT
// threads (one wave per 32 x 32 part) serves a 64 x NT tile of C (NT = 32, 64
// or 128): the 32 x 64 slice of values is 512 float4, the 32 x NT gathered B
// slice 8 NT float4.
template <int NT>
struct Chunk {
    static constexpr int kThreads = 4 * NT;
    static constexpr int kA = 512 / kThreads, kB = 8 * NT / kThreads;
    float4 a[kA], b[kB];
};

template <int NT>
__device__ __forceinline__ void load_chunk(Chunk<NT>& c, int qc, int q1, const int32_t* __restrict__ window_col,
                                           const float* __restrict__ values, const float* __restrict__ B, int64_t ldb,
                                           int n0, int N) {
    using S = Chunk<NT>;
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < S::kA; ++j) {
        const int f = t + S::kThreads * j;  // float4 of the 32 x 64 values slice
        const int k = f >> 4;               // chunk column (16 float4 per column)
        c.a[j] = qc + k < q1 ? *reinterpret_cast<const float4*>(values + (int64_t)(qc + k) * kWin + 4 * (f & 15))
                             : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int j = 0; j < S::kB; ++j) {
        const int f = t + S::kThreads * j;  // float4 of the 32 x NT B slice
        const int k = f / (NT / 4);
        const int col = qc + k < q1 ? window_col[qc + k] : -1;
        const int nc = n0 + 4 * (f % (NT / 4));
        c.b[j] = (col >= 0 && nc < N) ? *reinterpret_cast<const float4*>(B + (int64_t)col * ldb + nc)
                                      : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
}

template <int NT>
__device__ __forceinline__ void store_chunk(const Chunk<NT>& c, float* As, float* Bs) {
    using S = Chunk<NT>;
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < S::kA; ++j) *reinterpret_cast<float4*>(As + 4 * (t + S::kThreads * j)) = c.a[j];
#pragma unroll
    for (int j = 0; j < S::kB; ++j) *reinterpret_cast<float4*>(Bs + 4 * (t + S::kThreads * j)) = c.b[j];
}

// Waves: 2, 4 or 8 (NT = 32, 64, 128); wave v owns rows 32 (v % 2) .. +32
// and columns 32 (v / 2) .. +32 of the tile.  Compressed columns [q0, q1) of
// window w times the B tile starting at column n0, summed chunk by chunk in
// column order.
template <int NT>
__device__ __forceinline__ f32x16 window_tile(int q0, int q1, int n0, const int32_t* __restrict__ window_col,
                                              const float* __restrict__ values, int32_t N,
                                              const float* __restrict__ B, int64_t ldb, float* As, float* Bs) {
    const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wr = 32 * (wv & 1), wc = 32 * (wv >> 1);
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    Chunk<NT> c;
    if (q0 < q1) load_chunk<NT>(c, q0, q1, window_col, values, B, ldb, n0, N);
    for (int qc = q0; qc < q1; qc += kKc) {
        store_chunk<NT>(c, As, Bs);
        __syncthreads();
        if (qc + kKc < q1) load_chunk<NT>(c, qc + kKc, q1, window_col, values, B, ldb, n0, N);
#pragma unroll
        for (int kk = 0; kk < kKc / 2; ++kk) {
            const int k = 2 * kk + (l >> 5);
            const float a = As[k * kWin + wr + (l & 31)];
            const float b = Bs[k * NT + wc + (l & 31)];
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
        }
        __syncthreads();
    }
    return acc;
}

// D layout of the 32 x 32 MFMA: lane l, register r -> row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
__device__ __forceinline__ int tile_row(int r) {
    const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
    return 32 * (wv & 1) + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
}
__device__ __forceinline__ int tile_col(int n0) {
    const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
    return n0 + 32 * (wv >> 1) + (l & 31);
}

template <int NT>
__global__ __launch_bounds__(4 * NT) void wcsr_spmm_kernel(int64_t m, int64_t nw, const int32_t* __restrict__ window_ptr,
                                                           const int32_t* __restrict__ window_col,
                                                           const float* __restrict__ values, int32_t N,
                                                           const float* __restrict__ B, int64_t ldb, float alpha,
                                                           float beta, float* __restrict__ C, int64_t ldc) {
    // As[k][r], Bs[k][c]: chunk column k (32) by window row r (64) / tile column c (NT)
    __shared__ __attribute__((aligned(16))) float As[kKc * kWin];
    __shared__ __attribute__((aligned(16))) float Bs[kKc * NT];
    const int64_t w = blockIdx.x;
    const int n0 = blockIdx.y * NT;
    const f32x16 acc = window_tile<NT>(window_ptr[w], window_ptr[w + 1], n0, window_col, values, N, B, ldb, As, Bs);
    const int col = tile_col(n0);
    if (col >= N) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t row = w * kWin + tile_row(r);
        if (row < m) {
            float* cp = C + row * ldc + col;
            float o = alpha * acc[r];
            if (beta != 0.0f) o = fmaf(beta, *cp, o);
            *cp = o;
        }
    }
}

// ---- task split ([ASYNC] §4.2).  A window of more than `task_cols`
// compressed columns is cut into tasks of task_cols columns (the last one
// shorter), one workgroup each.  Each task of such a window stores its
// partial tile in a slot of its own; a second kernel adds a split window's
// partials in task order and writes C.  The page adds the parts with atomics;
// here the order of the sum is fixed, so results are reproducible.  The
// kernel boundary orders the partial stores before their reads: a
// completion counter inside one kernel would need a device-scope release per
// task (an L2 write-back), which costs more than the second launch.  The
// task table is built on the host, once per matrix (plan_host.cpp).

// One workgroup per (task, column tile).  head = {tasks, slots, -, -} of the
// table: a workgroup past the table's tasks, or every workgroup when the
// table needs more slots than `slots`, writes nothing.
template <int NT>
__global__ __launch_bounds__(4 * NT) void wcsr_task_kernel(int64_t m, const int32_t* __restrict__ head, int64_t slots,
                                                           const int4* __restrict__ tasks, float* __restrict__ partials,
                                                           const int32_t* __restrict__ window_col,
                                                           const float* __restrict__ values, int32_t N,
                                                           const float* __restrict__ B, int64_t ldb, float alpha,
                                                           float beta, float* __restrict__ C, int64_t ldc) {
    __shared__ __attribute__((aligned(16))) float As[kKc * kWin];
    __shared__ __attribute__((aligned(16))) float Bs[kKc * NT];
    if ((int)blockIdx.x >= head[0] || head[1] > slots) return;
    const int4 t = tasks[blockIdx.x];
    const int64_t w = t.x;
    const int n0 = blockIdx.y * NT;
    const f32x16 acc = window_tile<NT>(t.y, t.z, n0, window_col, values, N, B, ldb, As, Bs);
    const int col = tile_col(n0);
    if (col >= N) return;
    if (t.w < 0) {  // the window's only task: as the one-workgroup-per-window kernel
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t row = w * kWin + tile_row(r);
            if (row < m) {
                float* cp = C + row * ldc + col;
                float o = alpha * acc[r];
                if (beta != 0.0f) o = fmaf(beta, *cp, o);
                *cp = o;
            }
        }
    } else {  // slot t.w: 64 rows x N columns, row-major
        float* p = partials + (int64_t)t.w * kWin * N + col;
#pragma unroll
        for (int r = 0; r < 16; ++r) p[(int64_t)tile_row(r) * N] = acc[r];
    }
}

// One workgroup per split window (the grid is a bound: head[3] of them are
// real): C = alpha * (sum of the window's partial tiles in task order) + beta C.
__global__ __launch_bounds__(kBlock) void wcsr_partials_reduce_kernel(int64_t m, const int32_t* __restrict__ head,
                                                                      int64_t slots, const int4* __restrict__ splits,
                                                                      const float* __restrict__ partials, int32_t N,
                                                                      float alpha, float beta, float* __restrict__ C,
                                                                      int64_t ldc) {
    if ((int)blockIdx.x >= head[3] || head[1] > slots) return;
    const int4 sp = splits[blockIdx.x];  // {window, first slot, tasks, 0}
    const int64_t tile = (int64_t)kWin * N;
    const float* p0 = partials + (int64_t)sp.y * tile;
    for (int64_t e = threadIdx.x; e < tile; e += kBlock) {
        const int64_t row = (int64_t)sp.x * kWin + e / N;
        if (row >= m) break;  // e grows: every later element is past m too
        float s = p0[e];
        for (int k = 1; k < sp.z; ++k) s += p0[k * tile + e];
        float* cp = C + row * ldc + e % N;
        float o = alpha * s;
        if (beta != 0.0f) o = fmaf(beta, *cp, o);
        *cp = o;
    }
}

}  // namespace

size_t wcsr_convert_work_bytes(int64_t m) { return 256 + scan_work_bytes((m + kWin - 1) / kWin); }

int csr_to_wcsr_analyze_device(int64_t m, int64_t n, const int32_t* row_ptr, const int32_t* col_idx, int32_t pad,
                               int32_t* window_ptr, void* work, hipStream_t s, int32_t* flags_host) {
    int32_t* flags = static_cast<int32_t*>(work);
    int32_t* sums = reinterpret_cast<int32_t*>(static_cast<char*>(work) + 256);
    const int64_t nw = (m + kWin - 1) / kWin;
    if (launch_fill_i32(flags, 1, 0, s) != hipSuccess || launch_fill_i32(window_ptr, 1, 0, s) != hipSuccess)
        return SP_ERR_HIP;
    if (nw > 0) {
        hipLaunchKernelGGL(wcsr_analyze_kernel, dim3((unsigned)((nw + 3) / 4)), dim3(kBlock), 0, s, m, (int32_t)n, nw,
                           pad, row_ptr, col_idx, window_ptr + 1, flags);
        hipLaunchKernelGGL(wcsr_wide_kernel<false>, dim3((unsigned)nw), dim3(kWideThreads), 0, s, m, (int32_t)n, pad,
                           row_ptr, col_idx, nullptr, window_ptr + 1, flags, nullptr, nullptr, nullptr);
        if (hipGetLastError() != hipSuccess) return SP_ERR_HIP;
        const int rc = scan_inclusive_i32(window_ptr + 1, nw, sums, s);
        if (rc != SP_OK) return rc;
    }
    if (hipMemcpyAsync(flags_host, flags, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess) return SP_ERR_HIP;
    return SP_OK;
}

int csr_to_wcsr_fill_device(int64_t m, int64_t n, const int32_t* row_ptr, const int32_t* col_idx, const float* val,
                            const int32_t* window_ptr, int32_t* window_col, float* values, hipStream_t s) {
    const int64_t nw = (m + kWin - 1) / kWin;
    if (nw == 0) return SP_OK;
    hipLaunchKernelGGL(wcsr_fill_kernel, dim3((unsigned)((nw + 3) / 4)), dim3(kBlock), 0, s, m, (int32_t)n, nw,
                       row_ptr, col_idx, val, window_ptr, window_col, values);
    hipLaunchKernelGGL(wcsr_wide_kernel<true>, dim3((unsigned)nw), dim3(kWideThreads), 0, s, m, (int32_t)n, 1, row_ptr,
                       col_idx, val, nullptr, nullptr, window_ptr, window_col, values);
    return hipGetLastError() == hipSuccess ? SP_OK : SP_ERR_HIP;
}

int wcsr_spmm_device(int64_t m, const int32_t* window_ptr, const int32_t* window_col, const float* values,
                     int32_t N, const float* B, int64_t ldb, float alpha, float beta, float* C, int64_t ldc,
                     hipStream_t s) {
    const int64_t nw = (m + kWin - 1) / kWin;
    if (nw == 0 || N == 0) return SP_OK;
    if (N <= 32) {
        hipLaunchKernelGGL(wcsr_spmm_kernel<32>, dim3((unsigned)nw, 1), dim3(128), 0, s, m, nw, window_ptr, window_col,
                           values, N, B, ldb, alpha, beta, C, ldc);
    } else if (N <= 64) {
        hipLaunchKernelGGL(wcsr_spmm_kernel<64>, dim3((unsigned)nw, 1), dim3(256), 0, s, m, nw, window_ptr, window_col,
                           values, N, B, ldb, alpha, beta, C, ldc);
    } else {
        hipLaunchKernelGGL(wcsr_spmm_kernel<128>, dim3((unsigned)nw, (unsigned)((N + 127) / 128)), dim3(512), 0, s, m,
                           nw, window_ptr, window_col, values, N, B, ldb, alpha, beta, C, ldc);
    }
    return hipGetLastError() == hipSuccess ? SP_OK : SP_ERR_HIP;
}

// Task table in device memory: head {tasks, slots, 0, split windows} (256
// B), splits int4[nw] {window, first slot, tasks, 0}, tasks int4[nw +
// total_cols / task_cols] {window, first column, end column, slot or -1} (a
// bound: a window of c columns has at most 1 + c / task_cols tasks).  Where
// head, splits and tasks start depends on m alone.
namespace {
constexpr size_t kTaskHead = 256;
size_t up256(size_t b) { return (b + 255) / 256 * 256; }
int64_t task_bound(int64_t nw, int64_t total_cols, int32_t task_cols) { return nw + total_cols / task_cols; }
struct TaskTable {
    int32_t* head;
    int4* splits;
    int4* tasks;
};
TaskTable task_table(void* base, int64_t nw) {
    char* p = static_cast<char*>(base);
    return {reinterpret_cast<int32_t*>(p), reinterpret_cast<int4*>(p + kTaskHead),
            reinterpret_cast<int4*>(p + kTaskHead + up256(16 * (size_t)nw))};
}
}  // namespace

size_t wcsr_task_table_bytes(int64_t m, int64_t total_cols, int32_t task_cols) {
    const int64_t nw = (m + kWin - 1) / kWin;
    return kTaskHead + up256(16 * (size_t)nw) + up256(16 * (size_t)task_bound(nw, total_cols, task_cols));
}

// The table is built on the host (spx::host::build_wcsr_tasks) and uploaded.
int wcsr_tasks_build_device(int64_t m, const int32_t* window_ptr, int64_t total_cols, int32_t task_cols, void* table,
                            hipStream_t s, int32_t* head_host) {
    const int64_t nw = (m + kWin - 1) / kWin;
    std::vector<int32_t> wp((size_t)nw + 1);
    if (hipMemcpyAsync(wp.data(), window_ptr, wp.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return SP_ERR_HIP;
    std::vector<host::int4> tasks, splits;
    int32_t slots = 0;
    const int rc = host::build_wcsr_tasks(wp, total_cols, task_cols, tasks, splits, slots);
    if (rc != SP_OK) return rc;
    const size_t tasks_at = kTaskHead + up256(16 * (size_t)nw);
    std::vector<char> img(tasks_at + 16 * tasks.size(), 0);
    const int32_t head[4] = {(int32_t)tasks.size(), slots, 0, (int32_t)splits.size()};
    std::memcpy(img.data(), head, sizeof(head));
    if (!splits.empty()) std::memcpy(img.data() + kTaskHead, splits.data(), 16 * splits.size());
    if (!tasks.empty()) std::memcpy(img.data() + tasks_at, tasks.data(), 16 * tasks.size());
    if (hipMemcpyAsync(table, img.data(), img.size(), hipMemcpyHostToDevice, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return SP_ERR_HIP;
    std::memcpy(head_host, head, sizeof(head));
    return SP_OK;
}

size_t wcsr_spmm_tasks_work_bytes(int64_t nslots, int32_t N) { return (size_t)nslots * kWin * (size_t)N * sizeof(float); }

int wcsr_spmm_tasks_device(int64_t m, const void* table, int64_t ntasks, int64_t nslots, const int32_t* window_col,
                           const float* values, int32_t N, const float* B, int64_t ldb, float alpha, float beta,
                           float* C, int64_t ldc, void* work, hipStream_t s) {
    const int64_t nw = (m + kWin - 1) / kWin;
    if (nw == 0 || N == 0) return SP_OK;
    const TaskTable t = task_table(const_cast<void*>(table), nw);
    const int NT = N <= 32 ? 32 : N <= 64 ? 64 : 128;
    float* partials = static_cast<float*>(work);
    const dim3 grid((unsigned)ntasks, (unsigned)((N + NT - 1) / NT));
    if (NT == 32)
        hipLaunchKernelGGL(wcsr_task_kernel<32>, grid, dim3(128), 0, s, m, t.head, nslots, t.tasks, partials,
                           window_col, values, N, B, ldb, alpha, beta, C, ldc);
    else if (NT == 64)
        hipLaunchKernelGGL(wcsr_task_kernel<64>, grid, dim3(256), 0, s, m, t.head, nslots, t.tasks, partials,
                           window_col, values, N, B, ldb, alpha, beta, C, ldc);
    else
        hipLaunchKernelGGL(wcsr_task_kernel<128>, grid, dim3(512), 0, s, m, t.head, nslots, t.tasks, partials,
                           window_col, values, N, B, ldb, alpha, beta, C, ldc);
    if (hipGetLastError() != hipSuccess) return SP_ERR_HIP;
    // a split window has at least two slots: nslots / 2 bounds the split windows
    if (nslots >= 2) {
        hipLaunchKernelGGL(wcsr_partials_reduce_kernel, dim3((unsigned)(nslots / 2)), dim3(kBlock), 0, s, m, t.head,
                           nslots, t.splits, partials, N, alpha, beta, C, ldc);
        if (hipGetLastError() != hipSuccess) return SP_ERR_HIP;
    }
    return SP_OK;
}

}  // namespace spx
