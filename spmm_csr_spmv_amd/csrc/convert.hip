// Format conversions on the GPU: COO -> CSR and CSR -> CSC.
//
// 「稀疏矩阵存储格式…」 §3 describes COO -> CSR as a per-row count (one
// histogram pass), a prefix sum giving row_ptr, and moving column/value into
// each row's range.  「CUDA LSMR 专栏（二）」 §4 builds the CSC once, as the CSR
// of A^T, by the same counting transposition.
//
// The counting scatter uses integer atomics, so the order it leaves inside a
// segment depends on timing.  To make the result unique, every entry carries
// a 64-bit key that is unique within its segment and orders it the way the
// format requires; each segment is then sorted by key:
//   COO -> CSR : key = (col << 32) | input position   (by column, ties by input order)
//   CSR -> CSC : key = (row << 32) | CSR position      (by row, ties by CSR order)
// Segments of length 2..64 are sorted by one wave (rank by comparison),
// longer ones by one workgroup (bitonic sort of 4096-key chunks in LDS, then
// merge passes in global memory where each key finds its place by binary
// search in the partner run).
#include "device_common.h"

#include <vector>

namespace spx {

namespace {

constexpr int kScanTile = 2048;  // elements scanned per workgroup (8 per thread)
constexpr int kChunk = 4096;     // keys sorted in LDS at once
constexpr int kSmallSeg = 64;    // segments up to this length are sorted by one wave

enum Misc { kErr = 0, kCntSmall = 1, kCntLarge = 2, kMaxLen = 3, kMiscWords = 16 };

__global__ __launch_bounds__(kBlock) void fill_i32(int32_t* p, int64_t n, int32_t v) {
    for (int64_t i = blockIdx.x * (int64_t)kBlock + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBlock) p[i] = v;
}

// counts[r + 1] += 1 for every valid (r, c); flags invalid entries.
__global__ __launch_bounds__(kBlock) void coo_count(int64_t nnz, const int32_t* __restrict__ row,
                                                    const int32_t* __restrict__ col, int32_t m, int32_t n,
                                                    int32_t* __restrict__ counts1, int32_t* __restrict__ misc) {
    for (int64_t i = blockIdx.x * (int64_t)kBlock + threadIdx.x; i < nnz; i += (int64_t)gridDim.x * kBlock) {
        const int32_t r = row[i], c = col[i];
        if (r < 0 || r >= m || c < 0 || c >= n) {
            atomicOr(misc + kErr, 1);
        } else {
            atomicAdd(counts1 + r, 1);
        }
    }
}

__global__ __launch_bounds__(kBlock) void col_count(int64_t nnz, const int32_t* __restrict__ col, int32_t n,
                                                    int32_t* __restrict__ counts1, int32_t* __restrict__ misc) {
    for (int64_t i = blockIdx.x * (int64_t)kBlock + threadIdx.x; i < nnz; i += (int64_t)gridDim.x * kBlock) {
        const int32_t c = col[i];
        if (c < 0 || c >= n) {
            atomicOr(misc + kErr, 1);
        } else {
            atomicAdd(counts1 + c, 1);
        }
    }
}

// ---- inclusive scan of int32 in place (three passes) -----------------------
__device__ __forceinline__ int32_t block_inclusive_scan(int32_t v, int32_t* sh, int32_t& total) {
    // sh: kBlock ints
    const int tid = threadIdx.x;
    sh[tid] = v;
    __syncthreads();
    for (int off = 1; off < kBlock; off <<= 1) {
        const int32_t t = tid >= off ? sh[tid - off] : 0;
        __syncthreads();
        sh[tid] += t;
        __syncthreads();
    }
    const int32_t r = sh[tid];
    total = sh[kBlock - 1];
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kBlock) void scan_tiles(int32_t* __restrict__ a, int64_t n, int32_t* __restrict__ sums) {
    __shared__ int32_t sh[kBlock];
    const int64_t base = blockIdx.x * (int64_t)kScanTile + threadIdx.x * 8;
    int32_t v[8];
    int32_t run = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        v[j] = base + j < n ? a[base + j] : 0;
        run += v[j];
        v[j] = run;
    }
    int32_t total;
    const int32_t incl = block_inclusive_scan(run, sh, total);
    const int32_t excl = incl - run;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (base + j < n) a[base + j] = v[j] + excl;
    if (threadIdx.x == 0) sums[blockIdx.x] = total;
}

__global__ __launch_bounds__(kBlock) void scan_sums(int32_t* __restrict__ sums, int64_t ntiles) {
    __shared__ int32_t sh[kBlock];
    int32_t carry = 0;
    for (int64_t b = 0; b < ntiles; b += kBlock) {
        const int64_t i = b + threadIdx.x;
        const int32_t v = i < ntiles ? sums[i] : 0;
        int32_t total;
        const int32_t incl = block_inclusive_scan(v, sh, total);
        if (i < ntiles) sums[i] = incl + carry;
        carry += total;
    }
}

__global__ __launch_bounds__(kBlock) void scan_add(int32_t* __restrict__ a, int64_t n, const int32_t* __restrict__ sums) {
    if (blockIdx.x == 0) return;
    const int32_t add = sums[blockIdx.x - 1];
    const int64_t base = blockIdx.x * (int64_t)kScanTile;
    for (int j = threadIdx.x; j < kScanTile; j += kBlock)
        if (base + j < n) a[base + j] += add;
}

// ---- segment classification -------------------------------------------------
// cursor[s] = ptr[s]; segments of length 2..64 go to `small`, longer ones to
// `large`; tracks the longest segment.
__global__ __launch_bounds__(kBlock) void classify(int32_t nseg, const int32_t* __restrict__ ptr,
                                                   int32_t* __restrict__ cursor, int32_t* __restrict__ small,
                                                   int32_t* __restrict__ large, int32_t* __restrict__ misc) {
    // One atomic per wave and list: the wave's lanes take consecutive slots
    // (list order does not matter, every listed segment is sorted on its own).
    const int lane = threadIdx.x & 63;
    const uint64_t below = (1ull << lane) - 1;
    for (int32_t s0 = blockIdx.x * kBlock; s0 < nseg; s0 += gridDim.x * kBlock) {
        const int32_t s = s0 + threadIdx.x;
        const bool in = s < nseg;
        const int32_t b = in ? ptr[s] : 0, len = in ? ptr[s + 1] - b : 0;
        if (in) cursor[s] = b;
        const bool is_small = len >= 2 && len <= kSmallSeg, is_large = len > kSmallSeg;
        const uint64_t ms = __ballot(is_small), ml = __ballot(is_large);
        int32_t base_s = 0, base_l = 0;
        if (lane == 0) {
            if (ms) base_s = atomicAdd(misc + kCntSmall, (int)__popcll(ms));
            if (ml) base_l = atomicAdd(misc + kCntLarge, (int)__popcll(ml));
        }
        base_s = __shfl(base_s, 0, 64);
        base_l = __shfl(base_l, 0, 64);
        if (is_small) small[base_s + __popcll(ms & below)] = s;
        if (is_large) large[base_l + __popcll(ml & below)] = s;
        int32_t mx = len;
        for (int off = 32; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off, 64));
        if (lane == 0 && mx > 0) atomicMax(misc + kMaxLen, mx);
    }
}

// ---- keyed scatters ---------------------------------------------------------
__global__ __launch_bounds__(kBlock) void coo_scatter(int64_t nnz, const int32_t* __restrict__ row,
                                                      const int32_t* __restrict__ col, int32_t* __restrict__ cursor,
                                                      uint64_t* __restrict__ keys) {
    for (int64_t i = blockIdx.x * (int64_t)kBlock + threadIdx.x; i < nnz; i += (int64_t)gridDim.x * kBlock) {
        const int32_t p = atomicAdd(cursor + row[i], 1);
        keys[p] = ((uint64_t)(uint32_t)col[i] << 32) | (uint64_t)i;
    }
}

// Entry p of the CSR belongs to the last row r with row_ptr[r] <= p.
__device__ __forceinline__ int32_t row_of(const int32_t* __restrict__ row_ptr, int32_t m, int32_t p) {
    int32_t lo = 0, hi = m - 1;
    while (lo < hi) {
        const int32_t mid = lo + (hi - lo + 1) / 2;
        if (row_ptr[mid] <= p) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(kBlock) void csr_scatter(int64_t nnz, const int32_t* __restrict__ row_ptr, int32_t m,
                                                      const int32_t* __restrict__ col, int32_t* __restrict__ cursor,
                                                      uint64_t* __restrict__ keys) {
    for (int64_t p = blockIdx.x * (int64_t)kBlock + threadIdx.x; p < nnz; p += (int64_t)gridDim.x * kBlock) {
        const int32_t r = row_of(row_ptr, m, (int32_t)p);
        const int32_t q = atomicAdd(cursor + col[p], 1);
        keys[q] = ((uint64_t)(uint32_t)r << 32) | (uint64_t)p;
    }
}

// ---- segment sorts ------------------------------------------------------------
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
    const int lo = __shfl((int)(uint32_t)v, src, 64);
    const int hi = __shfl((int)(uint32_t)(v >> 32), src, 64);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// One wave per segment of 2..64 keys: rank = number of smaller keys (keys are unique).
__global__ __launch_bounds__(kBlock) void sort_small(const int32_t* __restrict__ list, const int32_t* __restrict__ misc,
                                                     const int32_t* __restrict__ ptr, uint64_t* __restrict__ keys) {
    const int32_t count = misc[kCntSmall];
    const int32_t wv = blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
    if (wv >= count) return;
    const int lane = threadIdx.x & 63;
    const int32_t s = list[wv];
    const int32_t b = ptr[s], len = ptr[s + 1] - b;
    const uint64_t key = lane < len ? keys[b + lane] : ~0ull;
    int rank = 0;
    for (int i = 0; i < len; ++i) rank += shfl_u64(key, i) < key ? 1 : 0;
    if (lane < len) keys[b + rank] = key;
}

// Bitonic sort of sh[0..P) (P a power of two, <= kChunk), ascending.
__device__ void bitonic_lds(uint64_t* sh, int P) {
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < P; i += kBlock) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const uint64_t a = sh[i], c = sh[ixj];
                    const bool up = (i & k) == 0;
                    if ((a > c) == up) {
                        sh[i] = c;
                        sh[ixj] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
}

// Number of keys in run[0..n) smaller than key.
__device__ __forceinline__ int32_t lower_bound_u64(const uint64_t* __restrict__ run, int32_t n, uint64_t key) {
    int32_t lo = 0, hi = n;
    while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (run[mid] < key) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// One workgroup per segment longer than 64 keys.
__global__ __launch_bounds__(kBlock) void sort_large(const int32_t* __restrict__ list, const int32_t* __restrict__ ptr,
                                                     uint64_t* __restrict__ keys, uint64_t* __restrict__ tmp) {
    __shared__ uint64_t sh[kChunk];
    const int32_t s = list[blockIdx.x];
    const int32_t b = ptr[s], len = ptr[s + 1] - b;
    uint64_t* seg = keys + b;
    // 1. sort every chunk of kChunk keys in LDS
    for (int32_t c0 = 0; c0 < len; c0 += kChunk) {
        const int32_t n = len - c0 < kChunk ? len - c0 : kChunk;
        int P = 2;
        while (P < n) P <<= 1;
        for (int i = threadIdx.x; i < P; i += kBlock) sh[i] = i < n ? seg[c0 + i] : ~0ull;
        __syncthreads();
        bitonic_lds(sh, P);
        for (int i = threadIdx.x; i < n; i += kBlock) seg[c0 + i] = sh[i];
        __syncthreads();
    }
    // 2. merge runs of width w, 2w, ... until one run covers the segment
    uint64_t* src = seg;
    uint64_t* dst = tmp + b;
    for (int32_t w = kChunk; w < len; w <<= 1) {
        for (int32_t e = threadIdx.x; e < len; e += kBlock) {
            const int32_t run = e / w;
            const int32_t pair0 = (run & ~1) * w;           // start of the left run of the pair
            const int32_t own0 = run * w;
            const bool left = (run & 1) == 0;
            const int32_t p0 = left ? own0 + w : pair0;     // partner run start
            int32_t pn = left ? (len - p0 < w ? len - p0 : w) : w;
            if (pn < 0) pn = 0;
            const uint64_t key = src[e];
            const int32_t rank = pn > 0 ? lower_bound_u64(src + p0, pn, key) : 0;
            dst[pair0 + (e - own0) + rank] = key;
        }
        __syncthreads();
        uint64_t* t = src;
        src = dst;
        dst = t;
    }
    if (src != seg) {
        for (int32_t e = threadIdx.x; e < len; e += kBlock) seg[e] = src[e];
    }
}

// ---- gathers -------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void gather_out(int64_t nnz, const uint64_t* __restrict__ keys,
                                                     const float* __restrict__ src_val, int32_t* __restrict__ idx_out,
                                                     float* __restrict__ val_out) {
    for (int64_t p = blockIdx.x * (int64_t)kBlock + threadIdx.x; p < nnz; p += (int64_t)gridDim.x * kBlock) {
        const uint64_t k = keys[p];
        idx_out[p] = (int32_t)(k >> 32);
        val_out[p] = src_val[(uint32_t)k];
    }
}

unsigned grid_for(int64_t n) {
    int64_t g = (n + kBlock - 1) / kBlock;
    if (g > 65536) g = 65536;
    if (g < 1) g = 1;
    return (unsigned)g;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout shared by both builders (nseg = number of segments).
struct Layout {
    size_t keys, tmp, cursor, small, large, sums, misc, total;
};

Layout layout(int64_t nseg, int64_t nnz) {
    Layout L;
    size_t off = 0;
    L.keys = off; off = align256(off + (size_t)nnz * 8);
    L.tmp = off; off = align256(off + (size_t)nnz * 8);
    L.cursor = off; off = align256(off + (size_t)(nseg + 1) * 4);
    L.small = off; off = align256(off + (size_t)(nseg + 1) * 4);
    L.large = off; off = align256(off + (size_t)(nseg + 1) * 4);
    const int64_t ntiles = (nseg + 1 + kScanTile - 1) / kScanTile;
    L.sums = off; off = align256(off + (size_t)(ntiles + 1) * 4);
    L.misc = off; off = align256(off + kMiscWords * 4);
    L.total = off;
    return L;
}

#define SPX_HIP(x)                                   \
    do {                                             \
        if ((x) != hipSuccess) return SP_ERR_HIP;    \
    } while (0)
#define SPX_LAUNCH() SPX_HIP(hipGetLastError())

// Inclusive scan of a[0..n) in place.
int scan_inplace(int32_t* a, int64_t n, int32_t* sums, hipStream_t s) {
    if (n <= 0) return SP_OK;
    const int64_t ntiles = (n + kScanTile - 1) / kScanTile;
    hipLaunchKernelGGL(scan_tiles, dim3((unsigned)ntiles), dim3(kBlock), 0, s, a, n, sums);
    SPX_LAUNCH();
    if (ntiles > 1) {
        hipLaunchKernelGGL(scan_sums, dim3(1), dim3(kBlock), 0, s, sums, ntiles);
        SPX_LAUNCH();
        hipLaunchKernelGGL(scan_add, dim3((unsigned)ntiles), dim3(kBlock), 0, s, a, n, sums);
        SPX_LAUNCH();
    }
    return SP_OK;
}

// Common tail: classify segments, sync, sort them.  Returns the host copy of
// misc in *h (error flag, counts, max length) after the sync.
int classify_and_sync(int32_t nseg, const int32_t* ptr, char* ws, const Layout& L, int32_t* h, hipStream_t s) {
    int32_t* misc = reinterpret_cast<int32_t*>(ws + L.misc);
    hipLaunchKernelGGL(classify, dim3(grid_for(nseg)), dim3(kBlock), 0, s, nseg, ptr,
                       reinterpret_cast<int32_t*>(ws + L.cursor), reinterpret_cast<int32_t*>(ws + L.small),
                       reinterpret_cast<int32_t*>(ws + L.large), misc);
    SPX_LAUNCH();
    SPX_HIP(hipMemcpyAsync(h, misc, kMiscWords * 4, hipMemcpyDeviceToHost, s));
    SPX_HIP(hipStreamSynchronize(s));
    return SP_OK;
}

int sort_segments(const int32_t* ptr, char* ws, const Layout& L, const int32_t* h, hipStream_t s) {
    uint64_t* keys = reinterpret_cast<uint64_t*>(ws + L.keys);
    const int32_t n_small = h[kCntSmall], n_large = h[kCntLarge];
    if (n_small > 0) {
        hipLaunchKernelGGL(sort_small, dim3((unsigned)((n_small + 3) / 4)), dim3(kBlock), 0, s,
                           reinterpret_cast<const int32_t*>(ws + L.small),
                           reinterpret_cast<const int32_t*>(ws + L.misc), ptr, keys);
        SPX_LAUNCH();
    }
    if (n_large > 0) {
        hipLaunchKernelGGL(sort_large, dim3((unsigned)n_large), dim3(kBlock), 0, s,
                           reinterpret_cast<const int32_t*>(ws + L.large), ptr, keys,
                           reinterpret_cast<uint64_t*>(ws + L.tmp));
        SPX_LAUNCH();
    }
    return SP_OK;
}

}  // namespace

namespace {
// flag[0] |= 1 when some idx[p] is outside [0, n).
__global__ __launch_bounds__(kBlock) void check_indices(const int32_t* __restrict__ idx, int64_t nnz, int32_t n,
                                                        int32_t* __restrict__ flag) {
    for (int64_t p = blockIdx.x * (int64_t)kBlock + threadIdx.x; p < nnz; p += (int64_t)gridDim.x * kBlock) {
        const int32_t c = idx[p];
        if (c < 0 || c >= n) atomicOr(flag, 1);
    }
}
}  // namespace

hipError_t launch_check_indices(const int32_t* idx, int64_t nnz, int32_t n, int32_t* flag, hipStream_t s) {
    if (nnz <= 0) return hipSuccess;
    hipLaunchKernelGGL(check_indices, dim3(grid_for(nnz)), dim3(kBlock), 0, s, idx, nnz, n, flag);
    return hipGetLastError();
}

size_t scan_work_bytes(int64_t n) { return align256((size_t)((n + kScanTile - 1) / kScanTile + 1) * 4); }

int scan_inclusive_i32(int32_t* a, int64_t n, int32_t* sums, hipStream_t s) { return scan_inplace(a, n, sums, s); }

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_i32, dim3(grid_for(n)), dim3(kBlock), 0, s, p, n, v);
    return hipGetLastError();
}

size_t coo_build_bytes(int64_t m, int64_t, int64_t nnz) { return layout(m, nnz).total; }
size_t csc_build_bytes(int64_t, int64_t n, int64_t nnz) { return layout(n, nnz).total; }

int coo_to_csr_device(int64_t m, int64_t n, int64_t nnz, const int32_t* coo_row, const int32_t* coo_col,
                      const float* coo_val, int32_t* row_ptr, int32_t* col_idx, float* val, void* work,
                      size_t work_bytes, hipStream_t s) {
    const Layout L = layout(m, nnz);
    if (work_bytes < L.total) return SP_ERR_WORKSPACE;
    char* ws = static_cast<char*>(work);
    int32_t* misc = reinterpret_cast<int32_t*>(ws + L.misc);
    hipLaunchKernelGGL(fill_i32, dim3(grid_for(m + 1)), dim3(kBlock), 0, s, row_ptr, m + 1, 0);
    SPX_LAUNCH();
    hipLaunchKernelGGL(fill_i32, dim3(1), dim3(kBlock), 0, s, misc, (int64_t)kMiscWords, 0);
    SPX_LAUNCH();
    if (nnz > 0) {
        hipLaunchKernelGGL(coo_count, dim3(grid_for(nnz)), dim3(kBlock), 0, s, nnz, coo_row, coo_col, (int32_t)m,
                           (int32_t)n, row_ptr + 1, misc);
        SPX_LAUNCH();
    }
    int rc = scan_inplace(row_ptr + 1, m, reinterpret_cast<int32_t*>(ws + L.sums), s);
    if (rc != SP_OK) return rc;
    int32_t h[kMiscWords];
    rc = classify_and_sync((int32_t)m, row_ptr, ws, L, h, s);
    if (rc != SP_OK) return rc;
    if (h[kErr] != 0) return SP_ERR_INDEX;
    if (nnz == 0) return SP_OK;
    uint64_t* keys = reinterpret_cast<uint64_t*>(ws + L.keys);
    hipLaunchKernelGGL(coo_scatter, dim3(grid_for(nnz)), dim3(kBlock), 0, s, nnz, coo_row, coo_col,
                       reinterpret_cast<int32_t*>(ws + L.cursor), keys);
    SPX_LAUNCH();
    rc = sort_segments(row_ptr, ws, L, h, s);
    if (rc != SP_OK) return rc;
    hipLaunchKernelGGL(gather_out, dim3(grid_for(nnz)), dim3(kBlock), 0, s, nnz, keys, coo_val, col_idx, val);
    SPX_LAUNCH();
    return SP_OK;
}

int csr_to_csc_device(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                      const float* val, int32_t* col_ptr, int32_t* row_idx, float* cval, void* work,
                      size_t work_bytes, hipStream_t s) {
    const Layout L = layout(n, nnz);
    if (work_bytes < L.total) return SP_ERR_WORKSPACE;
    char* ws = static_cast<char*>(work);
    int32_t* misc = reinterpret_cast<int32_t*>(ws + L.misc);
    // nnz must equal row_ptr[m]
    int32_t last = 0;
    SPX_HIP(hipMemcpyAsync(&last, row_ptr + m, 4, hipMemcpyDeviceToHost, s));
    SPX_HIP(hipStreamSynchronize(s));
    if ((int64_t)last != nnz) return SP_ERR_SIZE;
    hipLaunchKernelGGL(fill_i32, dim3(grid_for(n + 1)), dim3(kBlock), 0, s, col_ptr, n + 1, 0);
    SPX_LAUNCH();
    hipLaunchKernelGGL(fill_i32, dim3(1), dim3(kBlock), 0, s, misc, (int64_t)kMiscWords, 0);
    SPX_LAUNCH();
    if (nnz > 0) {
        hipLaunchKernelGGL(col_count, dim3(grid_for(nnz)), dim3(kBlock), 0, s, nnz, col_idx, (int32_t)n, col_ptr + 1,
                           misc);
        SPX_LAUNCH();
    }
    int rc = scan_inplace(col_ptr + 1, n, reinterpret_cast<int32_t*>(ws + L.sums), s);
    if (rc != SP_OK) return rc;
    int32_t h[kMiscWords];
    rc = classify_and_sync((int32_t)n, col_ptr, ws, L, h, s);
    if (rc != SP_OK) return rc;
    if (h[kErr] != 0) return SP_ERR_INDEX;
    if (nnz == 0) return SP_OK;
    uint64_t* keys = reinterpret_cast<uint64_t*>(ws + L.keys);
    hipLaunchKernelGGL(csr_scatter, dim3(grid_for(nnz)), dim3(kBlock), 0, s, nnz, row_ptr, (int32_t)m, col_idx,
                       reinterpret_cast<int32_t*>(ws + L.cursor), keys);
    SPX_LAUNCH();
    rc = sort_segments(col_ptr, ws, L, h, s);
    if (rc != SP_OK) return rc;
    hipLaunchKernelGGL(gather_out, dim3(grid_for(nnz)), dim3(kBlock), 0, s, nnz, keys, val, row_idx, cval);
    SPX_LAUNCH();
    return SP_OK;
}

}  // namespace spx
