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
// Segments of length 2..256 are sorted by rank counting (16, 32 or 64 lanes
// per segment up to 64 keys, one wave with 4 keys per lane up to 256),
// 257..4096 by one workgroup (bitonic sort in LDS); longer ones by the whole
// GPU: one workgroup per 4096-key chunk sorts it in LDS, then each merge
// level is one launch over all their keys, each key finding its place by
// binary search in the partner run.
//
// Counts and scatters work on runs: lanes of a wave that hold consecutive
// entries of one segment (sorted input has long runs) take one atomic for
// the whole run, the run's first lane adding its length.
#include "device_common.h"

#include <algorithm>
#include <mutex>

namespace spx {

namespace {

constexpr int kScanTile = 2048;  // elements scanned per workgroup (8 per thread)
constexpr int kChunk = 4096;     // keys sorted in LDS at once
constexpr int kTinySeg = 16;     // segments up to this length: 16 lanes each
constexpr int kHalfSeg = 32;     // up to this length: 32 lanes each
constexpr int kSmallSeg = 64;    // segments up to this length are sorted by one wave
constexpr int kMidSeg = 256;     // up to this length: one wave, 4 keys per lane
constexpr int kClassifyThreads = 1024;
constexpr int32_t kI32MaxLen = 2147483647;

// Segment classes by length: tiny 2..16, half 17..32, small 33..64, mid
// 65..256, large 257..4096, huge longer (segments of 0 or 1 keys need no
// sort).
enum SegClass { kTiny = 0, kHalf = 1, kSmall = 2, kMid = 3, kLarge = 4, kHuge = 5, kClasses = 6 };
enum Misc { kErr = 0, kCnt = 1 /* kCnt + class: listed segments */, kMaxLen = kCnt + kClasses, kMiscWords = 16 };

struct SegLists {
    int32_t* l[kClasses];
};

// Runs of equal segment ids in consecutive lanes of a wave.  `ok` marks the
// lanes that hold an entry; a run is a maximal stretch of ok lanes with the
// same id.  Returns the lane's run head (its first lane); *len receives, in
// a head lane, the run's length.
__device__ __forceinline__ int lane_run(bool ok, int32_t id, int* len) {
    const int lane = threadIdx.x & 63;
    const int32_t prev = __shfl_up(id, 1, 64);
    const bool prev_ok = __shfl_up(ok ? 1 : 0, 1, 64) != 0;
    const bool head = ok && (lane == 0 || !prev_ok || prev != id);
    const uint64_t heads = __ballot(head);
    const uint64_t stops = heads | __ballot(!ok);  // a run ends before the next head or empty lane
    const uint64_t after = stops & ~((2ull << lane) - 1ull);  // stops above this lane (none for lane 63)
    *len = (after ? __ffsll((unsigned long long)after) - 1 : 64) - lane;
    const uint64_t upto = heads & ((2ull << lane) - 1ull);
    return upto ? 63 - __clzll(upto) : lane;
}

__global__ __launch_bounds__(kBlock) void fill_i32(int32_t* p, int64_t n, int32_t v) {
    for (int64_t i = blockIdx.x * (int64_t)kBlock + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBlock) p[i] = v;
}

// Grid-stride loops over whole waves, so that every lane of a wave takes
// part in the run ballots: entry i = i0 + lane, present when i < nnz.
#define SPX_WAVE_LOOP(i0, nnz)                                                                        \
    for (int64_t i0 = blockIdx.x * (int64_t)kBlock + (threadIdx.x & ~63); i0 < (nnz); \
         i0 += (int64_t)gridDim.x * kBlock)

// counts[r + 1] += 1 for every valid (r, c); flags invalid entries.
__global__ __launch_bounds__(kBlock) void coo_count(int64_t nnz, const int32_t* __restrict__ row,
                                                    const int32_t* __restrict__ col, int32_t m, int32_t n,
                                                    int32_t* __restrict__ counts1, int32_t* __restrict__ misc) {
    const int lane = threadIdx.x & 63;
    SPX_WAVE_LOOP(i0, nnz) {
        const int64_t i = i0 + lane;
        const bool in = i < nnz;
        const int32_t r = in ? row[i] : 0, c = in ? col[i] : 0;
        const bool bad = in && (r < 0 || r >= m || c < 0 || c >= n);
        if (bad) atomicOr(misc + kErr, 1);
        int len;
        const int head = lane_run(in && !bad, r, &len);
        if (in && !bad && head == lane) atomicAdd(counts1 + r, len);
    }
}

__global__ __launch_bounds__(kBlock) void col_count(int64_t nnz, const int32_t* __restrict__ col, int32_t n,
                                                    int32_t* __restrict__ counts1, int32_t* __restrict__ misc) {
    const int lane = threadIdx.x & 63;
    SPX_WAVE_LOOP(i0, nnz) {
        const int64_t i = i0 + lane;
        const bool in = i < nnz;
        const int32_t c = in ? col[i] : 0;
        const bool bad = in && (c < 0 || c >= n);
        if (bad) atomicOr(misc + kErr, 1);
        int len;
        const int head = lane_run(in && !bad, c, &len);
        if (in && !bad && head == lane) atomicAdd(counts1 + c, len);
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
// cursor[s] = ptr[s]; every segment of 2 or more keys goes to the list of its
// class; tracks the longest segment.  One atomic per list and workgroup
// pass: the workgroup's segments of a class take consecutive slots (list
// order does not matter, every listed segment is sorted on its own).
__global__ __launch_bounds__(kClassifyThreads) void classify(int32_t nseg, const int32_t* __restrict__ ptr,
                                                            int32_t* __restrict__ cursor, SegLists lists,
                                                            int32_t* __restrict__ misc) {
    constexpr int NW = kClassifyThreads / 64;
    __shared__ int cnt[NW][kClasses];  // per wave, then the waves before it
    __shared__ int base[kClasses];
    __shared__ int wmax[NW];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const uint64_t below = (1ull << lane) - 1;
    for (int64_t s0 = (int64_t)blockIdx.x * kClassifyThreads; s0 < nseg; s0 += (int64_t)gridDim.x * kClassifyThreads) {
        const int64_t s = s0 + tid;
        const bool in = s < nseg;
        const int32_t b = in ? ptr[s] : 0, len = in ? ptr[s + 1] - b : 0;
        if (in) cursor[s] = b;
        const int cls = len < 2 ? -1
                        : len <= kTinySeg  ? kTiny
                        : len <= kHalfSeg  ? kHalf
                        : len <= kSmallSeg ? kSmall
                        : len <= kMidSeg   ? kMid
                        : len <= kChunk    ? kLarge
                                           : kHuge;
        uint64_t mine = 0;
#pragma unroll
        for (int c = 0; c < kClasses; ++c) {
            const uint64_t m = __ballot(cls == c);
            if (lane == 0) cnt[w][c] = (int)__popcll(m);
            if (cls == c) mine = m;
        }
        int32_t mx = len;
        for (int off = 32; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off, 64));
        if (lane == 0) wmax[w] = mx;
        __syncthreads();
        if (tid < kClasses) {
            int tot = 0;
            for (int k = 0; k < NW; ++k) {
                const int t = cnt[k][tid];
                cnt[k][tid] = tot;
                tot += t;
            }
            base[tid] = tot > 0 ? atomicAdd(misc + kCnt + tid, tot) : 0;
        } else if (tid == kClasses) {
            int mm = 0;
            for (int k = 0; k < NW; ++k) mm = max(mm, wmax[k]);
            if (mm > 0) atomicMax(misc + kMaxLen, mm);
        }
        __syncthreads();
        if (cls >= 0) lists.l[cls][base[cls] + cnt[w][cls] + __popcll(mine & below)] = (int32_t)s;
        __syncthreads();  // cnt and base are rewritten by the next pass
    }
}

// ---- keyed scatters ---------------------------------------------------------
// (All indices were checked by the count kernel before the scatters run.)
__global__ __launch_bounds__(kBlock) void coo_scatter(int64_t nnz, const int32_t* __restrict__ row,
                                                      const int32_t* __restrict__ col, int32_t* __restrict__ cursor,
                                                      uint64_t* __restrict__ keys) {
    const int lane = threadIdx.x & 63;
    SPX_WAVE_LOOP(i0, nnz) {
        const int64_t i = i0 + lane;
        const bool in = i < nnz;
        const int32_t r = in ? row[i] : 0;
        int len;
        const int head = lane_run(in, r, &len);
        const int32_t base = in && head == lane ? atomicAdd(cursor + r, len) : 0;
        const int32_t p = __shfl(base, head, 64) + (lane - head);
        if (in) keys[p] = ((uint64_t)(uint32_t)col[i] << 32) | (uint64_t)i;
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
    const int lane = threadIdx.x & 63;
    SPX_WAVE_LOOP(p0, nnz) {
        const int64_t p = p0 + lane;
        const bool in = p < nnz;
        const int32_t c = in ? col[p] : 0;
        int len;
        const int head = lane_run(in, c, &len);
        const int32_t base = in && head == lane ? atomicAdd(cursor + c, len) : 0;
        const int32_t q = __shfl(base, head, 64) + (lane - head);
        if (in) keys[q] = ((uint64_t)(uint32_t)row_of(row_ptr, m, (int32_t)p) << 32) | (uint64_t)p;
    }
}

// ---- segment sorts ------------------------------------------------------------
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
    const int lo = __shfl((int)(uint32_t)v, src, 64);
    const int hi = __shfl((int)(uint32_t)(v >> 32), src, 64);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// G lanes per segment of 2..G keys (64 / G segments per wave): rank = the
// number of smaller keys in the segment (keys are unique, and below ~0).
template <int G>
__global__ __launch_bounds__(kBlock) void sort_small(const int32_t* __restrict__ list, int32_t count,
                                                     const int32_t* __restrict__ ptr, uint64_t* __restrict__ keys) {
    const int lane = threadIdx.x & 63, g0 = lane & ~(G - 1), gl = lane & (G - 1);
    const int64_t k = ((int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6)) * (64 / G) + lane / G;
    if (k - lane / G >= count) return;  // the whole wave is past the list
    int32_t b = 0, len = 0;
    if (k < count) {
        const int32_t s = list[k];
        b = ptr[s];
        len = ptr[s + 1] - b;
    }
    const uint64_t key = gl < len ? keys[b + gl] : ~0ull;
    int longest = len;
    for (int off = 32; off > 0; off >>= 1) longest = max(longest, __shfl_xor(longest, off, 64));
    int rank = 0;
    for (int i = 0; i < longest; ++i) rank += shfl_u64(key, g0 + i) < key ? 1 : 0;
    if (gl < len) keys[b + rank] = key;
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

// Sorts seg[0..n) (n <= kChunk) in LDS; the whole workgroup takes part.
__device__ void sort_chunk(uint64_t* __restrict__ seg, int32_t n, uint64_t* sh) {
    int P = 2;
    while (P < n) P <<= 1;
    for (int i = threadIdx.x; i < P; i += kBlock) sh[i] = i < n ? seg[i] : ~0ull;
    __syncthreads();
    bitonic_lds(sh, P);
    for (int i = threadIdx.x; i < n; i += kBlock) seg[i] = sh[i];
    __syncthreads();
}

// One wave per segment of 65..256 keys, 4 keys per lane: rank = the number of
// smaller keys, read back one by one from the segment's copy in LDS.
__global__ __launch_bounds__(kBlock) void sort_mid(const int32_t* __restrict__ list, int32_t count,
                                                   const int32_t* __restrict__ ptr, uint64_t* __restrict__ keys) {
    constexpr int KPL = kMidSeg / 64;  // keys per lane
    __shared__ uint64_t sh[kBlock / 64][kMidSeg];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t k = (int64_t)blockIdx.x * (kBlock / 64) + w;
    int32_t b = 0, len = 0;
    if (k < count) {
        const int32_t s = list[k];
        b = ptr[s];
        len = ptr[s + 1] - b;
    }
    uint64_t key[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
        const int i = lane + 64 * j;
        key[j] = i < len ? keys[b + i] : ~0ull;
        sh[w][i] = key[j];
    }
    __syncthreads();
    int rank[KPL] = {};
    for (int i = 0; i < len; ++i) {
        const uint64_t o = sh[w][i];
#pragma unroll
        for (int j = 0; j < KPL; ++j) rank[j] += o < key[j] ? 1 : 0;
    }
#pragma unroll
    for (int j = 0; j < KPL; ++j)
        if (lane + 64 * j < len) keys[b + rank[j]] = key[j];
}

// One workgroup per segment of 257..kChunk keys.
__global__ __launch_bounds__(kBlock) void sort_large(const int32_t* __restrict__ list, const int32_t* __restrict__ ptr,
                                                     uint64_t* __restrict__ keys) {
    __shared__ uint64_t sh[kChunk];
    const int32_t s = list[blockIdx.x];
    const int32_t b = ptr[s];
    sort_chunk(keys + b, ptr[s + 1] - b, sh);
}

// ---- segments longer than kChunk: the whole GPU sorts them together.
// tab[k] = {begin, length, keys before segment k, chunks before segment k}
// over the huge segments, and tab[n] = {0, 0, all keys, all chunks}.
// One workgroup builds the table: prefix sums of the segments' key and chunk
// counts, 1024 segments per pass.
constexpr int kTableThreads = 1024;
__global__ __launch_bounds__(kTableThreads) void huge_table(const int32_t* __restrict__ list, int32_t n,
                                                           const int32_t* __restrict__ ptr, int4* __restrict__ tab) {
    constexpr int NW = kTableThreads / 64;
    __shared__ int wk[NW], wc[NW];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int carry_k = 0, carry_c = 0;  // keys and chunks of the passes before (every thread)
    for (int32_t k0 = 0; k0 < n; k0 += kTableThreads) {
        const int32_t k = k0 + tid;
        int32_t b = 0, len = 0;
        if (k < n) {
            const int32_t s = list[k];
            b = ptr[s];
            len = ptr[s + 1] - b;
        }
        const int ch = (len + kChunk - 1) / kChunk;
        int ik = len, ic = ch;  // inclusive sums over the wave
        for (int off = 1; off < 64; off <<= 1) {
            const int tk = __shfl_up(ik, off, 64), tc = __shfl_up(ic, off, 64);
            if (lane >= off) {
                ik += tk;
                ic += tc;
            }
        }
        if (lane == 63) {
            wk[w] = ik;
            wc[w] = ic;
        }
        __syncthreads();
        int bk = carry_k, bc = carry_c;
        for (int j = 0; j < w; ++j) {
            bk += wk[j];
            bc += wc[j];
        }
        if (k < n) tab[k] = make_int4(b, len, bk + ik - len, bc + ic - ch);
        for (int j = 0; j < NW; ++j) {
            carry_k += wk[j];
            carry_c += wc[j];
        }
        __syncthreads();  // wk and wc are rewritten by the next pass
    }
    if (tid == 0) tab[n] = make_int4(0, 0, carry_k, carry_c);
}

// The last k in [0, n) with field(tab[k]) <= f (field: .z keys or .w chunks).
template <bool kByChunk>
__device__ __forceinline__ int32_t huge_of(const int4* __restrict__ tab, int32_t n, int64_t f) {
    int32_t lo = 0, hi = n - 1;
    while (lo < hi) {
        const int32_t mid = lo + (hi - lo + 1) / 2;
        const int32_t v = kByChunk ? tab[mid].w : tab[mid].z;
        if (v <= f) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Workgroup c sorts chunk c of the huge segments in LDS.
__global__ __launch_bounds__(kBlock) void huge_chunks(const int4* __restrict__ tab, int32_t n,
                                                      uint64_t* __restrict__ keys) {
    __shared__ uint64_t sh[kChunk];
    const int32_t c = blockIdx.x;
    if (c >= tab[n].w) return;  // the grid is an upper bound
    const int4 t = tab[huge_of<true>(tab, n, c)];
    const int32_t j = c - t.w;  // chunk within the segment
    const int32_t n_keys = min(kChunk, t.y - j * kChunk);
    sort_chunk(keys + t.x + (int64_t)j * kChunk, n_keys, sh);
}

// One merge level over all huge segments: within each segment, sorted runs
// of width w are merged in pairs from src to dst; key e of run r goes to the
// start of its pair plus its place in its own run plus the number of smaller
// keys in the partner run.  A segment no longer than w is copied.
__global__ __launch_bounds__(kBlock) void huge_merge(const int4* __restrict__ tab, int32_t n, int32_t w,
                                                     const uint64_t* __restrict__ src, uint64_t* __restrict__ dst) {
    const int64_t f = blockIdx.x * (int64_t)kBlock + threadIdx.x;
    if (f >= tab[n].z) return;
    const int4 t = tab[huge_of<false>(tab, n, f)];
    const int32_t e = (int32_t)(f - t.z), len = t.y;
    const uint64_t* sseg = src + t.x;
    uint64_t* dseg = dst + t.x;
    const int64_t run = e / w;
    const int64_t pair0 = (run & ~1ll) * w;  // start of the left run of the pair
    const int64_t own0 = run * w;
    const bool left = (run & 1) == 0;
    const int64_t p0 = left ? own0 + w : pair0;  // partner run start
    int64_t pn = left ? min((int64_t)len - p0, (int64_t)w) : (int64_t)w;
    if (pn < 0) pn = 0;
    const uint64_t key = sseg[e];
    const int32_t rank = pn > 0 ? lower_bound_u64(sseg + p0, (int32_t)pn, key) : 0;
    dseg[pair0 + (e - own0) + rank] = key;
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
    size_t keys, tmp, cursor, tiny, half, small, mid, large, huge, htab, sums, misc, total;
};

// Segments longer than kChunk: at most this many.
int64_t max_huge(int64_t nnz) { return nnz / (kChunk + 1) + 1; }

Layout layout(int64_t nseg, int64_t nnz) {
    Layout L;
    size_t off = 0;
    L.keys = off; off = align256(off + (size_t)nnz * 8);
    L.tmp = off; off = align256(off + (size_t)nnz * 8);
    L.cursor = off; off = align256(off + (size_t)(nseg + 1) * 4);
    L.tiny = off; off = align256(off + (size_t)(nseg + 1) * 4);
    L.half = off; off = align256(off + (size_t)(nseg + 1) * 4);
    L.small = off; off = align256(off + (size_t)(nseg + 1) * 4);
    L.mid = off; off = align256(off + (size_t)(nseg + 1) * 4);
    L.large = off; off = align256(off + (size_t)(nseg + 1) * 4);
    L.huge = off; off = align256(off + (size_t)max_huge(nnz) * 4);
    L.htab = off; off = align256(off + (size_t)(max_huge(nnz) + 1) * 16);
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
    SegLists lists;
    lists.l[kTiny] = reinterpret_cast<int32_t*>(ws + L.tiny);
    lists.l[kHalf] = reinterpret_cast<int32_t*>(ws + L.half);
    lists.l[kSmall] = reinterpret_cast<int32_t*>(ws + L.small);
    lists.l[kMid] = reinterpret_cast<int32_t*>(ws + L.mid);
    lists.l[kLarge] = reinterpret_cast<int32_t*>(ws + L.large);
    lists.l[kHuge] = reinterpret_cast<int32_t*>(ws + L.huge);
    const int64_t passes = std::max<int64_t>(1, std::min<int64_t>((nseg + kClassifyThreads - 1) / kClassifyThreads, 4096));
    hipLaunchKernelGGL(classify, dim3((unsigned)passes), dim3(kClassifyThreads), 0, s, nseg, ptr,
                       reinterpret_cast<int32_t*>(ws + L.cursor), lists, misc);
    SPX_LAUNCH();
    SPX_HIP(hipMemcpyAsync(h, misc, kMiscWords * 4, hipMemcpyDeviceToHost, s));
    SPX_HIP(hipStreamSynchronize(s));
    return SP_OK;
}

int sort_segments(const int32_t* ptr, int64_t nnz, char* ws, const Layout& L, const int32_t* h, hipStream_t s) {
    uint64_t* keys = reinterpret_cast<uint64_t*>(ws + L.keys);
    const int32_t n_tiny = h[kCnt + kTiny], n_half = h[kCnt + kHalf], n_small = h[kCnt + kSmall];
    const int32_t n_mid = h[kCnt + kMid], n_large = h[kCnt + kLarge];
    constexpr int kWaves = kBlock / 64;
    if (n_tiny > 0) {  // 4 segments per wave
        const int64_t waves = (n_tiny + 3) / 4;
        hipLaunchKernelGGL(sort_small<kTinySeg>, dim3((unsigned)((waves + kWaves - 1) / kWaves)), dim3(kBlock), 0, s,
                           reinterpret_cast<const int32_t*>(ws + L.tiny), n_tiny, ptr, keys);
        SPX_LAUNCH();
    }
    if (n_half > 0) {  // 2 segments per wave
        const int64_t waves = (n_half + 1) / 2;
        hipLaunchKernelGGL(sort_small<kHalfSeg>, dim3((unsigned)((waves + kWaves - 1) / kWaves)), dim3(kBlock), 0, s,
                           reinterpret_cast<const int32_t*>(ws + L.half), n_half, ptr, keys);
        SPX_LAUNCH();
    }
    if (n_small > 0) {
        hipLaunchKernelGGL(sort_small<kSmallSeg>, dim3((unsigned)((n_small + kWaves - 1) / kWaves)), dim3(kBlock), 0,
                           s, reinterpret_cast<const int32_t*>(ws + L.small), n_small, ptr, keys);
        SPX_LAUNCH();
    }
    if (n_mid > 0) {
        hipLaunchKernelGGL(sort_mid, dim3((unsigned)((n_mid + kWaves - 1) / kWaves)), dim3(kBlock), 0, s,
                           reinterpret_cast<const int32_t*>(ws + L.mid), n_mid, ptr, keys);
        SPX_LAUNCH();
    }
    if (n_large > 0) {
        hipLaunchKernelGGL(sort_large, dim3((unsigned)n_large), dim3(kBlock), 0, s,
                           reinterpret_cast<const int32_t*>(ws + L.large), ptr, keys);
        SPX_LAUNCH();
    }
    const int32_t n_huge = h[kCnt + kHuge];
    if (n_huge > 0) {
        // the segment table is built on the device; the grids take upper
        // bounds (every huge segment is at most the longest, all together
        // at most nnz keys) and their kernels stop at the table's totals
        int4* htab = reinterpret_cast<int4*>(ws + L.htab);
        hipLaunchKernelGGL(huge_table, dim3(1), dim3(kTableThreads), 0, s,
                           reinterpret_cast<const int32_t*>(ws + L.huge), n_huge, ptr, htab);
        SPX_LAUNCH();
        const int64_t longest = h[kMaxLen];
        const int64_t max_keys = std::min<int64_t>(nnz, (int64_t)n_huge * longest);
        const int64_t max_chunks = std::min<int64_t>(max_keys / kChunk + n_huge, (int64_t)n_huge * ((longest + kChunk - 1) / kChunk));
        hipLaunchKernelGGL(huge_chunks, dim3((unsigned)max_chunks), dim3(kBlock), 0, s, htab, n_huge, keys);
        SPX_LAUNCH();
        uint64_t* src = keys;
        uint64_t* dst = reinterpret_cast<uint64_t*>(ws + L.tmp);
        const unsigned grid = (unsigned)((max_keys + kBlock - 1) / kBlock);
        int levels = 0;
        for (int64_t w = kChunk; w < longest; w <<= 1, ++levels) {
            hipLaunchKernelGGL(huge_merge, dim3(grid), dim3(kBlock), 0, s, htab, n_huge, (int32_t)w, src, dst);
            SPX_LAUNCH();
            std::swap(src, dst);
        }
        if (levels & 1) {  // the result is in tmp: a width past every segment copies it back
            hipLaunchKernelGGL(huge_merge, dim3(grid), dim3(kBlock), 0, s, htab, n_huge, (int32_t)kI32MaxLen, src,
                               dst);
            SPX_LAUNCH();
        }
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
    rc = sort_segments(row_ptr, nnz, ws, L, h, s);
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
    rc = sort_segments(col_ptr, nnz, ws, L, h, s);
    if (rc != SP_OK) return rc;
    hipLaunchKernelGGL(gather_out, dim3(grid_for(nnz)), dim3(kBlock), 0, s, nnz, keys, val, row_idx, cval);
    SPX_LAUNCH();
    return SP_OK;
}

// ---------------------------------------------------------------------------
// COO -> CSR for callers that cannot allocate device memory: the same
// conversion, its scratch taken from `scratch`, a static device array of
// kNoallocScratchBytes on every GPU the library runs on (held until the
// process ends).  Each region of it that the conversion reads is first
// written by the same call (counts and flags by fill kernels, cursors by the
// classification, keys by the scatter), so whatever a previous call left
// there does not matter.  All calls on one GPU share the array: two calls
// that overlap in time on one GPU (other streams, other host threads) race.
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
constexpr int kNoallocMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kNoallocMaxDevices] = {};
}  // namespace

// Device address of `scratch` on the current device.  The name of the array
// in host code is only a host-side stand-in: its device address is looked up
// once per device, with that device current, and kept.
static int scratch_on_current_device(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SP_ERR_HIP;
    if (dev < 0 || dev >= kNoallocMaxDevices) return SP_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SP_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SP_OK;
}

size_t coo_build_noalloc_limit() { return kNoallocScratchBytes; }

int coo_to_csr_noalloc(int64_t m, int64_t n, int64_t nnz, const int32_t* coo_row, const int32_t* coo_col,
                       const float* coo_val, int32_t* row_ptr, int32_t* col_idx, float* val, hipStream_t s) {
    if (coo_build_bytes(m, n, nnz) > kNoallocScratchBytes) return SP_ERR_WORKSPACE;
    void* ws = nullptr;
    const int rc = scratch_on_current_device(&ws);
    if (rc != SP_OK) return rc;
    return coo_to_csr_device(m, n, nnz, coo_row, coo_col, coo_val, row_ptr, col_idx, val, ws, kNoallocScratchBytes,
                             s);
}

}  // namespace spx
