// CSR SpMM  C = alpha * A B + beta * C  for gfx950 (B: K x N, C: M x N,
// both row-major).
//
// 「通用稀疏矩阵乘法CUDA算子实现」 §3: every A(i,k) read is reused across a
// tile of consecutive columns B(k, n:n+T) held in registers, and C is
// written once by a single owner.  Here a row is owned by a sub-group of G
// lanes, each lane holding V = 4 consecutive columns (one 16-byte load of B
// per entry), so one tile is T = 4G columns (G <= 64, T <= 256); blockIdx.y
// walks the tiles.  Small N (8) gives G = 2 and 32 rows in flight per wave
// (§3.1), medium N (32..128) a wave or half-wave per row (§3.2), and wider N
// more tiles per row group (§3.3).
//
// The row bins are the plan's (the same as SpMV): groups of short rows stage
// their (column, value) pairs through LDS; wave / block rows spread a row's
// entries over the sub-groups and reduce across them; split rows write
// per-segment partial tiles that the last segment adds in fixed order.
#include <algorithm>

#include "device_common.h"

namespace spx {

namespace {

template <int V>
struct Acc {
    float v[V];
};

template <int V>
__device__ __forceinline__ void acc_zero(Acc<V>& a) {
#pragma unroll
    for (int i = 0; i < V; ++i) a.v[i] = 0.0f;
}

template <int V>
__device__ __forceinline__ void acc_fma(Acc<V>& a, float s, const float* __restrict__ b) {
    if constexpr (V == 4) {
        const float4 q = *reinterpret_cast<const float4*>(b);
        a.v[0] = fmaf(s, q.x, a.v[0]);
        a.v[1] = fmaf(s, q.y, a.v[1]);
        a.v[2] = fmaf(s, q.z, a.v[2]);
        a.v[3] = fmaf(s, q.w, a.v[3]);
    } else {
        a.v[0] = fmaf(s, b[0], a.v[0]);
    }
}

template <int V>
__device__ __forceinline__ void store_tile(float* __restrict__ c, const Acc<V>& a, float alpha, float beta) {
    if constexpr (V == 4) {
        float4 o = make_float4(alpha * a.v[0], alpha * a.v[1], alpha * a.v[2], alpha * a.v[3]);
        if (beta != 0.0f) {
            const float4 old = *reinterpret_cast<const float4*>(c);
            o.x = fmaf(beta, old.x, o.x);
            o.y = fmaf(beta, old.y, o.y);
            o.z = fmaf(beta, old.z, o.z);
            o.w = fmaf(beta, old.w, o.w);
        }
        *reinterpret_cast<float4*>(c) = o;
    } else {
        float o = alpha * a.v[0];
        if (beta != 0.0f) o = fmaf(beta, c[0], o);
        c[0] = o;
    }
}

struct Ctx {
    const int32_t* ptr;
    const int32_t* idx;
    const float* val;
    const float* B;
    int64_t ldb;
    float* C;
    int64_t ldc;
    int N;
    float alpha, beta;
};

// ---- group: consecutive short rows, (col, val) staged in LDS ---------------
template <int V>
__device__ void spmm_group(const Ctx& x, const int4 t, int G, int n0, int32_t* lcol, float* lval) {
    const int r0 = t.x, r1 = t.y, b = t.z, e = t.w;
    const int tid = threadIdx.x;
    for (int q = b + tid; q < e; q += kBlock) {
        lcol[q - b] = __builtin_nontemporal_load(x.idx + q);
        lval[q - b] = __builtin_nontemporal_load(x.val + q);
    }
    __syncthreads();
    const int nsub = kBlock / G;
    const int sub = tid / G;
    const bool colok = n0 < x.N;
    for (int row = r0 + sub; row < r1; row += nsub) {
        Acc<V> a;
        acc_zero(a);
        const int kb = x.ptr[row] - b, ke = x.ptr[row + 1] - b;
        if (colok) {
#pragma unroll 4
            for (int k = kb; k < ke; ++k) acc_fma<V>(a, lval[k], x.B + (int64_t)lcol[k] * x.ldb + n0);
            store_tile<V>(x.C + (int64_t)row * x.ldc + n0, a, x.alpha, x.beta);
        }
    }
}

// Entries [b, e) of one row spread over `nsub` sub-groups starting at `sub`
// with stride `step`; the per-lane partial tile is returned.
template <int V>
__device__ __forceinline__ Acc<V> strided_row(const Ctx& x, int b, int e, int first, int step, int n0) {
    Acc<V> a;
    acc_zero(a);
    if (n0 < x.N) {
#pragma unroll 4
        for (int k = b + first; k < e; k += step) {
            const int c = x.idx[k];
            acc_fma<V>(a, x.val[k], x.B + (int64_t)c * x.ldb + n0);
        }
    }
    return a;
}

template <int V>
__device__ __forceinline__ void reduce_sub_groups(Acc<V>& a, int G) {
#pragma unroll
    for (int i = 0; i < V; ++i) a.v[i] = cross_group_sum(a.v[i], G);
}

// ---- wave: one row per wave ---------------------------------------------------
template <int V>
__device__ void spmm_wave(const Ctx& x, const int4 t, bool valid, int G, int n0) {
    const int l = threadIdx.x & 63;
    const int nsub = 64 / G, sub = l / G;
    Acc<V> a;
    if (valid) {
        a = strided_row<V>(x, t.y, t.z, sub, nsub, n0);
    } else {
        acc_zero(a);
    }
    reduce_sub_groups<V>(a, G);
    if (valid && sub == 0 && n0 < x.N) store_tile<V>(x.C + (int64_t)t.x * x.ldc + n0, a, x.alpha, x.beta);
}

// Workgroup-wide tile sum over [b, e); result valid in wave 0, sub-group 0.
template <int V>
__device__ __forceinline__ Acc<V> block_tile_sum(const Ctx& x, int b, int e, int G, int n0, float* lds) {
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int nsub = 64 / G, sub = l / G, lane = l - sub * G;
    Acc<V> a = strided_row<V>(x, b, e, w * nsub + sub, 4 * nsub, n0);
    reduce_sub_groups<V>(a, G);
    if (sub == 0) {
#pragma unroll
        for (int i = 0; i < V; ++i) lds[(w * G + lane) * V + i] = a.v[i];
    }
    __syncthreads();
    if (w == 0 && sub == 0) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const float s0 = lds[(0 * G + lane) * V + i], s1 = lds[(1 * G + lane) * V + i];
            const float s2 = lds[(2 * G + lane) * V + i], s3 = lds[(3 * G + lane) * V + i];
            a.v[i] = (s0 + s1) + (s2 + s3);
        }
    }
    return a;
}

template <int V>
__device__ void spmm_block(const Ctx& x, const int4 t, int G, int n0, float* lds) {
    Acc<V> a = block_tile_sum<V>(x, t.y, t.z, G, n0, lds);
    const int tid = threadIdx.x;
    if (tid < G && n0 < x.N) store_tile<V>(x.C + (int64_t)t.x * x.ldc + n0, a, x.alpha, x.beta);
}

template <int V>
__device__ void spmm_split(const Ctx& x, const int4 t, const int4* __restrict__ split_rows, float* partials,
                           int32_t* counters, int ntiles, int G, int n0, float* lds) {
    const int4 sr = split_rows[t.x];  // {row, partial_base, nseg, 0}
    Acc<V> a = block_tile_sum<V>(x, t.z, t.w, G, n0, lds);
    const int tid = threadIdx.x;
    const bool owner = tid < G && n0 < x.N;
    if (owner) {
        float* p = partials + (int64_t)(sr.y + t.y) * x.N + n0;
#pragma unroll
        for (int i = 0; i < V; ++i) atomic_store_f(p + i, a.v[i]);
    }
    __threadfence();
    __syncthreads();
    __shared__ int last;
    if (tid == 0) {
        int32_t* cnt = counters + (int64_t)t.x * ntiles + blockIdx.y;
        const int arrived = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        last = (arrived == sr.z - 1);
        if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (last) {
        __threadfence();
        if (owner) {
            acc_zero(a);
            for (int k = 0; k < sr.z; ++k) {
                const float* p = partials + (int64_t)(sr.y + k) * x.N + n0;
#pragma unroll
                for (int i = 0; i < V; ++i) a.v[i] += atomic_load_f(p + i);
            }
            store_tile<V>(x.C + (int64_t)sr.x * x.ldc + n0, a, x.alpha, x.beta);
        }
    }
}

template <int V>
__global__ __launch_bounds__(kBlock) void spmm_bins_kernel(
    const int4* __restrict__ tasks, int n_split, int n_block, int n_wave, int n_group, int xcd_remap,
    const int4* __restrict__ split_rows, float* partials, int32_t* counters, int G, int group_cap, Ctx x) {
    extern __shared__ float dyn_lds[];
    const int ntiles = gridDim.y;
    const int lane_col = (threadIdx.x & 63) % G;
    const int n0 = blockIdx.y * (G * V) + lane_col * V;
    int b = blockIdx.x;
    if (b < n_split) {
        spmm_split<V>(x, tasks[b], split_rows, partials, counters, ntiles, G, n0, dyn_lds);
        return;
    }
    b -= n_split;
    if (b < n_block) {
        spmm_block<V>(x, tasks[n_split + b], G, n0, dyn_lds);
        return;
    }
    b -= n_block;
    const int n_wave_wg = (n_wave + 3) / 4;
    if (b < n_wave_wg) {
        const int w = 4 * b + (threadIdx.x >> 6);
        const bool valid = w < n_wave;
        const int4 t = valid ? tasks[n_split + n_block + w] : make_int4(0, 0, 0, 0);
        spmm_wave<V>(x, t, valid, G, n0);
        return;
    }
    b -= n_wave_wg;
    const int first = n_split + n_block + n_wave_wg;
    const int g = xcd_remap ? xcd_contiguous(blockIdx.x, first, n_group) : b;
    int32_t* lcol = reinterpret_cast<int32_t*>(dyn_lds);
    float* lval = dyn_lds + group_cap;
    spmm_group<V>(x, tasks[n_split + n_block + n_wave + g], G, n0, lcol, lval);
}

// ---- phase-swept SpMM (small N) ---------------------------------------------
// 「通用稀疏矩阵乘法CUDA算子实现」 §3.1: with few right-hand sides each entry's B
// row segment is short, and the B reads, not the arithmetic, set the time;
// §2.5: reads that leave the cache are the cost.  Here the columns are cut into
// phases of 2^pb columns (a B slice of 2^pb rows) and every wave sweeps the
// phases in the same order, so that at any time the waves of an XCD read about
// one slice, which its L2 holds.  A workgroup owns kSwRows consecutive rows of
// C, kept in LDS, cut into one contiguous row range per wave with about equal
// entry counts (so that the waves move through the phases at the same pace).
// A wave's entries are stored contiguously, phase by phase, rows then columns
// ascending inside a phase, as a word (row within the workgroup's rows) <<
// kSwColBits | column, and the value, and are read in steps of EPS = 64 / NV
// entries: NV lanes per entry, four columns each (N = 4 NV), U steps with their
// loads and gathers in flight together.  The products of a step are summed per
// (phase, row) by a segmented scan over the step (that key never decreases
// along the stream), and the last entry of each run adds the run's sum to its
// row in LDS, phase by phase.  Only one wave touches a row, in program order,
// so every C element is a sum in a fixed order: results are reproducible bit
// for bit, with no floating-point atomics and no partial sums in memory.
constexpr uint32_t kSwColMask = (1u << kSwColBits) - 1u;

template <int NV, int U>
__global__ __launch_bounds__(kSwWaves * 64) void spmm_sweep_kernel(int P, int pb,
                                                                   const int32_t* __restrict__ off,
                                                                   const int32_t* __restrict__ wrow,
                                                                   const uint32_t* __restrict__ pk,
                                                                   const float* __restrict__ pv,
                                                                   const float* __restrict__ B, int64_t ldb,
                                                                   float alpha, float beta, float* __restrict__ C,
                                                                   int64_t ldc) {
    constexpr int N = 4 * NV;
    constexpr int EPS = 64 / NV;
    __shared__ __attribute__((aligned(16))) float csh[kSwRows * N];
    const int g = blockIdx.x, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int j = lane / NV, h = lane - j * NV;
    const int rb = g * kSwRows;                  // first row of the workgroup
    const int row0 = wrow[g * kSwWaves + w];     // the wave's rows [row0, row1)
    const int nrows = wrow[g * kSwWaves + w + 1] - row0;
    float* cw = csh + (row0 - rb) * N;
    for (int k = lane; k < nrows * NV; k += 64)
        *reinterpret_cast<float4*>(cw + 4 * k) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    const int64_t cell = ((int64_t)g * kSwWaves + w) * P;
    const int wb = off[cell], we = off[cell + P];  // the wave's entries, phase by phase
    const float* __restrict__ bh = B + 4 * h;
    for (int e = wb; e < we; e += U * EPS) {
        uint32_t word[U];
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = e + u * EPS + j;
            word[u] = 0u;
            v[u] = 0.0f;
            if (q < we) {
                word[u] = __builtin_nontemporal_load(pk + q);
                v[u] = __builtin_nontemporal_load(pv + q);
            }
        }
        float4 b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            b[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (e + u * EPS + j < we)
                b[u] = *reinterpret_cast<const float4*>(bh + (int64_t)(word[u] & kSwColMask) * ldb);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool valid = e + u * EPS + j < we;
            const int row = (int)(word[u] >> kSwColBits);
            // run key: (phase, row); entries past the end get keys of their own
            const int key = valid ? (int)(((word[u] & kSwColMask) >> pb) << kSwRowBits) | row : -1 - j;
            float4 a = make_float4(v[u] * b[u].x, v[u] * b[u].y, v[u] * b[u].z, v[u] * b[u].w);
#pragma unroll
            for (int d = 1; d < EPS; d <<= 1) {
                const int ks = __shfl_up(key, d * NV, 64);
                const float sx = __shfl_up(a.x, d * NV, 64), sy = __shfl_up(a.y, d * NV, 64);
                const float sz = __shfl_up(a.z, d * NV, 64), sw = __shfl_up(a.w, d * NV, 64);
                if (j >= d && ks == key) {
                    a.x += sx;
                    a.y += sy;
                    a.z += sz;
                    a.w += sw;
                }
            }
            const int kn = __shfl_down(key, NV, 64);
            const bool last = valid && (j == EPS - 1 || kn != key);
            // A step can hold runs of one row from several phases: their adds
            // go in rounds, one phase per round, lowest first (the stream is in
            // phase order, so the lowest pending lane has the lowest phase);
            // inside a phase every run has a row of its own.
            const int ph = key >> kSwRowBits;
            uint64_t pend = __ballot(last);
            while (pend) {
                const int p0 = __shfl(ph, __ffsll((unsigned long long)pend) - 1, 64);
                const bool mine = last && ph == p0;
                if (mine) {
                    float4* c = reinterpret_cast<float4*>(csh + row * N + 4 * h);
                    float4 o = *c;
                    o.x += a.x;
                    o.y += a.y;
                    o.z += a.z;
                    o.w += a.w;
                    *c = o;
                }
                pend &= ~__ballot(mine);
            }
        }
    }
    // the wave's rows of C, with the axpby epilogue
    for (int k = lane; k < nrows * NV; k += 64) {
        const int rr = k / NV, hh = k - rr * NV;
        const float4 acc = *reinterpret_cast<const float4*>(cw + rr * N + 4 * hh);
        Acc<4> t;
        t.v[0] = acc.x;
        t.v[1] = acc.y;
        t.v[2] = acc.z;
        t.v[3] = acc.w;
        store_tile<4>(C + (int64_t)(row0 + rr) * ldc + 4 * hh, t, alpha, beta);
    }
}

// Turns the slot -> CSR entry map that the host uploaded into d.sw_pk into the
// packed words (row within its workgroup's rows, column) and the values.  Slot
// s is read and written by one thread only.
__global__ __launch_bounds__(kBlock) void sweep_build_kernel(int rows, int64_t nnz, const int32_t* __restrict__ ptr,
                                                             const int32_t* __restrict__ idx,
                                                             const float* __restrict__ val, uint32_t* pk, float* pv) {
    for (int64_t s = (int64_t)blockIdx.x * kBlock + threadIdx.x; s < nnz; s += (int64_t)gridDim.x * kBlock) {
        const int q = (int)pk[s];
        int lo = 0, hi = rows;  // ptr[lo] <= q < ptr[hi]: the row of entry q is the last such lo
        while (hi - lo > 1) {
            const int mid = lo + ((hi - lo) >> 1);
            if (ptr[mid] <= q)
                lo = mid;
            else
                hi = mid;
        }
        pk[s] = ((uint32_t)(lo % kSwRows) << kSwColBits) | ((uint32_t)idx[q] & kSwColMask);
        pv[s] = val[q];
    }
}

}  // namespace

bool spmm_sweep_ok(const DirDevice& d, int32_t N, const float* B, int64_t ldb, const float* C, int64_t ldc) {
    return d.sw_pb > 0 && (N == 4 || N == 8 || N == 16) && ldb % 4 == 0 && ldc % 4 == 0 &&
           (reinterpret_cast<uintptr_t>(B) & 15) == 0 && (reinterpret_cast<uintptr_t>(C) & 15) == 0;
}

hipError_t launch_spmm_sweep(const DirDevice& d, int32_t N, float alpha, const float* B, int64_t ldb, float beta,
                             float* C, int64_t ldc, hipStream_t s) {
    const dim3 grid((unsigned)d.sw_nblk), block(kSwWaves * 64);
    if (N == 4)
        hipLaunchKernelGGL((spmm_sweep_kernel<1, 4>), grid, block, 0, s, d.sw_P, d.sw_pb, d.sw_off, d.sw_wrow,
                           d.sw_pk, d.sw_pv, B, ldb, alpha, beta, C, ldc);
    else if (N == 8)
        hipLaunchKernelGGL((spmm_sweep_kernel<2, 4>), grid, block, 0, s, d.sw_P, d.sw_pb, d.sw_off, d.sw_wrow,
                           d.sw_pk, d.sw_pv, B, ldb, alpha, beta, C, ldc);
    else
        hipLaunchKernelGGL((spmm_sweep_kernel<4, 4>), grid, block, 0, s, d.sw_P, d.sw_pb, d.sw_off, d.sw_wrow,
                           d.sw_pk, d.sw_pv, B, ldb, alpha, beta, C, ldc);
    return hipGetLastError();
}

hipError_t launch_sweep_build(const DirDevice& d, int64_t nnz, hipStream_t s) {
    if (nnz == 0) return hipSuccess;
    const int64_t grid = std::min<int64_t>((nnz + kBlock - 1) / kBlock, 8192);
    hipLaunchKernelGGL(sweep_build_kernel, dim3((unsigned)grid), dim3(kBlock), 0, s, d.rows, nnz, d.ptr, d.idx,
                       d.val, d.sw_pk, d.sw_pv);
    return hipGetLastError();
}

hipError_t launch_spmm(const DirDevice& d, int32_t N, float alpha, const float* B, int64_t ldb, float beta,
                       float* C, int64_t ldc, hipStream_t s) {
    const bool vec = (N % 4 == 0) && (ldb % 4 == 0) && (ldc % 4 == 0) &&
                     ((reinterpret_cast<uintptr_t>(B) & 15) == 0) && ((reinterpret_cast<uintptr_t>(C) & 15) == 0);
    const int V = vec ? 4 : 1;
    const int cols = (N + V - 1) / V;  // vector columns
    int G = 1;
    while (G < cols && G < 64) G <<= 1;
    const int ntiles = (cols + G - 1) / G;
    const int n_wave_wg = (d.n_wave + 3) / 4;
    const int64_t grid = (int64_t)d.n_split + d.n_block + n_wave_wg + d.n_group;
    if (grid == 0) return hipSuccess;
    Ctx x{d.ptr, d.idx, d.val, B, ldb, C, ldc, N, alpha, beta};
    size_t lds = (size_t)d.group_cap * 8;
    const size_t red = (size_t)4 * G * V * sizeof(float);
    if (lds < red) lds = red;
    dim3 g3((unsigned)grid, (unsigned)ntiles);
    if (vec) {
        hipLaunchKernelGGL(spmm_bins_kernel<4>, g3, dim3(kBlock), lds, s, d.tasks, d.n_split, d.n_block, d.n_wave,
                           d.n_group, d.xcd_remap, d.split_rows, d.partials, d.counters, G, d.group_cap, x);
    } else {
        hipLaunchKernelGGL(spmm_bins_kernel<1>, g3, dim3(kBlock), lds, s, d.tasks, d.n_split, d.n_block, d.n_wave,
                           d.n_group, d.xcd_remap, d.split_rows, d.partials, d.counters, G, d.group_cap, x);
    }
    return hipGetLastError();
}

}  // namespace spx
