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

}  // namespace

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
