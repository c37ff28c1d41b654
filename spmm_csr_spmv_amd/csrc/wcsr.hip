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
// column of 64 values per round, coalesced).
//
// SpMM: one workgroup per (window, column tile of C: 32 columns when N <= 32,
// 64 when N <= 64, else 128), one wave per 32 x 32 part of the tile.  Chunks of
// 32 compressed columns: the 32 x 64 slice of values is contiguous, the 32
// gathered B row segments are staged in LDS, and each wave runs
// v_mfma_f32_32x32x2_f32 on its 32 x 32 part of the tile (fp32 in, fp32
// accumulate: the products are the plain fp32 ones of the CSR kernels, only
// the order of the sum differs).  The next chunk is loaded into registers
// while the current one is multiplied.  The page splits large windows into
// tasks and adds their parts with atomics; here a window is one workgroup and
// the many windows of a matrix balance the GPU, so every output is written
// once and the result is reproducible.
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

// flags[0] |= 1: a column outside [0, n);  |= 2: a row not sorted by column.
// Four windows per workgroup, one per wave.
__global__ __launch_bounds__(kBlock) void wcsr_analyze_kernel(int64_t m, int32_t n, int64_t nw, int32_t pad,
                                                              const int32_t* __restrict__ ptr,
                                                              const int32_t* __restrict__ idx,
                                                              int32_t* __restrict__ counts, int32_t* __restrict__ flags) {
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= nw) return;
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
    if (w >= nw) return;
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
// and columns 32 (v / 2) .. +32 of the tile.
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
    const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wr = 32 * (wv & 1), wc = 32 * (wv >> 1);
    const int q0 = window_ptr[w], q1 = window_ptr[w + 1];
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
    // D layout of the 32 x 32 MFMA: lane l, register r -> row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
    const int col = n0 + wc + (l & 31);
    if (col >= N) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t row = w * kWin + wr + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        if (row < m) {
            float* cp = C + row * ldc + col;
            float o = alpha * acc[r];
            if (beta != 0.0f) o = fmaf(beta, *cp, o);
            *cp = o;
        }
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

}  // namespace spx
