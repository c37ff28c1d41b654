// Measurement probe for bench.py (libspx_probe.so, not part of the product ABI).
//
// Reads a CSR's column and value arrays once, as a one-pass CSR SpMV must
// (「CUDA LSMR 专栏（二）」 §1: at least 8 bytes per entry), and for every entry
// either does nothing else (mode 0: the stream rate), or gathers x[col & mask]
// and accumulates value * x (mode 1: the stream plus the gather of x that
// 「通用稀疏矩阵乘法CUDA算子实现」 §2.5 names as the real cost once x leaves the
// cache).  The mask confines the gathers to a table of mask + 1 floats: the
// whole x, an L2-sized slice, or an L1-sized one.  Row sums are not formed:
// the time is a floor for any one-pass kernel over the same columns.
//
// A wave takes chunks of 1024 entries: four 16-byte loads of columns and of
// values per lane, each instruction covering 64 consecutive 16-byte pieces
// (whole-wave coalesced), then the 16 gathers together.  One float per lane is
// written so that nothing is optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void gather_probe_kernel(const i32x4* __restrict__ col4,
                                                                const f32x4* __restrict__ val4, int64_t chunks,
                                                                const float* __restrict__ x, uint32_t mask, int mode,
                                                                float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t waves = ((int64_t)gridDim.x * kThreads) >> 6;
    float acc = 0.0f;
    for (int64_t ch = wave; ch < chunks; ch += waves) {
        i32x4 c[4];
        f32x4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            c[k] = __builtin_nontemporal_load(col4 + 256 * ch + 64 * k + lane);
            v[k] = __builtin_nontemporal_load(val4 + 256 * ch + 64 * k + lane);
        }
        if (mode == 0) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                acc += v[k].x * (float)(c[k].x & 1) + v[k].y * (float)(c[k].y & 1) + v[k].z * (float)(c[k].z & 1) +
                       v[k].w * (float)(c[k].w & 1);
        } else {
            float g[16];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                g[4 * k + 0] = x[(uint32_t)c[k].x & mask];
                g[4 * k + 1] = x[(uint32_t)c[k].y & mask];
                g[4 * k + 2] = x[(uint32_t)c[k].z & mask];
                g[4 * k + 3] = x[(uint32_t)c[k].w & mask];
            }
#pragma unroll
            for (int k = 0; k < 4; ++k)
                acc += v[k].x * g[4 * k] + v[k].y * g[4 * k + 1] + v[k].z * g[4 * k + 2] + v[k].w * g[4 * k + 3];
        }
    }
    out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

// Feed probe: the rate at which the memory side fills LDS, the operand feed of
// the BSR SpMM (「通用稀疏矩阵乘法CUDA算子实现」 §3.4 stages A and B tiles
// through on-chip memory).  Each wave copies 1 KB pieces into its own
// 16-piece LDS ring with global_load_lds (16 bytes per lane, whole-wave
// coalesced), waiting only when 16 pieces are in flight; nothing is computed.
// Piece i of wave g is (g * stride + i) & mask of a buffer of mask + 1
// pieces: stride 0 gives each wave its own consecutive pieces (a buffer of
// exactly waves x iters pieces is then read once per launch), an odd stride
// spreads the waves over the buffer so that every piece is read many times.
constexpr int kFeedDepth = 16;

constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__global__ __launch_bounds__(kThreads) void feed_probe_kernel(const uint8_t* __restrict__ src, int64_t mask,
                                                              int iters, int64_t stride, float* __restrict__ out) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kThreads / 64][kFeedDepth][1024];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t g = (int64_t)blockIdx.x * (kThreads / 64) + w;
    const int64_t first = stride == 0 ? g * iters : g * stride;
    for (int i = 0; i < iters; ++i) {
        const uint8_t* p = src + ((first + i) & mask) * 1024 + lane * 16;
        __builtin_amdgcn_global_load_lds((const void*)p,
                                         (__attribute__((address_space(3))) void*)&ring[w][i % kFeedDepth][0], 16,
                                         0, 0);
        __builtin_amdgcn_s_waitcnt(vm_wait(kFeedDepth - 1));
    }
    __builtin_amdgcn_s_waitcnt(vm_wait(0));
    __syncthreads();
    out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = (float)ring[w][lane & (kFeedDepth - 1)][lane];
}

}  // namespace

extern "C" {

// Bytes of `out` the probe writes (one float per lane of its grid).
int64_t spx_probe_out_bytes(void) { return (int64_t)256 * 8 * kThreads * 4; }

// Entries the probe covers: the first 1024 * floor(nnz / 1024).
int64_t spx_probe_entries(int64_t nnz) { return nnz < 0 ? 0 : nnz / 1024 * 1024; }

// Runs the probe once over the first spx_probe_entries(nnz) entries of
// col/val (device, 16-byte aligned) on `stream`; x holds at least mask + 1
// floats; out holds spx_probe_out_bytes().  Returns 0, or 1 for a bad
// argument, 2 for a failed launch.
int spx_probe_gather(const int32_t* col, const float* val, int64_t nnz, const float* x, uint32_t mask, int mode,
                     float* out, void* stream) {
    if (!col || !val || !x || !out || nnz < 0) return 1;
    if ((reinterpret_cast<uintptr_t>(col) | reinterpret_cast<uintptr_t>(val)) & 15) return 1;
    const int64_t chunks = nnz / 1024;
    hipLaunchKernelGGL(gather_probe_kernel, dim3(256 * 8), dim3(kThreads), 0, (hipStream_t)stream,
                       reinterpret_cast<const i32x4*>(col), reinterpret_cast<const f32x4*>(val), chunks, x, mask,
                       mode, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Grid of the feed probe: 2 workgroups of 4 waves per CU on 256 CUs.
int64_t spx_feed_probe_waves(void) { return (int64_t)512 * (kThreads / 64); }

// Runs the feed probe once: every wave copies `iters` 1 KB pieces of a buffer
// of `pieces` KB (a power of two; src holds pieces * 1024 bytes, device) as
// described above; out holds 512 * 256 floats.  Returns 0, 1 for a bad
// argument, 2 for a failed launch.
int spx_probe_feed(const uint8_t* src, int64_t pieces, int iters, int64_t stride, float* out, void* stream) {
    if (!src || !out || pieces <= 0 || (pieces & (pieces - 1)) != 0 || iters <= 0 || stride < 0) return 1;
    hipLaunchKernelGGL(feed_probe_kernel, dim3(512), dim3(kThreads), 0, (hipStream_t)stream, src, pieces - 1, iters,
                       stride, out);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
