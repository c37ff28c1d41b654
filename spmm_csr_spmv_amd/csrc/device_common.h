// Device helpers shared by the kernels: wave64 reductions, XCD-aware
// workgroup remapping and guarded vector loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace spx {

// ---------------------------------------------------------------- wave64 sums
// ds_swizzle in bit-mask mode: lane i (within its 32-lane half) reads lane
// (i & 0x1f) ^ XOR.  All 64 lanes must execute these (the callers keep the
// whole wave active through every reduction).
template <int XOR>
__device__ __forceinline__ float swz_xor(float v) {
    static_assert(XOR > 0 && XOR < 32, "swizzle xor mask is 5 bits");
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (XOR << 10) | 0x1f));
}

// Sum over aligned groups of g lanes (g a power of two, 1..64); every lane of
// a group gets the group's sum.  The reduction tree is fixed by g, so the
// result is bitwise reproducible.
__device__ __forceinline__ float group_sum(float v, int g) {
    if (g >= 2) v += swz_xor<1>(v);
    if (g >= 4) v += swz_xor<2>(v);
    if (g >= 8) v += swz_xor<4>(v);
    if (g >= 16) v += swz_xor<8>(v);
    if (g >= 32) v += swz_xor<16>(v);
    if (g >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// Sum of all 64 lanes, valid in every lane.
__device__ __forceinline__ float wave_sum(float v) {
    v += swz_xor<1>(v);
    v += swz_xor<2>(v);
    v += swz_xor<4>(v);
    v += swz_xor<8>(v);
    v += swz_xor<16>(v);
    // lanes 0..31 hold the low half's sum, 32..63 the high half's
    const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    return lo + hi;
}

// Sum across lanes that share (lane % g): reduces the 64/g sub-groups of a
// wave onto every lane, keeping the per-lane column slot.
__device__ __forceinline__ float cross_group_sum(float v, int g) {
    if (g <= 1) v += swz_xor<1>(v);
    if (g <= 2) v += swz_xor<2>(v);
    if (g <= 4) v += swz_xor<4>(v);
    if (g <= 8) v += swz_xor<8>(v);
    if (g <= 16) v += swz_xor<16>(v);
    if (g <= 32) v += __shfl_xor(v, 32, 64);
    return v;
}

// ------------------------------------------------------- XCD-aware remapping
// The dispatcher hands workgroup b of a launch to XCD (b % 8).  For the
// workgroups in [first, first + count) this returns a task index in
// [0, count) such that every XCD receives one contiguous run of tasks, so
// neighbouring tasks (which touch neighbouring columns of x) share an L2.
__device__ __forceinline__ int xcd_contiguous(int b, int first, int count) {
    const int k = b & (kXcds - 1);
    int start = 0;
    for (int j = 0; j < k; ++j) {
        const int off = (j - first) & (kXcds - 1);  // first workgroup >= first on XCD j
        start += off < count ? (count - off + kXcds - 1) / kXcds : 0;
    }
    const int off_k = (k - first) & (kXcds - 1);
    return start + (b - first - off_k) / kXcds;
}

// ---------------------------------------------------------- memory helpers
__device__ __forceinline__ int4 ldg4(const int32_t* p) { return *reinterpret_cast<const int4*>(p); }
__device__ __forceinline__ float4 ldg4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// Loads that stream through the caches with the non-temporal hint (the matrix
// arrays are read exactly once per product).
typedef int32_t v4i32 __attribute__((ext_vector_type(4)));
typedef float v4f32 __attribute__((ext_vector_type(4)));
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int4 ldg4_nt(const int32_t* p) {
    const v4i32 v = __builtin_nontemporal_load(reinterpret_cast<const v4i32*>(p));
    return make_int4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 ldg4_nt(const float* p) {
    const v4f32 v = __builtin_nontemporal_load(reinterpret_cast<const v4f32*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float atomic_load_f(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_f(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------- streamed products
// Products val[q] * x[idx[q]] for q in [b, e).  Lane `lane` of `stride`
// lanes owns the 4-entry chunks starting at (b & ~3) + 4*lane + 4*stride*k.
// Chunks are taken U at a time: the U column/value loads (16-byte loads for
// full chunks, guarded scalar loads at the ragged ends) are all issued before
// the gathers of x, and all gathers before any product, so every lane keeps
// up to 8U independent memory requests in flight.  `emit(q, prod)` receives
// each valid product; slots outside [b, e) are never read nor multiplied.
template <int U, class Emit>
__device__ __forceinline__ void stream_products(const int32_t* __restrict__ idx, const float* __restrict__ val,
                                                const float* __restrict__ x, int b, int e, int lane, int stride,
                                                Emit emit) {
    const int base = b & ~3;
    for (int v0 = base + 4 * lane; v0 < e; v0 += 4 * stride * U) {
        int c[U][4];
        float a[U][4];
        bool ok[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + 4 * stride * u;
            if (v >= b && v + 4 <= e) {
                const int4 ci = ldg4_nt(idx + v);
                const float4 ai = ldg4_nt(val + v);
                c[u][0] = ci.x; c[u][1] = ci.y; c[u][2] = ci.z; c[u][3] = ci.w;
                a[u][0] = ai.x; a[u][1] = ai.y; a[u][2] = ai.z; a[u][3] = ai.w;
#pragma unroll
                for (int j = 0; j < 4; ++j) ok[u][j] = true;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int q = v + j;
                    ok[u][j] = q >= b && q < e;
                    c[u][j] = ok[u][j] ? idx[q] : 0;
                    a[u][j] = ok[u][j] ? val[q] : 0.0f;
                }
            }
        }
        float xv[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) xv[u][j] = ok[u][j] ? x[c[u][j]] : 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + 4 * stride * u;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (ok[u][j]) emit(v + j, a[u][j] * xv[u][j]);
        }
    }
}

__device__ __forceinline__ void store_axpby(float* __restrict__ y, int row, float acc, float alpha, float beta) {
    float o = alpha * acc;
    if (beta != 0.0f) o = fmaf(beta, y[row], o);
    y[row] = o;
}

}  // namespace spx
