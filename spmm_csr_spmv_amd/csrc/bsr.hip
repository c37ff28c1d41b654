// BSR SpMM on MFMA:  C = alpha * A B + beta * C  with A in 64 x 64 bf16
// blocks, B bf16 (row-major), C fp32 (row-major).
//
// 「通用稀疏矩阵乘法CUDA算子实现」 §3.4: for block-sparse A the outer loop runs
// over the non-zero blocks of a block row and the inner work is a small dense
// GEMM, staged through on-chip memory with loads overlapped with compute; §5:
// bf16 storage, fp32 accumulation.  The AsyncSparse page (§2.2.1, §3, §6.1)
// uses 64 x 64 blocks and one output tile per (block row, column slice).
//
// Workgroup = 4 waves, output tile 64 rows x NT columns; the tile is computed
// with v_mfma_f32_32x32x16_bf16.  Per block: the 64 x 64 A block goes to LDS
// row-major (rows padded by 16 B so the 16-byte fragment reads of 32 rows hit
// distinct banks); the 64 x NT slice of B goes to LDS with pairs of k rows
// interleaved, word (p, n) = {B[2p][n], B[2p+1][n]}, which is the register
// image of two consecutive k of one column in an MFMA B operand, so a lane's
// 8-element B operand is four 32-bit LDS reads.
#include "device_common.h"

namespace spx {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBs = 64;             // block edge
constexpr int kApad = 8;            // bf16 padding per A row in LDS
constexpr int kArow = kBs + kApad;  // LDS row length of A (bf16)

// Interleave two rows of 8 bf16 (lo = row 2p, hi = row 2p+1) into 8 words
// {lo[i], hi[i]}.
__device__ __forceinline__ void pair_rows(const u32x4 lo, const u32x4 hi, u32x4& o0, u32x4& o1) {
    o0.x = (lo.x & 0xffffu) | (hi.x << 16);
    o0.y = (lo.x >> 16) | (hi.x & 0xffff0000u);
    o0.z = (lo.y & 0xffffu) | (hi.y << 16);
    o0.w = (lo.y >> 16) | (hi.y & 0xffff0000u);
    o1.x = (lo.z & 0xffffu) | (hi.z << 16);
    o1.y = (lo.z >> 16) | (hi.z & 0xffff0000u);
    o1.z = (lo.w & 0xffffu) | (hi.w << 16);
    o1.w = (lo.w >> 16) | (hi.w & 0xffff0000u);
}

// ---------------------------------------------------------------------------
// Simple kernel for N % 64 == 0 (tile 64 x 64, one 32 x 32 MFMA tile per
// wave, no prefetch).  Serves the widths the pipelined kernel does not.
__global__ __launch_bounds__(kBlock) void bsr_spmm_n64(const int32_t* __restrict__ brow_ptr,
                                                       const int32_t* __restrict__ bcol,
                                                       const uint16_t* __restrict__ bval,
                                                       const uint16_t* __restrict__ B, int64_t ldb, float alpha,
                                                       float beta, float* __restrict__ C, int64_t ldc, int nnzb,
                                                       int kb_count) {
    constexpr int NT = 64;
    __shared__ __attribute__((aligned(16))) uint16_t lA[kBs * kArow];
    __shared__ __attribute__((aligned(16))) uint32_t lB[(kBs / 2) * NT];
    const int I = blockIdx.x;
    const int n_base = blockIdx.y * NT;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int w_row = 32 * (w >> 1), w_col = 32 * (w & 1);
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    // out-of-range block pointers or block columns are skipped, never read through
    const int kb0 = max(brow_ptr[I], 0), kb1 = min(brow_ptr[I + 1], nnzb);
    for (int kb = kb0; kb < kb1; ++kb) {
        const int J = bcol[kb];
        if (J < 0 || J >= kb_count) continue;  // uniform across the workgroup
        const uint16_t* a_src = bval + (int64_t)kb * (kBs * kBs);
        for (int c = tid; c < kBs * kBs / 8; c += kBlock)
            *reinterpret_cast<u32x4*>(lA + (c >> 3) * kArow + (c & 7) * 8) =
                __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a_src + (c >> 3) * kBs + (c & 7) * 8));
        const uint16_t* b_src = B + (int64_t)J * kBs * ldb + n_base;
        for (int c = tid; c < (kBs / 2) * (NT / 8); c += kBlock) {
            const int p = c / (NT / 8), ch = c % (NT / 8);
            u32x4 o0, o1;
            pair_rows(*reinterpret_cast<const u32x4*>(b_src + (int64_t)(2 * p) * ldb + ch * 8),
                      *reinterpret_cast<const u32x4*>(b_src + (int64_t)(2 * p + 1) * ldb + ch * 8), o0, o1);
            *reinterpret_cast<u32x4*>(lB + p * NT + ch * 8) = o0;
            *reinterpret_cast<u32x4*>(lB + p * NT + ch * 8 + 4) = o1;
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < kBs / 16; ++ks) {
            const int k0 = ks * 16 + 8 * (l >> 5);
            const uint32_t* bsrc = lB + (k0 >> 1) * NT + w_col + (l & 31);
            const u32x4 bw = {bsrc[0], bsrc[NT], bsrc[2 * NT], bsrc[3 * NT]};
            const u32x4 aw = *reinterpret_cast<const u32x4*>(lA + (w_row + (l & 31)) * kArow + k0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, aw), __builtin_bit_cast(bf16x8, bw),
                                                          acc, 0, 0, 0);
        }
        __syncthreads();
    }
    // D layout of the 32x32 MFMA: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, column l%32
    const int col = n_base + w_col + (l & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = I * kBs + w_row + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        float* c = C + (int64_t)row * ldc + col;
        float o = alpha * acc[r];
        if (beta != 0.0f) o = fmaf(beta, *c, o);
        *c = o;
    }
}

// ---------------------------------------------------------------------------
// Pipelined kernel for N % NT == 0, NT = 128 or 256.  Wave w owns columns
// [w NT/4, (w+1) NT/4) of the tile as 2 x (NT/128) MFMA tiles of 32 x 32, so
// every A operand read from LDS feeds NT/128 MFMAs and every B operand two.
// The next block's A and B are loaded into registers while the current
// block's MFMAs run.  Loads are issued without branches (block index clamped,
// data zeroed for a block past the row's end or with an out-of-range column)
// so the compiler waits for exactly the registers it needs.
//
// Workgroups are mapped to XCDs (workgroup id mod 8) so that the XCDs are
// split evenly between the column tiles: each XCD's L2 then caches only the
// B columns of its own tile.
template <int NT>
__global__ __launch_bounds__(kBlock) void bsr_spmm_pipelined(const int32_t* __restrict__ brow_ptr,
                                                             const int32_t* __restrict__ bcol,
                                                             const uint16_t* __restrict__ bval,
                                                             const uint16_t* __restrict__ B, int64_t ldb, float alpha,
                                                             float beta, float* __restrict__ C, int64_t ldc, int nnzb,
                                                             int kb_count, int mb, int ntiles, int xcd_split) {
    static_assert(NT == 128 || NT == 256, "tile width");
    constexpr int UC = NT / 128;         // 32-column MFMA tiles per wave
    constexpr int BROW = NT + 8;         // LDS words per k-pair row of B (padded)
    constexpr int BITEMS = NT / 64;      // (k pair, 8-column chunk) items per thread
    constexpr int CHUNKS = NT / 8;       // 8-column chunks per row of the slice
    __shared__ __attribute__((aligned(16))) uint16_t lA[kBs * kArow];
    __shared__ __attribute__((aligned(16))) uint32_t lB[(kBs / 2) * BROW];

    // ---- work item -> (block row, column tile)
    int I, tile;
    const int b = blockIdx.x;
    if (xcd_split) {
        const int per = 8 / ntiles;  // XCDs per column tile
        const int x = b & 7;
        tile = x / per;
        I = (b >> 3) * per + (x % per);
    } else {
        I = b / ntiles;
        tile = b % ntiles;
    }
    if (I >= mb) return;
    const int n_base = tile * NT;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int w_col = w * (NT / 4);

    f32x16 acc[2][UC];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < UC; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[t][u][r] = 0.0f;

    // per-thread share of a block: A chunks c = tid, tid + 256 (row c/8, chunk c%8);
    // B items c = tid + 256 j: k pair p = c / CHUNKS, chunk ch = c % CHUNKS
    u32x4 ra[2], rlo[BITEMS], rhi[BITEMS];
    uint32_t keep = 0;
    auto fetch = [&](int kb, bool live) {
        const int J0 = bcol[kb];
        const bool valid = J0 >= 0 && J0 < kb_count;
        const int J = valid ? J0 : 0;
        const uint16_t* a_src = bval + (int64_t)kb * (kBs * kBs);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int c = tid + kBlock * j;
            ra[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a_src + (c >> 3) * kBs + (c & 7) * 8));
        }
        const uint16_t* b_src = B + (int64_t)J * kBs * ldb + n_base;
#pragma unroll
        for (int j = 0; j < BITEMS; ++j) {
            const int c = tid + kBlock * j;
            const int p = c / CHUNKS, ch = c % CHUNKS;
            rlo[j] = *reinterpret_cast<const u32x4*>(b_src + (int64_t)(2 * p) * ldb + ch * 8);
            rhi[j] = *reinterpret_cast<const u32x4*>(b_src + (int64_t)(2 * p + 1) * ldb + ch * 8);
        }
        // applied when the registers are staged, not here: masking loaded data
        // right away would make the compiler wait for the loads at this point
        keep = (live && valid) ? 0xffffffffu : 0u;
    };
    auto stage = [&]() {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int c = tid + kBlock * j;
            *reinterpret_cast<u32x4*>(lA + (c >> 3) * kArow + (c & 7) * 8) = ra[j] & keep;
        }
#pragma unroll
        for (int j = 0; j < BITEMS; ++j) {
            const int c = tid + kBlock * j;
            const int p = c / CHUNKS, ch = c % CHUNKS;
            u32x4 o0, o1;
            pair_rows(rlo[j] & keep, rhi[j] & keep, o0, o1);
            uint32_t* dst = lB + p * BROW + ch * 8;
            *reinterpret_cast<u32x4*>(dst) = o0;
            *reinterpret_cast<u32x4*>(dst + 4) = o1;
        }
    };
    auto compute = [&]() {
#pragma unroll
        for (int ks = 0; ks < kBs / 16; ++ks) {
            const int k0 = ks * 16 + 8 * (l >> 5);
            bf16x8 bop[UC], aop[2];
#pragma unroll
            for (int u = 0; u < UC; ++u) {
                const uint32_t* bsrc = lB + (k0 >> 1) * BROW + w_col + 32 * u + (l & 31);
                const u32x4 bw = {bsrc[0], bsrc[BROW], bsrc[2 * BROW], bsrc[3 * BROW]};
                bop[u] = __builtin_bit_cast(bf16x8, bw);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const u32x4 aw = *reinterpret_cast<const u32x4*>(lA + (32 * t + (l & 31)) * kArow + k0);
                aop[t] = __builtin_bit_cast(bf16x8, aw);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int u = 0; u < UC; ++u)
                    acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[t], bop[u], acc[t][u], 0, 0, 0);
        }
    };

    const int kb0 = max(brow_ptr[I], 0), kb1 = min(brow_ptr[I + 1], nnzb);
    if (kb0 < kb1) {
        const int last = kb1 - 1;
        fetch(kb0, true);
        for (int kb = kb0; kb < kb1; ++kb) {
            stage();
            __syncthreads();
            fetch(min(kb + 1, last), kb + 1 <= last);  // in flight during the MFMAs below
            compute();
            __syncthreads();
        }
    }

    // D layout of the 32x32 MFMA: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int u = 0; u < UC; ++u) {
            const int col = n_base + w_col + 32 * u + (l & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = I * kBs + 32 * t + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
                float* c = C + (int64_t)row * ldc + col;
                float o = alpha * acc[t][u][r];
                if (beta != 0.0f) o = fmaf(beta, *c, o);
                *c = o;
            }
        }
    }
}

template <int NT>
hipError_t launch_pipelined(int64_t mb, int64_t kb, int64_t nnzb, const int32_t* brow_ptr, const int32_t* bcol,
                            const uint16_t* bval, int32_t N, const uint16_t* B, int64_t ldb, float alpha, float beta,
                            float* C, int64_t ldc, hipStream_t s) {
    const int ntiles = N / NT;
    const int split = (ntiles > 1 && 8 % ntiles == 0) ? 1 : 0;
    const int per = split ? 8 / ntiles : 1;
    const int64_t grid = split ? ((mb + per - 1) / per) * 8 : mb * ntiles;
    hipLaunchKernelGGL(bsr_spmm_pipelined<NT>, dim3((unsigned)grid), dim3(kBlock), 0, s, brow_ptr, bcol, bval, B, ldb,
                       alpha, beta, C, ldc, (int)nnzb, (int)kb, (int)mb, ntiles, split);
    return hipGetLastError();
}

}  // namespace

size_t bsr_work_bytes(int64_t, int64_t, int32_t, int64_t, int32_t) { return 0; }

// Tile width of the pipelined kernel for wide N (128 or 256).
constexpr int kBsrTile = 256;

int bsr_spmm_device(int64_t mb, int64_t kb, int32_t bs, int64_t nnzb, const int32_t* brow_ptr, const int32_t* bcol,
                    const uint16_t* bval, int32_t N, const uint16_t* B, int64_t ldb, float alpha, float beta,
                    float* C, int64_t ldc, void* work, size_t work_bytes, hipStream_t s) {
    (void)work;
    (void)work_bytes;
    (void)bs;
    if (mb == 0 || N == 0) return SP_OK;
    hipError_t err;
    if (N % kBsrTile == 0) {
        err = launch_pipelined<kBsrTile>(mb, kb, nnzb, brow_ptr, bcol, bval, N, B, ldb, alpha, beta, C, ldc, s);
    } else if (N % 128 == 0) {
        err = launch_pipelined<128>(mb, kb, nnzb, brow_ptr, bcol, bval, N, B, ldb, alpha, beta, C, ldc, s);
    } else {
        hipLaunchKernelGGL(bsr_spmm_n64, dim3((unsigned)mb, (unsigned)(N / 64)), dim3(kBlock), 0, s, brow_ptr, bcol,
                           bval, B, ldb, alpha, beta, C, ldc, (int)nnzb, (int)kb);
        err = hipGetLastError();
    }
    return err == hipSuccess ? SP_OK : SP_ERR_HIP;
}

}  // namespace spx
