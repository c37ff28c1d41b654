// BSR SpMM on MFMA:  C = alpha * A B + beta * C  with A in 64 x 64 bf16
// blocks, B bf16 (row-major), C fp32 (row-major).
//
// 「通用稀疏矩阵乘法CUDA算子实现」 §3.4: for block-sparse A the outer loop runs
// over the non-zero blocks of a block row and the inner work is a small dense
// GEMM, staged through on-chip memory; §5: bf16 storage, fp32 accumulation.
// The AsyncSparse page (§2.2.1, §3) uses 64 x 64 blocks and one output tile per
// (block row, column slice); here that tile is computed with
// v_mfma_f32_32x32x16_bf16.
//
// Workgroup = 4 waves, output tile 64 rows x NT columns (NT = 128 or 64).
// Per block: the 64 x 64 A block goes to LDS row-major (rows padded by 16 B
// so the 16-byte fragment reads of 32 rows hit distinct banks); the 64 x NT
// slice of B goes to LDS with pairs of k rows interleaved, word (p, n) =
// {B[2p][n], B[2p+1][n]}, which is exactly the register image of two
// consecutive k of one column in an MFMA B operand, so a lane's 8-element
// operand is four 32-bit LDS reads.
#include "device_common.h"

namespace spx {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBs = 64;             // block edge
constexpr int kApad = 8;            // bf16 padding per A row in LDS
constexpr int kArow = kBs + kApad;  // LDS row length of A (bf16)

template <int NT>
__global__ __launch_bounds__(kBlock) void bsr_spmm_kernel(const int32_t* __restrict__ brow_ptr,
                                                          const int32_t* __restrict__ bcol,
                                                          const uint16_t* __restrict__ bval,
                                                          const uint16_t* __restrict__ B, int64_t ldb, float alpha,
                                                          float beta, float* __restrict__ C, int64_t ldc, int nnzb,
                                                          int kb_count) {
    static_assert(NT == 128 || NT == 64, "tile width");
    constexpr int TM = NT == 128 ? 2 : 1;  // 32-row MFMA tiles per wave
    __shared__ __attribute__((aligned(16))) uint16_t lA[kBs * kArow];
    __shared__ __attribute__((aligned(16))) uint32_t lB[(kBs / 2) * NT];

    const int I = blockIdx.x;
    const int n_base = blockIdx.y * NT;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    // wave placement inside the 64 x NT tile
    const int w_row = NT == 128 ? 0 : 32 * (w >> 1);
    const int w_col = NT == 128 ? 32 * w : 32 * (w & 1);

    f32x16 acc[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;

    // out-of-range block pointers or block columns are skipped, never read through
    const int kb0 = max(brow_ptr[I], 0), kb1 = min(brow_ptr[I + 1], nnzb);
    for (int kb = kb0; kb < kb1; ++kb) {
        const int J = bcol[kb];
        if (J < 0 || J >= kb_count) continue;  // uniform across the workgroup
        // A block: 512 chunks of 8 bf16, two per thread
        const uint16_t* a_src = bval + (int64_t)kb * (kBs * kBs);
#pragma unroll
        for (int c = tid; c < kBs * kBs / 8; c += kBlock) {
            const int row = c >> 3, ch = c & 7;
            const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a_src + row * kBs + ch * 8));
            *reinterpret_cast<u32x4*>(lA + row * kArow + ch * 8) = v;
        }
        // B slice: rows J*64 .. +64, columns n_base .. +NT; one (k pair, 8-col chunk) per step
        const uint16_t* b_src = B + (int64_t)J * kBs * ldb + n_base;
#pragma unroll
        for (int c = tid; c < (kBs / 2) * (NT / 8); c += kBlock) {
            const int p = c / (NT / 8), ch = c % (NT / 8);
            const u32x4 lo = *reinterpret_cast<const u32x4*>(b_src + (int64_t)(2 * p) * ldb + ch * 8);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(b_src + (int64_t)(2 * p + 1) * ldb + ch * 8);
            u32x4 o0, o1;
            // word i of the output holds column (ch*8 + i): low half from row 2p, high from row 2p+1
            o0.x = (lo.x & 0xffffu) | (hi.x << 16);
            o0.y = (lo.x >> 16) | (hi.x & 0xffff0000u);
            o0.z = (lo.y & 0xffffu) | (hi.y << 16);
            o0.w = (lo.y >> 16) | (hi.y & 0xffff0000u);
            o1.x = (lo.z & 0xffffu) | (hi.z << 16);
            o1.y = (lo.z >> 16) | (hi.z & 0xffff0000u);
            o1.z = (lo.w & 0xffffu) | (hi.w << 16);
            o1.w = (lo.w >> 16) | (hi.w & 0xffff0000u);
            uint32_t* dst = lB + p * NT + ch * 8;
            *reinterpret_cast<u32x4*>(dst) = o0;
            *reinterpret_cast<u32x4*>(dst + 4) = o1;
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < kBs / 16; ++ks) {
            const int k0 = ks * 16 + 8 * (l >> 5);
            // B operand: column w_col + (l & 31), k rows k0 .. k0+7
            u32x4 bw;
            const uint32_t* bsrc = lB + (k0 >> 1) * NT + w_col + (l & 31);
            bw.x = bsrc[0 * NT];
            bw.y = bsrc[1 * NT];
            bw.z = bsrc[2 * NT];
            bw.w = bsrc[3 * NT];
            const bf16x8 bop = __builtin_bit_cast(bf16x8, bw);
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                const int row = w_row + 32 * t + (l & 31);
                const u32x4 aw = *reinterpret_cast<const u32x4*>(lA + row * kArow + k0);
                const bf16x8 aop = __builtin_bit_cast(bf16x8, aw);
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop, acc[t], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // D layout of the 32x32 MFMA: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, column l%32
    const int col = n_base + w_col + (l & 31);
#pragma unroll
    for (int t = 0; t < TM; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = I * kBs + w_row + 32 * t + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
            float* c = C + (int64_t)row * ldc + col;
            float o = alpha * acc[t][r];
            if (beta != 0.0f) o = fmaf(beta, *c, o);
            *c = o;
        }
    }
}

}  // namespace

size_t bsr_work_bytes(int64_t, int64_t, int32_t, int64_t, int32_t) { return 0; }

int bsr_spmm_device(int64_t mb, int64_t kb, int32_t bs, int64_t nnzb, const int32_t* brow_ptr, const int32_t* bcol,
                    const uint16_t* bval, int32_t N, const uint16_t* B, int64_t ldb, float alpha, float beta,
                    float* C, int64_t ldc, void* work, size_t work_bytes, hipStream_t s) {
    (void)work;
    (void)work_bytes;
    (void)bs;
    if (mb == 0 || N == 0) return SP_OK;
    if (N % 128 == 0) {
        hipLaunchKernelGGL(bsr_spmm_kernel<128>, dim3((unsigned)mb, (unsigned)(N / 128)), dim3(kBlock), 0, s,
                           brow_ptr, bcol, bval, B, ldb, alpha, beta, C, ldc, (int)nnzb, (int)kb);
    } else {
        hipLaunchKernelGGL(bsr_spmm_kernel<64>, dim3((unsigned)mb, (unsigned)(N / 64)), dim3(kBlock), 0, s,
                           brow_ptr, bcol, bval, B, ldb, alpha, beta, C, ldc, (int)nnzb, (int)kb);
    }
    return hipGetLastError() == hipSuccess ? SP_OK : SP_ERR_HIP;
}

}  // namespace spx
