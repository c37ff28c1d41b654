// CSR -> BSR conversion and BSR SpMV with fp32 blocks (square bs x bs blocks,
// bs in {1, 2, 4, 8, 16, 32, 64}).
//
// 「GPU加速实战用BCSR格式优化稀疏矩阵乘法附CUDA代码」 §1: a block is stored when it
// holds at least one entry; the format is a block row pointer, a block column
// index per stored block and the dense blocks one after another (row-major,
// §2.1).  The AsyncSparse page §2.2.1 measures the waste of that layout by the
// fill ratio nnz / (nnz_blocks * bs * bs).
//
// Conversion.  One lane per element row; the bs lanes of a block row form an
// aligned lane group and a wave holds 64 / bs block rows.  With the rows
// sorted by column, the block columns of a block row are the merge of its bs
// sorted rows: each round, the group takes the smallest pending block column
// (group-wide minimum), every lane consumes its entries in that block column,
// and the round counts (analyze pass) or writes (fill pass) one block.  In
// the fill pass a lane builds its row of the block in its own LDS slot
// (entries that share a column are added in CSR order, starting from the
// first) and stores the row, so no two lanes ever write the same word.
//
// SpMV.  The blocks of a block row are contiguous, so a wave streams them with
// whole-wave 16-byte loads (lane l holds elements 4l .. 4l+3 of every 256-
// element step).  For bs >= 16 a lane's column slice is the same in every
// step of a block, so the 4 x values it needs are loaded once per block; the
// per-row partial sums are reduced across the lanes of a row at the end (the
// reading of the page's "warp covers whole blocks" strategy on wave64; its
// "warp covers whole columns" strategy is bsr_spmv_rows_kernel below).  For
// bs >= 16 the sixteen waves of a workgroup take the blocks of one block row
// in turn and their row sums are added in wave order; for bs <= 8 each wave
// serves one block row.
#include "device_common.h"

namespace spx {

namespace {

constexpr int kNone = 0x7fffffff;

template <int X>
__device__ __forceinline__ int swz_xor_i(int v) {
    return __builtin_amdgcn_ds_swizzle(v, (X << 10) | 0x1f);
}

// Minimum over aligned groups of g lanes (g a power of two, 1..64).
__device__ __forceinline__ int group_min(int v, int g) {
    if (g >= 2) v = min(v, swz_xor_i<1>(v));
    if (g >= 4) v = min(v, swz_xor_i<2>(v));
    if (g >= 8) v = min(v, swz_xor_i<4>(v));
    if (g >= 16) v = min(v, swz_xor_i<8>(v));
    if (g >= 32) v = min(v, swz_xor_i<16>(v));
    if (g >= 64) v = min(v, __shfl_xor(v, 32, 64));
    return v;
}

// fp32 -> bf16 bit pattern, round to nearest, ties to even (add 0x7fff plus
// the lowest kept bit, keep the upper half); NaN stays NaN (made quiet).
__device__ __forceinline__ uint16_t to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Block column of entry q of a row, or kNone past the row's end; an index
// outside [0, n) ends the row (the analyze pass reports it).
__device__ __forceinline__ int block_col(const int32_t* __restrict__ idx, int q, int qe, int n, int bs) {
    if (q >= qe) return kNone;
    const int c = idx[q];
    return (c >= 0 && c < n) ? c / bs : kNone;
}

// flags[0] |= 1: a column index outside [0, n);  |= 2: a row not sorted by column.
template <int BS>
__global__ __launch_bounds__(64) void bsr_analyze_kernel(int64_t m, int32_t n, int32_t mb,
                                                         const int32_t* __restrict__ ptr,
                                                         const int32_t* __restrict__ idx, int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ flags) {
    constexpr int G = 64 / BS;
    const int l = threadIdx.x, sub = l / BS, r = l % BS;
    const int64_t I = (int64_t)blockIdx.x * G + sub;
    const int64_t i = I * BS + r;
    const bool in = I < mb && i < m;
    int p = in ? ptr[i] : 0;
    const int pe = in ? ptr[i + 1] : 0;
    int bad = 0;
    for (int q = p; q < pe; ++q) {
        const int c = idx[q];
        if (c < 0 || c >= n) bad |= 1;
        if (q > p && c < idx[q - 1]) bad |= 2;
    }
    if (bad) atomicOr(flags, bad);
    int cur = block_col(idx, p, pe, n, BS);
    int count = 0;
    while (true) {
        const int J = group_min(cur, BS);
        if (__all(J == kNone)) break;
        if (J != kNone) {
            ++count;
            while (cur == J) {
                ++p;
                cur = block_col(idx, p, pe, n, BS);
            }
        }
    }
    if (r == 0 && I < mb) counts[I] = count;
}

template <int BS, bool BF16>
__global__ __launch_bounds__(64) void bsr_fill_kernel(int64_t m, int32_t n, int32_t mb, const int32_t* __restrict__ ptr,
                                                      const int32_t* __restrict__ idx, const float* __restrict__ val,
                                                      const int32_t* __restrict__ brow_ptr, int32_t* __restrict__ bcol,
                                                      void* __restrict__ bval) {
    constexpr int G = 64 / BS;
    __shared__ float rowbuf[64 * BS];
    const int l = threadIdx.x, sub = l / BS, r = l % BS;
    const int64_t I = (int64_t)blockIdx.x * G + sub;
    const int64_t i = I * BS + r;
    const bool in = I < mb && i < m;
    int p = in ? ptr[i] : 0;
    const int pe = in ? ptr[i + 1] : 0;
    int k = I < mb ? brow_ptr[I] : 0;
    const int kend = I < mb ? brow_ptr[I + 1] : 0;
    float* rb = rowbuf + l * BS;
    int cur = block_col(idx, p, pe, n, BS);
    while (true) {
        const int J = group_min(cur, BS);
        if (__all(J == kNone)) break;
        if (J != kNone) {
#pragma unroll
            for (int c = 0; c < BS; ++c) rb[c] = 0.0f;
            while (cur == J) {
                const int col = idx[p];
                float v = val[p];
                ++p;
                while (p < pe && idx[p] == col) {
                    v = v + val[p];
                    ++p;
                }
                rb[col % BS] = v;
                cur = block_col(idx, p, pe, n, BS);
            }
            if (k < kend) {  // never past the block row's range, whatever the input
                if (r == 0) bcol[k] = J;
                const int64_t o = ((int64_t)k * BS + r) * BS;
                if constexpr (BF16) {
                    uint16_t* dst = static_cast<uint16_t*>(bval) + o;
#pragma unroll
                    for (int c = 0; c < BS; ++c) dst[c] = to_bf16(rb[c]);
                } else {
                    float* dst = static_cast<float*>(bval) + o;
                    if constexpr (BS % 4 == 0) {
#pragma unroll
                        for (int c = 0; c < BS; c += 4)
                            *reinterpret_cast<float4*>(dst + c) = make_float4(rb[c], rb[c + 1], rb[c + 2], rb[c + 3]);
                    } else {
#pragma unroll
                        for (int c = 0; c < BS; ++c) dst[c] = rb[c];
                    }
                }
            }
            ++k;
        }
    }
}

// x[j .. j+3] with columns >= n read as absent (their products are dropped).
__device__ __forceinline__ float4 load_x4(const float* __restrict__ x, int64_t j, int64_t n) {
    if (j + 4 <= n) return *reinterpret_cast<const float4*>(x + j);
    return make_float4(j < n ? x[j] : 0.0f, j + 1 < n ? x[j + 1] : 0.0f, j + 2 < n ? x[j + 2] : 0.0f,
                       j + 3 < n ? x[j + 3] : 0.0f);
}

__device__ __forceinline__ float dot4(float acc, const float4 a, const float4 xv, int64_t j, int64_t n) {
    acc += j < n ? a.x * xv.x : 0.0f;
    acc += j + 1 < n ? a.y * xv.y : 0.0f;
    acc += j + 2 < n ? a.z * xv.z : 0.0f;
    acc += j + 3 < n ? a.w * xv.w : 0.0f;
    return acc;
}

// bs in {16, 32, 64}: SPLIT workgroups of W waves per block row, workgroup
// (I, part) owning rows [part BS/SPLIT, (part + 1) BS/SPLIT) of block row I,
// i.e. one contiguous slice of every block of the row.  The outputs of the
// workgroups are disjoint, so the sums need no second stage; splitting a long
// block row over several workgroups balances the rows' unequal block counts.
template <int BS, int W, int SPLIT>
__global__ __launch_bounds__(64 * W) void bsr_spmv_big(int64_t m, int64_t n, int32_t kb, int64_t nnzb,
                                                       const int32_t* __restrict__ brow_ptr,
                                                       const int32_t* __restrict__ bcol, const float* __restrict__ bval,
                                                       float alpha, const float* __restrict__ x, float beta,
                                                       float* __restrict__ y) {
    constexpr int RS = BS / SPLIT;                        // rows of the slice
    constexpr int E = RS * BS, P = E / 256, Q = BS / 4;  // slice elements, steps per slice, lanes per row slice
    static_assert(E % 256 == 0, "a slice is whole 256-element steps");
    __shared__ float red[W][RS];
    const int I = blockIdx.x / SPLIT, part = blockIdx.x % SPLIT;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int c = (4 * l) % BS, rloc = (4 * l) / BS;
    const int kb0 = (int)min<int64_t>(max(brow_ptr[I], 0), nnzb), kb1 = (int)min<int64_t>(max(brow_ptr[I + 1], 0), nnzb);
    float acc[P];
#pragma unroll
    for (int ph = 0; ph < P; ++ph) acc[ph] = 0.0f;
    for (int b = kb0 + w; b < kb1; b += W) {
        const int J = bcol[b];
        if (J < 0 || J >= kb) continue;
        const int64_t j = (int64_t)J * BS + c;
        const float4 xv = load_x4(x, j, n);
        const float* blk = bval + (int64_t)b * BS * BS + (int64_t)part * E + 4 * l;
        float4 a[P];
#pragma unroll
        for (int ph = 0; ph < P; ++ph) a[ph] = ldg4_nt(blk + 256 * ph);
#pragma unroll
        for (int ph = 0; ph < P; ++ph) acc[ph] = dot4(acc[ph], a[ph], xv, j, n);
    }
    // rows: step ph, lanes of one row slice share rloc; add the Q lanes of a slice
#pragma unroll
    for (int ph = 0; ph < P; ++ph) {
        float v = group_sum(acc[ph], Q);
        if (l % Q == 0) red[w][ph * (256 / BS) + rloc] = v;
    }
    __syncthreads();
    if (tid < RS) {
        const int64_t row = (int64_t)I * BS + part * RS + tid;
        if (row < m) {
            float s = red[0][tid];
#pragma unroll
            for (int k = 1; k < W; ++k) s += red[k][tid];
            store_axpby(y, (int)row, s, alpha, beta);
        }
    }
}

// bs in {1, 2, 4, 8}: one wave per block row, four block rows per workgroup.
template <int BS>
__global__ __launch_bounds__(kBlock) void bsr_spmv_small(int64_t m, int64_t n, int32_t mb, int32_t kb, int64_t nnzb,
                                                         const int32_t* __restrict__ brow_ptr,
                                                         const int32_t* __restrict__ bcol,
                                                         const float* __restrict__ bval, float alpha,
                                                         const float* __restrict__ x, float beta,
                                                         float* __restrict__ y) {
    constexpr int E = BS * BS;
    const int l = threadIdx.x & 63;
    const int I = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (I >= mb) return;
    const int kb0 = (int)min<int64_t>(max(brow_ptr[I], 0), nnzb), kb1 = (int)min<int64_t>(max(brow_ptr[I + 1], 0), nnzb);
    // lane l holds elements [4l, 4l + 4) of each 256-element step of the block row's stream
    const int64_t e0 = (int64_t)kb0 * E, e1 = (int64_t)kb1 * E;
    float acc0 = 0.0f, acc1 = 0.0f;
    for (int64_t base = e0; base < e1; base += 256) {
        const int64_t e = base + 4 * l;
        if (e >= e1) continue;
        if constexpr (BS == 1) {
            // four 1 x 1 blocks
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (e + t < e1) {
                    const int J = bcol[e + t];
                    if (J >= 0 && J < kb && J < n) acc0 += bval[e + t] * x[J];
                }
            }
        } else {
            const int b = (int)(e / E), o = (int)(e % E), r = o / BS, c = o % BS;
            const int J = bcol[b];
            if (J < 0 || J >= kb) continue;
            const float4 a = ldg4_nt(bval + e);  // e is a multiple of 4 and E >= 4: 16-byte aligned
            const int64_t j = (int64_t)J * BS + c;
            if constexpr (BS == 2) {
                // the whole 2 x 2 block: row 0 = (a.x, a.y), row 1 = (a.z, a.w)
                const float x0 = j < n ? x[j] : 0.0f, x1 = j + 1 < n ? x[j + 1] : 0.0f;
                acc0 += j < n ? a.x * x0 : 0.0f;
                acc0 += j + 1 < n ? a.y * x1 : 0.0f;
                acc1 += j < n ? a.z * x0 : 0.0f;
                acc1 += j + 1 < n ? a.w * x1 : 0.0f;
            } else {
                (void)r;
                acc0 = dot4(acc0, a, load_x4(x, j, n), j, n);
            }
        }
    }
    // add the lanes that hold the same row: all lanes for bs <= 2; for bs = 4
    // the lanes of equal l % 4; for bs = 8 the lanes of equal (l % 16) / 2
    int64_t row0 = (int64_t)I * BS;
    if constexpr (BS <= 2) {
        acc0 = wave_sum(acc0);
        if (BS == 2) acc1 = wave_sum(acc1);
        if (l == 0) {
            if (row0 < m) store_axpby(y, (int)row0, acc0, alpha, beta);
            if (BS == 2 && row0 + 1 < m) store_axpby(y, (int)(row0 + 1), acc1, alpha, beta);
        }
    } else if constexpr (BS == 4) {
        acc0 = cross_group_sum(acc0, 4);
        if (l < 4 && row0 + l < m) store_axpby(y, (int)(row0 + l), acc0, alpha, beta);
    } else {
        acc0 += swz_xor<1>(acc0);
        acc0 += swz_xor<16>(acc0);
        acc0 += __shfl_xor(acc0, 32, 64);
        if (l < 16 && (l & 1) == 0 && row0 + l / 2 < m) store_axpby(y, (int)(row0 + l / 2), acc0, alpha, beta);
    }
}

// The page's second strategy (§2.2, a warp covers whole columns), on wave64:
// each block row is served by a group of BS lanes (64 / BS block rows per
// wave), lane r of the group owns element row r of its block row and walks
// the row's blocks, reading only its own row of each block (BS contiguous
// values, 16-byte loads) and the block column's x segment, so every lane holds
// sums of its own row only and no lanes are reduced together.  As in the
// whole-block kernel, the W waves of a workgroup share the blocks of the same
// block rows (wave w takes every W-th block) and their row sums are added in
// wave order at the end, so that both mappings run with the same parallelism
// and differ only in how a wave reads the blocks.  With 64 x 64 blocks the
// block column is the same for the whole wave, so the x segment is one
// broadcast per block.  The page's trade-off holds: no reduction inside a
// wave, but a lane's block reads are strided by a block row's length.
template <int BS, int W>
__global__ __launch_bounds__(64 * W) void bsr_spmv_rows_kernel(int64_t m, int64_t n, int32_t mb, int32_t kb,
                                                               int64_t nnzb, const int32_t* __restrict__ brow_ptr,
                                                               const int32_t* __restrict__ bcol,
                                                               const float* __restrict__ bval, float alpha,
                                                               const float* __restrict__ x, float beta,
                                                               float* __restrict__ y) {
    constexpr int G = 64 / BS;  // block rows per workgroup (one per lane group)
    __shared__ float red[W][64];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, k = lane / BS, r = lane % BS;
    const int64_t I = (int64_t)blockIdx.x * G + k;
    float acc = 0.0f;
    if (I < mb) {
        const int kb0 = (int)min<int64_t>(max(brow_ptr[I], 0), nnzb);
        const int kb1 = (int)min<int64_t>(max(brow_ptr[I + 1], 0), nnzb);
        for (int b = kb0 + w; b < kb1; b += W) {
            int J = bcol[b];
            if constexpr (BS == 64) J = __builtin_amdgcn_readfirstlane(J);  // one block row per wave
            if (J < 0 || J >= kb) continue;
            const float* __restrict__ arow = bval + (int64_t)b * BS * BS + (int64_t)r * BS;
            const int64_t j0 = (int64_t)J * BS;
            if constexpr (BS >= 4) {
#pragma unroll
                for (int c = 0; c < BS; c += 4)
                    acc = dot4(acc, ldg4_nt(arow + c), load_x4(x, j0 + c, n), j0 + c, n);
            } else {
#pragma unroll
                for (int c = 0; c < BS; ++c)
                    if (j0 + c < n) acc += arow[c] * x[j0 + c];
            }
        }
    }
    red[w][lane] = acc;
    __syncthreads();
    if (w == 0) {
        float t = red[0][lane];
#pragma unroll
        for (int q = 1; q < W; ++q) t += red[q][lane];
        const int64_t row = I * BS + r;
        if (I < mb && row < m) store_axpby(y, (int)row, t, alpha, beta);
    }
}

template <int BS>
int spmv_rows_bs(int64_t m, int64_t n, int64_t nnzb, const int32_t* brow_ptr, const int32_t* bcol, const float* bval,
                 float alpha, const float* x, float beta, float* y, hipStream_t s) {
    const int64_t mb = (m + BS - 1) / BS, kb = (n + BS - 1) / BS;
    if (mb == 0) return SP_OK;
    constexpr int W = 16, G = 64 / BS;
    hipLaunchKernelGGL((bsr_spmv_rows_kernel<BS, W>), dim3((unsigned)((mb + G - 1) / G)), dim3(64 * W), 0, s, m, n,
                       (int32_t)mb, (int32_t)kb, nnzb, brow_ptr, bcol, bval, alpha, x, beta, y);
    return hipGetLastError() == hipSuccess ? SP_OK : SP_ERR_HIP;
}

template <int BS>
int analyze_bs(int64_t m, int64_t n, const int32_t* ptr, const int32_t* idx, int32_t* brow_ptr, int32_t* flags,
               int32_t* sums, hipStream_t s) {
    const int64_t mb = (m + BS - 1) / BS;
    if (launch_fill_i32(brow_ptr, 1, 0, s) != hipSuccess) return SP_ERR_HIP;
    if (mb == 0) return SP_OK;
    const int64_t waves = (mb + (64 / BS) - 1) / (64 / BS);
    hipLaunchKernelGGL(bsr_analyze_kernel<BS>, dim3((unsigned)waves), dim3(64), 0, s, m, (int32_t)n, (int32_t)mb, ptr,
                       idx, brow_ptr + 1, flags);
    if (hipGetLastError() != hipSuccess) return SP_ERR_HIP;
    return scan_inclusive_i32(brow_ptr + 1, mb, sums, s);
}

template <int BS>
int fill_bs(int64_t m, int64_t n, const int32_t* ptr, const int32_t* idx, const float* val, const int32_t* brow_ptr,
            int32_t* bcol, void* bval, int32_t out_bf16, hipStream_t s) {
    const int64_t mb = (m + BS - 1) / BS;
    if (mb == 0) return SP_OK;
    const int64_t waves = (mb + (64 / BS) - 1) / (64 / BS);
    if (out_bf16) {
        hipLaunchKernelGGL((bsr_fill_kernel<BS, true>), dim3((unsigned)waves), dim3(64), 0, s, m, (int32_t)n,
                           (int32_t)mb, ptr, idx, val, brow_ptr, bcol, bval);
    } else {
        hipLaunchKernelGGL((bsr_fill_kernel<BS, false>), dim3((unsigned)waves), dim3(64), 0, s, m, (int32_t)n,
                           (int32_t)mb, ptr, idx, val, brow_ptr, bcol, bval);
    }
    return hipGetLastError() == hipSuccess ? SP_OK : SP_ERR_HIP;
}

template <int BS>
int spmv_bs(int64_t m, int64_t n, int64_t nnzb, const int32_t* brow_ptr, const int32_t* bcol, const float* bval,
            float alpha, const float* x, float beta, float* y, hipStream_t s) {
    const int64_t mb = (m + BS - 1) / BS, kb = (n + BS - 1) / BS;
    if (mb == 0) return SP_OK;
    if constexpr (BS >= 16) {
        // 64 x 64 blocks: four 16-row slices per block row; smaller blocks: the
        // whole block row in one workgroup; 16 waves per workgroup
        constexpr int SPLIT = BS == 64 ? 4 : 1, W = 16;
        hipLaunchKernelGGL((bsr_spmv_big<BS, W, SPLIT>), dim3((unsigned)(mb * SPLIT)), dim3(64 * W), 0, s, m, n,
                           (int32_t)kb, nnzb, brow_ptr, bcol, bval, alpha, x, beta, y);
    } else {
        hipLaunchKernelGGL(bsr_spmv_small<BS>, dim3((unsigned)((mb + 3) / 4)), dim3(kBlock), 0, s, m, n,
                           (int32_t)mb, (int32_t)kb, nnzb, brow_ptr, bcol, bval, alpha, x, beta, y);
    }
    return hipGetLastError() == hipSuccess ? SP_OK : SP_ERR_HIP;
}

}  // namespace

// workspace: [16 flag words | scan partial sums]
size_t bsr_convert_work_bytes(int64_t m, int32_t bs) {
    const int64_t mb = bs > 0 ? (m + bs - 1) / bs : 0;
    return 256 + scan_work_bytes(mb);
}

int csr_to_bsr_analyze_device(int64_t m, int64_t n, const int32_t* row_ptr, const int32_t* col_idx, int32_t bs,
                              int32_t* brow_ptr, void* work, hipStream_t s, int32_t* flags_host) {
    int32_t* flags = static_cast<int32_t*>(work);
    int32_t* sums = reinterpret_cast<int32_t*>(static_cast<char*>(work) + 256);
    if (launch_fill_i32(flags, 1, 0, s) != hipSuccess) return SP_ERR_HIP;
    int rc;
    switch (bs) {
        case 1: rc = analyze_bs<1>(m, n, row_ptr, col_idx, brow_ptr, flags, sums, s); break;
        case 2: rc = analyze_bs<2>(m, n, row_ptr, col_idx, brow_ptr, flags, sums, s); break;
        case 4: rc = analyze_bs<4>(m, n, row_ptr, col_idx, brow_ptr, flags, sums, s); break;
        case 8: rc = analyze_bs<8>(m, n, row_ptr, col_idx, brow_ptr, flags, sums, s); break;
        case 16: rc = analyze_bs<16>(m, n, row_ptr, col_idx, brow_ptr, flags, sums, s); break;
        case 32: rc = analyze_bs<32>(m, n, row_ptr, col_idx, brow_ptr, flags, sums, s); break;
        case 64: rc = analyze_bs<64>(m, n, row_ptr, col_idx, brow_ptr, flags, sums, s); break;
        default: return SP_ERR_UNSUPPORTED;
    }
    if (rc != SP_OK) return rc;
    if (hipMemcpyAsync(flags_host, flags, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess) return SP_ERR_HIP;
    return SP_OK;
}

int csr_to_bsr_fill_device(int64_t m, int64_t n, const int32_t* row_ptr, const int32_t* col_idx, const float* val,
                           int32_t bs, const int32_t* brow_ptr, int32_t* bcol, void* bval, int32_t out_bf16,
                           hipStream_t s) {
    switch (bs) {
        case 1: return fill_bs<1>(m, n, row_ptr, col_idx, val, brow_ptr, bcol, bval, out_bf16, s);
        case 2: return fill_bs<2>(m, n, row_ptr, col_idx, val, brow_ptr, bcol, bval, out_bf16, s);
        case 4: return fill_bs<4>(m, n, row_ptr, col_idx, val, brow_ptr, bcol, bval, out_bf16, s);
        case 8: return fill_bs<8>(m, n, row_ptr, col_idx, val, brow_ptr, bcol, bval, out_bf16, s);
        case 16: return fill_bs<16>(m, n, row_ptr, col_idx, val, brow_ptr, bcol, bval, out_bf16, s);
        case 32: return fill_bs<32>(m, n, row_ptr, col_idx, val, brow_ptr, bcol, bval, out_bf16, s);
        case 64: return fill_bs<64>(m, n, row_ptr, col_idx, val, brow_ptr, bcol, bval, out_bf16, s);
        default: return SP_ERR_UNSUPPORTED;
    }
}

int bsr_spmv_device(int64_t m, int64_t n, int32_t bs, int64_t nnzb, const int32_t* brow_ptr, const int32_t* bcol,
                    const float* bval, float alpha, const float* x, float beta, float* y, hipStream_t s) {
    switch (bs) {
        case 1: return spmv_bs<1>(m, n, nnzb, brow_ptr, bcol, bval, alpha, x, beta, y, s);
        case 2: return spmv_bs<2>(m, n, nnzb, brow_ptr, bcol, bval, alpha, x, beta, y, s);
        case 4: return spmv_bs<4>(m, n, nnzb, brow_ptr, bcol, bval, alpha, x, beta, y, s);
        case 8: return spmv_bs<8>(m, n, nnzb, brow_ptr, bcol, bval, alpha, x, beta, y, s);
        case 16: return spmv_bs<16>(m, n, nnzb, brow_ptr, bcol, bval, alpha, x, beta, y, s);
        case 32: return spmv_bs<32>(m, n, nnzb, brow_ptr, bcol, bval, alpha, x, beta, y, s);
        case 64: return spmv_bs<64>(m, n, nnzb, brow_ptr, bcol, bval, alpha, x, beta, y, s);
        default: return SP_ERR_UNSUPPORTED;
    }
}

int bsr_spmv_rows_device(int64_t m, int64_t n, int32_t bs, int64_t nnzb, const int32_t* brow_ptr, const int32_t* bcol,
                         const float* bval, float alpha, const float* x, float beta, float* y, hipStream_t s) {
    switch (bs) {
        case 1: return spmv_rows_bs<1>(m, n, nnzb, brow_ptr, bcol, bval, alpha, x, beta, y, s);
        case 2: return spmv_rows_bs<2>(m, n, nnzb, brow_ptr, bcol, bval, alpha, x, beta, y, s);
        case 4: return spmv_rows_bs<4>(m, n, nnzb, brow_ptr, bcol, bval, alpha, x, beta, y, s);
        case 8: return spmv_rows_bs<8>(m, n, nnzb, brow_ptr, bcol, bval, alpha, x, beta, y, s);
        case 16: return spmv_rows_bs<16>(m, n, nnzb, brow_ptr, bcol, bval, alpha, x, beta, y, s);
        case 32: return spmv_rows_bs<32>(m, n, nnzb, brow_ptr, bcol, bval, alpha, x, beta, y, s);
        case 64: return spmv_rows_bs<64>(m, n, nnzb, brow_ptr, bcol, bval, alpha, x, beta, y, s);
        default: return SP_ERR_UNSUPPORTED;
    }
}

}  // namespace spx
