// BSR SpMM on MFMA:  C = alpha * A B + beta * C  with A in 64 x 64 bf16
// blocks, B bf16 (row-major), C fp32 (row-major).
//
// 「通用稀疏矩阵乘法CUDA算子实现」 §3.4: for block-sparse A the outer loop runs
// over the non-zero blocks of a block row and the inner work is a small dense
// GEMM, staged through on-chip memory with loads overlapped with compute; §5:
// bf16 storage, fp32 accumulation.  The AsyncSparse page (§2.2.1, §3, §6.1)
// uses 64 x 64 blocks and one output tile per (block row, column slice).
//
// One workgroup per (block row, column tile of C); all tiles are computed with
// v_mfma_f32_32x32x16_bf16 on fp32 accumulators.  Three kernels by width:
//   N % 256 == 0: copy-engine kernel (global_load_lds into a four-stage LDS
//                 ring, B operands by LDS transpose reads, copy waves apart
//                 from MFMA waves);
//   N % 128 == 0: register-prefetch kernel, B repacked into k-pair words;
//   otherwise:    plain kernel, one 64 x 64 tile, no prefetch; the last
//                 tile's columns past N (N % 8 == 0) are neither read nor written.
// Each block contributes A_blk B[J*64 : J*64+64, tile] to its block row's tile.
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
// Simple kernel for any N % 8 == 0 (tile 64 x 64, one 32 x 32 MFMA tile per
// wave, no prefetch).  Serves the widths the pipelined kernels do not; in the
// last tile the 8-column chunks of B at or past N load as zeros and those
// columns of C are not stored ([GEN] §6.1 pads B to the tile width instead).
__global__ __launch_bounds__(kBlock) void bsr_spmm_n64(const int32_t* __restrict__ brow_ptr,
                                                       const int32_t* __restrict__ bcol,
                                                       const uint16_t* __restrict__ bval,
                                                       const uint16_t* __restrict__ B, int64_t ldb, float alpha,
                                                       float beta, float* __restrict__ C, int64_t ldc, int nnzb,
                                                       int kb_count, int N) {
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
            u32x4 o0 = {0u, 0u, 0u, 0u}, o1 = {0u, 0u, 0u, 0u};
            if (n_base + ch * 8 < N)  // whole 8-column chunks (N % 8 == 0)
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
    if (col >= N) return;
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
// Pipelined kernel for N % NT == 0 with NT = 128 (widths that the copy-engine
// kernel does not take; the template also builds NT = 256).  Wave w owns columns
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

// ---------------------------------------------------------------------------
// Copy-engine kernel for N % 256 == 0 (gfx950).
//
// Tile 64 x NT (NT = 256) per workgroup of eight waves.  Waves 0..3 compute:
// wave w owns columns [w NT/4, (w+1) NT/4) as 2 x (NT/128) MFMA tiles of
// 32 x 32.  Waves 4..7 only copy.  The k dimension advances in stages of half
// a block (32 k); four stages are in flight.  A stage is filled by
// global_load_lds (16 bytes per lane straight into LDS, no registers, no
// repacking).  The copy waves stall whenever the memory pipeline is full; as
// they issue no MFMAs, the compute waves keep the matrix cores fed meanwhile.
// With 80 KB of LDS per workgroup two workgroups share a CU.
//
// LDS layouts (16-byte chunks, XOR-swizzled so the operand reads spread over
// the banks; a copy instruction fills 1 KB of consecutive chunks and each
// lane picks the source chunk that belongs at its position):
//   A stage: row r (64 rows) x 4 chunks of 8 k;  chunk c of row r at 4 r + (c ^ fa(r)).
//   B stage: row k (32 rows) x NT/8 chunks of 8 columns, B's own row-major
//            order;  chunk c of row k at k NT/8 + (c ^ gb(k)).
// A operands are one 16-byte LDS read per lane.  B operands come from
// ds_read_b64_tr_b16: within each 16-lane group it returns to lane 4a + b,
// element e, the b-th 16-bit value of the 8-byte row addressed by lane
// a + 4e.  Addressing lane L at row 4 i + 8 (L / 32) + (L % 16) / 4 and
// column 16 ((L / 16) % 2) + 4 (L % 4) therefore gives lane L the values
// B[8 (L / 32) + 4 i + e][L % 32], e = 0..3: half i of the MFMA B operand.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kKh = 32;      // k rows per stage
constexpr int kStages = 4;   // stages in flight

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding and leaves the other counters alone (vmcnt in bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int NT>
struct DmaShape {
    static constexpr int kABytes = kBs * kKh * 2;                 // 4 KB
    static constexpr int kBBytes = kKh * NT * 2;                  // 16 or 32 KB
    static constexpr int kBChunks = NT / 8;                       // chunks per B row
    static constexpr int kBCopies = kBBytes / (kBlock * 16);      // B copy instructions per thread
    static constexpr int kPerStage = 1 + kBCopies;                // copy instructions per thread per stage
    static constexpr int kUC = NT / 128;                          // 32-column MFMA tiles per wave
};

__device__ __forceinline__ int dma_fa(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }
__device__ __forceinline__ int dma_gb(int k) { return (k & 3) << 2; }

// Issue the copies of stage h (block kb0 + h/2 with column index J0, k half
// h%2) into (la, lb); w is the copying wave's index (0..3).  A block with an
// out-of-range column index still copies (from block column 0) so that the
// count of copies per stage is fixed; its product is masked by the consumers.
template <int NT>
__device__ __forceinline__ void dma_copy(uint8_t* la, uint8_t* lb, int h, int kb0, int J0,
                                         const uint16_t* __restrict__ bval, const uint16_t* __restrict__ B,
                                         int64_t ldb, int n_base, int kb_count, int w, int l) {
    using S = DmaShape<NT>;
    const int kb = kb0 + (h >> 1), kh = h & 1;
    const int J = (J0 >= 0 && J0 < kb_count) ? J0 : 0;
    {
        const int p = w * 64 + l;  // chunk position in the A stage
        const int r = p >> 2, c = (p & 3) ^ dma_fa(r);
        const uint16_t* src = bval + (int64_t)kb * (kBs * kBs) + r * kBs + kh * kKh + c * 8;
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(la + w * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < S::kBCopies; ++j) {
        const int q = (j * 4 + w) * 64 + l;  // chunk position in the B stage
        const int k = q / S::kBChunks, c = (q % S::kBChunks) ^ dma_gb(k);
        const uint16_t* src = B + ((int64_t)J * kBs + kh * kKh + k) * ldb + n_base + c * 8;
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(lb + (j * 4 + w) * 1024), 16, 0, 0);
    }
}

template <int NT>
__device__ __forceinline__ void dma_compute(const uint8_t* la, const uint8_t* lb, f32x16 (&acc)[2][DmaShape<NT>::kUC],
                                            bool ok, int w, int l) {
    using S = DmaShape<NT>;
#pragma unroll
    for (int ks = 0; ks < kKh / 16; ++ks) {
        bf16x8 aop[2], bop[S::kUC];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int r = 32 * t + (l & 31), c = 2 * ks + (l >> 5);
            const u32x4 v = *reinterpret_cast<const u32x4*>(la + (r * 4 + (c ^ dma_fa(r))) * 16);
            // a block with an out-of-range column contributes nothing (selected,
            // not branched, so the accumulators stay in place)
            aop[t] = __builtin_bit_cast(bf16x8, ok ? v : u32x4{0u, 0u, 0u, 0u});
        }
#pragma unroll
        for (int u = 0; u < S::kUC; ++u) {
            s16x4 half[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int k = 16 * ks + 8 * (l >> 5) + 4 * i + ((l & 15) >> 2);
                const int n = w * (NT / 4) + 32 * u + 16 * ((l >> 4) & 1) + 4 * (l & 3);
                const uint8_t* p = lb + (k * S::kBChunks + ((n >> 3) ^ dma_gb(k))) * 16 + (n & 7) * 2;
                half[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
            }
            const s16x4 lo = half[0], hi = half[1];
            const short __attribute__((ext_vector_type(8))) both = {lo[0], lo[1], lo[2], lo[3],
                                                                    hi[0], hi[1], hi[2], hi[3]};
            bop[u] = __builtin_bit_cast(bf16x8, both);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int u = 0; u < S::kUC; ++u)
                acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[t], bop[u], acc[t][u], 0, 0, 0);
    }
}

template <int NT>
__global__ __launch_bounds__(2 * kBlock) void bsr_spmm_dma(const int32_t* __restrict__ brow_ptr,
                                                           const int32_t* __restrict__ bcol,
                                                           const uint16_t* __restrict__ bval,
                                                           const uint16_t* __restrict__ B, int64_t ldb, float alpha,
                                                           float beta, float* __restrict__ C, int64_t ldc, int nnzb,
                                                           int kb_count, int mb, int ntiles) {
    static_assert(NT == 256, "tile width (two workgroups of 80 KB LDS per CU)");
    using S = DmaShape<NT>;
    // one array per stage, so that the wait-count logic can tell the copies
    // into one stage from the operand reads of another
    __shared__ __attribute__((aligned(1024))) uint8_t a0[S::kABytes], a1[S::kABytes], a2[S::kABytes], a3[S::kABytes];
    __shared__ __attribute__((aligned(1024))) uint8_t b0[S::kBBytes], b1[S::kBBytes], b2[S::kBBytes], b3[S::kBBytes];

    const int I = blockIdx.x / ntiles, tile = blockIdx.x % ntiles;
    if (I >= mb) return;
    const int n_base = tile * NT;
    // waves 0..3 run the MFMAs, waves 4..7 issue the copies: a copy instruction
    // that waits for the memory pipeline then never holds back an MFMA
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
    const bool producer = wave >= 4;
    const int w = wave & 3;

    f32x16 acc[2][S::kUC];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < S::kUC; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[t][u][r] = 0.0f;

    // out-of-range block pointers are clamped; with no block columns at all B
    // has no rows and nothing is read
    const int kb0 = max(brow_ptr[I], 0);
    const int kb1 = kb_count > 0 ? min(brow_ptr[I + 1], nnzb) : kb0;
    const int T = kb1 > kb0 ? 2 * (kb1 - kb0) : 0;  // stages

    bool ok0 = false, ok1 = false, ok2 = false, ok3 = false;
#define SPX_ISSUE(h, la, lb, okv, J)                                                         \
    {                                                                                         \
        okv = (J) >= 0 && (J) < kb_count;                                                     \
        if (producer) dma_copy<NT>(la, lb, h, kb0, J, bval, B, ldb, n_base, kb_count, w, l);  \
    }
    // column index of the next stage to issue, read one stage ahead of its use
    const int last = kb1 - 1;
    int jn = 0;
    if (T > 0) {
        const int j0 = bcol[kb0];
        jn = bcol[min(kb0 + 1, last)];
        SPX_ISSUE(0, a0, b0, ok0, j0);
        SPX_ISSUE(1, a1, b1, ok1, j0);
        SPX_ISSUE(2, a2, b2, ok2, jn);
    }

    // Stage h: the producers wait until its copies have landed (copies of at
    // most two later stages may still be in flight); barrier; the producers
    // refill the buffer consumed at h - 1 with stage h + 3 while the consumers
    // run the MFMAs of stage h.  The consumers' operand reads of stage h - 1
    // completed before they reached the barrier (the MFMAs consumed them).
#define SPX_STEP(h, la, lb, okv, nla, nlb, nokv)                                   \
    {                                                                               \
        if (producer) {                                                             \
            const int ahead = min(T - 1 - (h), 2);                                  \
            if (ahead == 2)                                                         \
                __builtin_amdgcn_s_waitcnt(vm_wait(2 * S::kPerStage));              \
            else if (ahead == 1)                                                    \
                __builtin_amdgcn_s_waitcnt(vm_wait(S::kPerStage));                  \
            else                                                                    \
                __builtin_amdgcn_s_waitcnt(vm_wait(0));                             \
        }                                                                           \
        asm volatile("s_barrier" ::: "memory");                                     \
        if ((h) + 3 < T) SPX_ISSUE((h) + 3, nla, nlb, nokv, jn);                    \
        jn = bcol[min(kb0 + (((h) + 4) >> 1), last)];                               \
        if (!producer) dma_compute<NT>(la, lb, acc, okv, w, l);                     \
    }
    for (int h = 0; h < T; h += 4) {
        SPX_STEP(h, a0, b0, ok0, a3, b3, ok3);
        if (h + 1 < T) SPX_STEP(h + 1, a1, b1, ok1, a0, b0, ok0);
        if (h + 2 < T) SPX_STEP(h + 2, a2, b2, ok2, a1, b1, ok1);
        if (h + 3 < T) SPX_STEP(h + 3, a3, b3, ok3, a2, b2, ok2);
    }
#undef SPX_STEP
#undef SPX_ISSUE
    if (producer) return;

    // D layout of the 32x32 MFMA: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int u = 0; u < S::kUC; ++u) {
            const int col = n_base + w * (NT / 4) + 32 * u + (l & 31);
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
hipError_t launch_dma(int64_t mb, int64_t kb, int64_t nnzb, const int32_t* brow_ptr, const int32_t* bcol,
                      const uint16_t* bval, int32_t N, const uint16_t* B, int64_t ldb, float alpha, float beta,
                      float* C, int64_t ldc, hipStream_t s) {
    const int ntiles = N / NT;
    hipLaunchKernelGGL(bsr_spmm_dma<NT>, dim3((unsigned)(mb * ntiles)), dim3(2 * kBlock), 0, s, brow_ptr, bcol, bval, B,
                       ldb, alpha, beta, C, ldc, (int)nnzb, (int)kb, (int)mb, ntiles);
    return hipGetLastError();
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

int bsr_spmm_device(int64_t mb, int64_t kb, int32_t bs, int64_t nnzb, const int32_t* brow_ptr, const int32_t* bcol,
                    const uint16_t* bval, int32_t N, const uint16_t* B, int64_t ldb, float alpha, float beta,
                    float* C, int64_t ldc, void* work, size_t work_bytes, hipStream_t s) {
    (void)work;
    (void)work_bytes;
    (void)bs;
    if (mb == 0 || N == 0) return SP_OK;
    hipError_t err;
    if (N % 256 == 0) {
        err = launch_dma<256>(mb, kb, nnzb, brow_ptr, bcol, bval, N, B, ldb, alpha, beta, C, ldc, s);
    } else if (N % 128 == 0) {
        err = launch_pipelined<128>(mb, kb, nnzb, brow_ptr, bcol, bval, N, B, ldb, alpha, beta, C, ldc, s);
    } else {
        hipLaunchKernelGGL(bsr_spmm_n64, dim3((unsigned)mb, (unsigned)((N + 63) / 64)), dim3(kBlock), 0, s, brow_ptr,
                           bcol, bval, B, ldb, alpha, beta, C, ldc, (int)nnzb, (int)kb, (int)N);
        err = hipGetLastError();
    }
    return err == hipSuccess ? SP_OK : SP_ERR_HIP;
}

}  // namespace spx
