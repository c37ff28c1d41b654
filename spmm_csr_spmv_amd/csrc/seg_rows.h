// Row sums of a pass of 4096 consecutive CSR-ordered entries (column-panel
// stream, pstream.hip).
//
// 「通用稀疏矩阵乘法CUDA算子实现」 §2.4: long rows are cut into pieces whose
// partial sums are combined in a fixed order, so the result does not depend
// on scheduling.  Here a pass is held by a 256-thread workgroup as 1024 runs
// of four entries, run v = 256 u + tid (u = 0..3) holding entries 4v..4v+3;
// each entry carries its row (non-decreasing over the pass) and its product.
// The sum of a row is formed by a segmented suffix scan over the runs: inside
// each wave with shuffles, then over the 16 wave blocks; the run that holds a
// row's first entry in the pass writes the row's sum to LDS.  Rows that start
// and end inside one run are written directly.  Every sum is added in an
// order fixed by the entry layout alone, so results are reproducible bit for
// bit.
#pragma once

#include "device_common.h"

namespace spx {

constexpr int kPassRuns = 1024;  // runs of four entries per pass

// LDS scratch of one pass.
struct PassScratch {
    int16_t frs[kPassRuns + 1];  // first row of each run (-1: no entry); [1024] = -1
    int16_t lrs[kPassRuns];      // last row of each run
    float agg_h[16];
    int agg_m[16];
    float cf[17];
};

// One run of four consecutive entries: rows ro[j] are non-decreasing over the
// valid prefix j < nv.
struct Run {
    int fr, lr;     // first and last row offset (-1: no valid entry)
    float hsum;     // sum of the entries of row fr
    float tsum;     // sum of the entries of row lr
};

__device__ __forceinline__ Run make_run(const int (&ro)[4], const float (&pr)[4], int nv) {
    Run r;
    r.fr = nv > 0 ? ro[0] : -1;
    r.lr = nv > 0 ? ro[nv - 1] : -1;
    float h = 0.0f, t = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (j < nv && ro[j] == r.fr) h += pr[j];
        if (j < nv && ro[j] == r.lr) t += pr[j];
    }
    r.hsum = h;
    r.tsum = t;
    return r;
}

// Rows strictly between fr and lr start and end inside the run: write them.
__device__ __forceinline__ void write_middle(const int (&ro)[4], const float (&pr)[4], int nv, const Run& r,
                                             float* ysh) {
    if (nv < 3 || r.fr == r.lr) return;
    // candidates: entries 1 and 2 (entry 0 has row fr, entry nv-1 row lr)
    int cur = -1;
    float s = 0.0f;
#pragma unroll
    for (int j = 1; j < 3; ++j) {
        const bool mid = j < nv - 1 && ro[j] != r.fr && ro[j] != r.lr;
        if (mid) {
            if (ro[j] != cur) {
                if (cur >= 0) ysh[cur] = s;
                cur = ro[j];
                s = 0.0f;
            }
            s += pr[j];
        }
    }
    if (cur >= 0) ysh[cur] = s;
}

// Writes ysh[row] for every row that has an entry in the pass.  The caller
// must have made ysh's previous contents visible (barrier) before the call;
// every thread of the workgroup calls this with its own four runs.  On return
// the writes of the pass are not yet visible to other threads.
__device__ __forceinline__ void pass_row_sums(const int (&ro)[4][4], const float (&pr)[4][4], const int (&nv)[4],
                                              float* ysh, PassScratch& s) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    Run run[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        run[u] = make_run(ro[u], pr[u], nv[u]);
        write_middle(ro[u], pr[u], nv[u], run[u], ysh);
        s.frs[256 * u + tid] = (int16_t)run[u].fr;
        s.lrs[256 * u + tid] = (int16_t)run[u].lr;
    }
    if (tid == 0) s.frs[kPassRuns] = -1;
    __syncthreads();  // run rows published

    // segmented suffix scan: C_v = hsum_v + m_v * C_{v+1}, where
    // m_v = (run v is one row) and (run v+1 starts with that row).
    float H[4];
    int M[4];
    bool link[4], cont[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int v = 256 * u + tid;
        link[u] = run[u].lr >= 0 && s.frs[v + 1] == run[u].lr;
        cont[u] = v > 0 && run[u].fr >= 0 && s.lrs[v - 1] == run[u].fr;
        H[u] = run[u].hsum;
        M[u] = (run[u].fr == run[u].lr && link[u]) ? 1 : 0;
    }
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float h2 = __shfl_down(H[u], k, 64);
            const int m2 = __shfl_down(M[u], k, 64);
            if (lane + k < 64 && M[u]) {
                H[u] += h2;
                M[u] = m2;
            }
        }
    }
    // block B = 4u + w holds runs [64B, 64B + 64); lane 0 has its aggregate
    if (lane == 0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            s.agg_h[4 * u + w] = H[u];
            s.agg_m[4 * u + w] = M[u];
        }
    }
    __syncthreads();
    if (w == 0) {
        // the same suffix scan over the 16 block aggregates, in lanes 0..15
        float h = lane < 16 ? s.agg_h[lane] : 0.0f;
        int m = lane < 16 ? s.agg_m[lane] : 0;
#pragma unroll
        for (int k = 1; k < 16; k <<= 1) {
            const float h2 = __shfl_down(h, k, 64);
            const int m2 = __shfl_down(m, k, 64);
            if (lane + k < 16 && m) {
                h += h2;
                m = m2;
            }
        }
        if (lane < 16) s.cf[lane] = h;
        if (lane == 16) s.cf[16] = 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int B = 4 * u + w;
        const float after = s.cf[B + 1];
        const float C = M[u] ? H[u] + after : H[u];  // C_v
        float Cn = __shfl_down(C, 1, 64);             // C_{v+1}
        if (lane == 63) Cn = after;
        const Run& r = run[u];
        if (r.fr >= 0) {
            if (!cont[u]) ysh[r.fr] = C;                                   // head row starts here
            if (r.lr != r.fr) ysh[r.lr] = link[u] ? r.tsum + Cn : r.tsum;  // tail row starts here
        }
    }
}

}  // namespace spx
