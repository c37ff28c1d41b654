// Layout constants of the plan's kernels and the host side of a plan
// direction: the row profile, the row bins, the SELL-C-sigma order, the
// column-panel and x-window streams and the phase-swept SpMM copy, computed
// from host copies of the row pointer and column indices.  No HIP here: these
// builders run (and are tested under the host sanitizers) without a GPU;
// api.cpp reads the arrays back from the device and uploads the results.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <thread>
#include <vector>

#include "spmm_csr_spmv.h"

namespace spx {

constexpr int kBlock = 256;          // threads per workgroup for every kernel
constexpr int kGroupMaxNnz = 4096;   // LDS capacity of a group task (entries)
constexpr int kGroupMaxRows = 1024;  // rows per group task
constexpr int kXcds = 8;             // MI355X: workgroups go round-robin to 8 XCDs
constexpr int kPsEntries = 4096;     // column-panel stream: entries per chunk (16 per thread)
constexpr int kPsMaxRows = 2048;     // column-panel stream: rows per chunk (LDS row sums)
constexpr int kXwChunk = 15360;      // x-window stream: entries per row chunk (LDS products)
constexpr int kXwMaxRows = 1536;     // x-window stream: rows per row chunk
constexpr int kXwMaxWindows = 256;   // x-window stream: windows of x
constexpr int kXwMinBits = 5;        // x-window stream: narrowest window, 2^5 columns
constexpr int kXwMaxBits = 15;       // x-window stream: widest window, 2^15 columns = 128 KB of LDS
constexpr int kXwPiece = 32768;      // x-window stream: window entries per product workgroup
constexpr int kXwPieceRuns = 1024;   // x-window stream: chunks per product workgroup
constexpr int kXwProdGrid = 256;     // x-window stream: product workgroups (one per CU, 32 per XCD)
constexpr int kSwWaves = 8;          // phase-swept SpMM: waves per workgroup
constexpr int kSwRows = 2048;        // phase-swept SpMM: rows per workgroup (C rows in LDS)
constexpr int kSwRowBits = 11;       // phase-swept SpMM: row within the workgroup's rows
constexpr int kSwColBits = 21;       // phase-swept SpMM: column bits (at most 2^21 columns)
constexpr int kSwMaxRowLen = 8192;   // phase-swept SpMM: longest row the automatic rule accepts
constexpr int kSwSliceBytes = 512 << 10;  // phase-swept SpMM: B slice of one phase (automatic rule)

namespace host {

// Host stand-ins of the device vector types: same members and layout (16 and
// 8 bytes), so a vector of them is uploaded byte for byte.
struct int4 {
    int32_t x, y, z, w;
};
struct int2 {
    int32_t x, y;
};
static_assert(sizeof(int4) == 16 && sizeof(int2) == 8, "layout of the device vector types");
inline int4 make_int4(int32_t x, int32_t y, int32_t z, int32_t w) { return int4{x, y, z, w}; }
inline int2 make_int2(int32_t x, int32_t y) { return int2{x, y}; }

// Runs f(i) for every i in [0, n) on up to 16 host threads, each taking one
// contiguous block of indices; f must not throw.  Results do not depend on
// the thread count when every f(i) writes only what belongs to i.
template <class F>
void parallel_for(int64_t n, F f) {
    const int64_t hw = (int64_t)std::thread::hardware_concurrency();
    const int64_t T = std::max<int64_t>(1, std::min<int64_t>({hw, (int64_t)16, n / 64}));
    if (T < 2) {
        for (int64_t i = 0; i < n; ++i) f(i);
        return;
    }
    const int64_t per = (n + T - 1) / T;
    std::vector<std::thread> pool;
    pool.reserve((size_t)T);
    for (int64_t t = 0; t < T; ++t)
        pool.emplace_back([&f, t, per, n] {
            for (int64_t i = t * per; i < std::min(n, (t + 1) * per); ++i) f(i);
        });
    for (std::thread& th : pool) th.join();
}

// Host side of one direction (A or A^T) of a plan.
struct HostDir {
    int32_t rows = 0, cols = 0;
    int64_t nnz = 0;
    // task tables, in launch order
    std::vector<int4> tasks;       // split | block | wave | group
    std::vector<int4> split_rows;  // {row, partial_base, nseg, 0}
    int32_t n_split = 0, n_block = 0, n_wave = 0, n_group = 0;
    int64_t n_partials = 0;        // total split segments
    // SELL
    bool use_sell = false;
    std::vector<int64_t> sell_slice_ptr;
    std::vector<int32_t> sell_perm, sell_len;
    int64_t sell_slots = 0;
    // column-panel stream (pstream.hip)
    int32_t ps_P = 0, ps_cb = 0;
    std::vector<int4> ps_chunks;       // panel-major
    int32_t ps_coff[kXcds + 1] = {};
    std::vector<int32_t> ps_start;     // [P][rows] stream position of row r's panel-p entries
    int64_t ps_total = 0;              // stream entries, padding included
    std::vector<int4> ps_split_tasks;  // {partial index, 0, nz_begin, nz_end}
    std::vector<int4> ps_split_rows;   // {row, partial_base, nseg, 0}
    std::vector<uint32_t> ps_skip;     // bit r of word r / 32: row r is a split row
    // x-window stream (xwin.hip)
    int32_t xw_bits = 0, xw_nw = 0;
    std::vector<int4> xw_chunks;       // {stream_begin, stream_end, row_begin, row_end or -(partial + 1)}
    std::vector<int2> xw_chunk_q;      // {first CSR entry, entries}
    std::vector<int32_t> xw_runs;      // [n_chunks][nw + 1] chunk-major run starts
    std::vector<int32_t> xw_wm_runs;   // [n_chunks][nw] window-major run starts
    std::vector<int2> xw_wm_tab;       // [nw][n_chunks] + 1: {chunk-major, window-major start}, window-major order
    std::vector<int4> xw_pieces;       // {window | runs << 8, chunk, start, groups}, by XCD, window order
    std::vector<int2> xw_prod_ranges;  // [kXwProdGrid] pieces of each product workgroup
    std::vector<int4> xw_split_rows;   // {row, partial_base, nseg, 0}
    std::vector<int32_t> xw_pos;       // [nnz] stream position of each CSR entry
    int64_t xw_total = 0, xw_n_partials = 0;
    sp_profile prof{};
};

// hptr: the direction's row pointer (rows + 1 entries); hidx: its column
// indices (nnz), already checked to lie in [0, cols).
void profile_rows(const std::vector<int32_t>& hptr, HostDir& d);
void assign_bins(const std::vector<int32_t>& hptr, const sp_plan_options& o, HostDir& d);
void build_sell(const std::vector<int32_t>& hptr, const sp_plan_options& o, HostDir& d);
// SP_OK when every index lies in [0, cols), else SP_ERR_INDEX.
int check_columns(const std::vector<int32_t>& hidx, int64_t cols);
// Column bits of the panel stream with P panels, or -1 when a panel would be
// wider than 2^22 columns (no stream).
int pstream_bits(int64_t cols, int32_t P);
int build_pstream_layout(const std::vector<int32_t>& hptr, const std::vector<int32_t>& hidx, const sp_plan_options& o,
                         int32_t P, HostDir& d);
int build_xwin_layout(const std::vector<int32_t>& hptr, const std::vector<int32_t>& hidx, int32_t bits, HostDir& d);
// Phase-swept SpMM copy: wrow[g kSwWaves + w] first row of each wave (last =
// rows), off[(g kSwWaves + w) P + p] first stream slot of each cell (last =
// nnz), src[s] the CSR entry of stream slot s.
void build_sweep_layout(const std::vector<int32_t>& hptr, const std::vector<int32_t>& hidx, int64_t rows, int32_t pb,
                        int32_t P, int32_t nblk, std::vector<int32_t>& wrow, std::vector<int32_t>& off,
                        std::vector<int32_t>& src);
// WCSR task split (wcsr.hip), from the window pointer wp (nw + 1 entries): a
// window of at most task_cols compressed columns is one task, a wider one
// ceil(cols / task_cols) tasks of task_cols columns (the last shorter) whose
// partial slots follow each other, the split windows in window order.
// tasks = {window, first column, end column, slot or -1}, widest first (equal
// widths in window, then column order); splits = {window, first slot, tasks,
// 0}.  SP_ERR_INDEX when wp is not nondecreasing inside [0, total_cols].
int build_wcsr_tasks(const std::vector<int32_t>& wp, int64_t total_cols, int32_t task_cols, std::vector<int4>& tasks,
                     std::vector<int4>& splits, int32_t& slots);

}  // namespace host
}  // namespace spx
