// Internal declarations shared by the host code (api.cpp) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "spmm_csr_spmv.h"
#include "layout.h"

namespace spx {

// Task tables of one direction (A or A^T), laid out in device memory as one
// int4 array: [split tasks | block tasks | wave tasks | group tasks].
//   split task  {split_row_id, segment_no, nz_begin, nz_end}
//   block task  {row, nz_begin, nz_end, 0}
//   wave task   {row, nz_begin, nz_end, 0}
//   group task  {row_begin, row_end, nz_begin, nz_end}
//   split row   {row, partial_base, nseg, 0}   (separate array)
struct DirDevice {
    int32_t rows, cols;
    const int32_t* ptr;
    const int32_t* idx;
    const float* val;
    const int4* tasks;      // device
    int32_t n_split, n_block, n_wave, n_group;
    const int4* split_rows; // device
    int32_t n_split_rows;
    float* partials;        // device, partial sums of split segments
    int32_t* counters;      // device, arrival counters (self-resetting)
    int32_t xcd_remap;
    int32_t group_cap;      // LDS entries reserved for a group task
    // optional column-panel stream of all rows up to ps split length (pstream.hip)
    int32_t ps_P;                    // 0 = off; else 1, 2, 4 or 8 panels
    int32_t ps_cb;                   // column bits: panel width 1 << ps_cb
    int32_t ps_coff[kXcds + 1];      // first chunk of each panel
    const int4* ps_chunks;           // {q_begin, q_end, row_begin, row_end}
    uint32_t* ps_pk;                 // (row - row_begin) << cb | column in panel
    float* ps_pv;
    float* ps_ypart;                 // [P][ps_ystride] panel row sums
    int64_t ps_ystride;
    int32_t ps_n_split_tasks;        // long rows, segments over the CSR
    const int4* ps_split_tasks;      // {partial index, 0, nz_begin, nz_end}
    int32_t ps_n_split_rows;
    const int4* ps_split_rows;       // {row, partial_base, nseg, 0}
    float* ps_partials;
    const uint32_t* ps_skip;         // [ceil(rows / 32)] bit r: row r is a long (split) row
    // optional x-window stream (xwin.hip)
    int32_t xw_bits;                 // 0 = off; windows of 1 << xw_bits columns
    int32_t xw_nw;                   // windows
    const int4* xw_pieces;           // {window | chunks << 8, chunk_begin, window-major start, groups of 8}
    const int2* xw_prod_ranges;      // [kXwProdGrid] pieces of each product workgroup (by XCD, window order)
    int32_t xw_n_pieces;
    uint16_t* xw_wcol;               // window-major stream: column within the window (0 in padding)
    float* xw_wval;                  // window-major stream: value (0 in padding)
    uint16_t* xw_off;                // chunk-major stream: LDS byte offset of the entry's slot in its chunk's CSR
                                     // order (4 * position); a padding slot points at one of 64 spare slots past the chunk
    float* xw_prod;                  // chunk-major stream: product (written by every call)
    const int32_t* xw_wm_runs;       // [n_chunks][nw] window-major start of chunk c's run in window w (bind only)
    const int2* xw_wm_tab;           // [nw][n_chunks] + 1 {chunk-major, window-major start} of run (c, w)
    int32_t xw_row_grid;             // workgroups of the row kernel (each takes every grid-th chunk)
    int64_t xw_total;                // stream slots
    int32_t xw_n_chunks;
    const int4* xw_chunks;           // {stream_begin, stream_end, row_begin or long row, row_end or -(partial + 1)}
    const int2* xw_chunk_q;          // {first CSR entry, entries}
    const int32_t* xw_runs;          // [n_chunks][nw + 1] chunk-major start of chunk c's run in window w
    int32_t xw_n_split_rows;
    const int4* xw_split_rows;       // {row, partial_base, nseg, 0}
    float* xw_partials;
    int32_t* xw_counters;            // [n_split_rows] arrival counters (self-resetting)
    // optional phase-swept copy for SpMM with small N (spmm.hip): columns cut
    // into sw_P phases of 2^sw_pb columns; blocks of kSwRows rows, cut into
    // kSwWaves wave ranges of about equal entry counts; per (block, wave,
    // phase) the wave's entries of that phase, rows then columns ascending:
    // word (row - block's first row) << kSwColBits | column, and the value
    int32_t sw_pb;                   // 0 = off
    int32_t sw_P, sw_nblk;
    const int32_t* sw_off;           // [(g kSwWaves + w) P + p] first entry; last = nnz
    const int32_t* sw_wrow;          // [g kSwWaves + w] first row of each wave; last = rows
    uint32_t* sw_pk;
    float* sw_pv;
    // optional SELL-C-sigma copy of the group rows
    int32_t use_sell;
    int32_t sell_slices;
    const int64_t* sell_slice_ptr;   // [slices + 1]
    const int32_t* sell_perm;        // [rows]  sorted position -> row
    const int32_t* sell_len;         // [rows]  length at sorted position, -1 = row served elsewhere
    const int32_t* sell_col;         // [slots] columns, or int16 column - row when sell_narrow
    int32_t sell_narrow;             // 1: every SELL column lies within 32767 of its row
    const float* sell_val;           // [slots]
};

// ---- launchers (return hipError_t of the launch) ----
hipError_t launch_spmv(const DirDevice& d, float alpha, const float* x, float beta, float* y,
                       hipStream_t s);
hipError_t launch_spmm(const DirDevice& d, int32_t N, float alpha, const float* B, int64_t ldb,
                       float beta, float* C, int64_t ldc, hipStream_t s);
hipError_t launch_sell_fill(const DirDevice& d, int64_t slots, int32_t* sell_col, float* sell_val,
                            hipStream_t s);
// Largest |column - row| over the SELL rows, atomically maxed into *out (set to 0 first).
hipError_t launch_sell_offset(const DirDevice& d, int32_t* out, hipStream_t s);
hipError_t launch_spmv_pstream(const DirDevice& d, float alpha, const float* x, float beta, float* y,
                               hipStream_t s);
// Writes the panel stream of d from start[p * rows + r] (position of row r's
// first panel-p entry), which the caller uploaded to device memory.
hipError_t launch_pstream_build(const DirDevice& d, const int32_t* start, hipStream_t s);
hipError_t launch_spmv_xwin(const DirDevice& d, float alpha, const float* x, float beta, float* y, hipStream_t s);
// Writes the stream copies of d from pos[q] (chunk-major stream position of
// CSR entry q), which the caller uploaded.
hipError_t launch_xwin_build(const DirDevice& d, const int32_t* pos, hipStream_t s);

// Phase-swept SpMM (spmm.hip): true when the call can take it (N in {4, 8, 16},
// 16-byte aligned B and C rows); the build writes the stream from src[s] (the
// CSR entry of stream slot s), which the caller uploaded into d.sw_pk.
bool spmm_sweep_ok(const DirDevice& d, int32_t N, const float* B, int64_t ldb, const float* C, int64_t ldc);
hipError_t launch_spmm_sweep(const DirDevice& d, int32_t N, float alpha, const float* B, int64_t ldb, float beta,
                             float* C, int64_t ldc, hipStream_t s);
hipError_t launch_sweep_build(const DirDevice& d, int64_t nnz, hipStream_t s);

// Conversions: workspace sizes and the two builders (host driver in convert.hip).
size_t coo_build_bytes(int64_t m, int64_t n, int64_t nnz);
size_t csc_build_bytes(int64_t m, int64_t n, int64_t nnz);
int coo_to_csr_device(int64_t m, int64_t n, int64_t nnz, const int32_t* coo_row, const int32_t* coo_col,
                      const float* coo_val, int32_t* row_ptr, int32_t* col_idx, float* val, void* work,
                      size_t work_bytes, hipStream_t s);
int csr_to_csc_device(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                      const float* val, int32_t* col_ptr, int32_t* row_idx, float* cval, void* work,
                      size_t work_bytes, hipStream_t s);

// COO -> CSR with the scratch in the library's static per-GPU array
// (convert.hip); SP_ERR_WORKSPACE when coo_build_bytes() exceeds its size.
size_t coo_build_noalloc_limit();
int coo_to_csr_noalloc(int64_t m, int64_t n, int64_t nnz, const int32_t* coo_row, const int32_t* coo_col,
                       const float* coo_val, int32_t* row_ptr, int32_t* col_idx, float* val, hipStream_t s);

// Inclusive prefix sum of a[0..n) in place; sums is scratch of scan_work_bytes(n) (convert.hip).
size_t scan_work_bytes(int64_t n);
int scan_inclusive_i32(int32_t* a, int64_t n, int32_t* sums, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);

// CSR -> BSR and BSR SpMV with fp32 blocks (bsr_convert.hip).
size_t bsr_convert_work_bytes(int64_t m, int32_t bs);
int csr_to_bsr_analyze_device(int64_t m, int64_t n, const int32_t* row_ptr, const int32_t* col_idx, int32_t bs,
                              int32_t* brow_ptr, void* work, hipStream_t s, int32_t* flags_host);
int csr_to_bsr_fill_device(int64_t m, int64_t n, const int32_t* row_ptr, const int32_t* col_idx, const float* val,
                           int32_t bs, const int32_t* brow_ptr, int32_t* bcol, void* bval, int32_t out_bf16,
                           hipStream_t s);
int bsr_spmv_device(int64_t m, int64_t n, int32_t bs, int64_t nnzb, const int32_t* brow_ptr, const int32_t* bcol,
                    const float* bval, float alpha, const float* x, float beta, float* y, hipStream_t s);
int bsr_spmv_rows_device(int64_t m, int64_t n, int32_t bs, int64_t nnzb, const int32_t* brow_ptr, const int32_t* bcol,
                         const float* bval, float alpha, const float* x, float beta, float* y, hipStream_t s);

// CSR -> WCSR and the windowed SpMM (wcsr.hip); windows of 64 rows.
size_t wcsr_convert_work_bytes(int64_t m);
int csr_to_wcsr_analyze_device(int64_t m, int64_t n, const int32_t* row_ptr, const int32_t* col_idx, int32_t pad,
                               int32_t* window_ptr, void* work, hipStream_t s, int32_t* flags_host);
int csr_to_wcsr_fill_device(int64_t m, int64_t n, const int32_t* row_ptr, const int32_t* col_idx, const float* val,
                            const int32_t* window_ptr, int32_t* window_col, float* values, hipStream_t s);
int wcsr_spmm_device(int64_t m, const int32_t* window_ptr, const int32_t* window_col, const float* values,
                     int32_t N, const float* B, int64_t ldb, float alpha, float beta, float* C, int64_t ldc,
                     hipStream_t s);
// Task split of the windowed SpMM: the task table (built on the host once per
// matrix, synchronises) and the product over it; head_host receives {tasks,
// slots, 0, split windows}.
size_t wcsr_task_table_bytes(int64_t m, int64_t total_cols, int32_t task_cols);
int wcsr_tasks_build_device(int64_t m, const int32_t* window_ptr, int64_t total_cols, int32_t task_cols, void* table,
                            hipStream_t s, int32_t* head_host);
size_t wcsr_spmm_tasks_work_bytes(int64_t nslots, int32_t N);
int wcsr_spmm_tasks_device(int64_t m, const void* table, int64_t ntasks, int64_t nslots, const int32_t* window_col,
                           const float* values, int32_t N, const float* B, int64_t ldb, float alpha, float beta,
                           float* C, int64_t ldc, void* work, hipStream_t s);

// Plan option validation (api.cpp); dispatch key and tuning cache (tune.cpp).
int check_plan_options(const sp_plan_options& o);
void make_dispatch_key(const sp_profile& p, int32_t transposed, int32_t N, uint64_t version, sp_dispatch_key* key);
bool tune_cache_find(const sp_dispatch_key& key, sp_plan_options* out);

// BSR SpMM (bsr.hip).
size_t bsr_work_bytes(int64_t mb, int64_t kb, int32_t bs, int64_t nnzb, int32_t N);
int bsr_spmm_device(int64_t mb, int64_t kb, int32_t bs, int64_t nnzb, const int32_t* brow_ptr,
                    const int32_t* bcol, const uint16_t* bval, int32_t N, const uint16_t* B, int64_t ldb,
                    float alpha, float beta, float* C, int64_t ldc, void* work, size_t work_bytes,
                    hipStream_t s);

}  // namespace spx
