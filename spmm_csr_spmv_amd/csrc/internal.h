// Internal declarations shared by the host code (api.cpp) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "spmm_csr_spmv.h"

namespace spx {

constexpr int kBlock = 256;          // threads per workgroup for every kernel
constexpr int kGroupMaxNnz = 4096;   // LDS capacity of a group task (entries)
constexpr int kGroupMaxRows = 1024;  // rows per group task
constexpr int kXcds = 8;             // MI355X: workgroups go round-robin to 8 XCDs

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
    // optional column panels of the group rows (see spmv.hip)
    int32_t npanels;                 // 0 = off
    const int4* ptasks;              // [split | block | wave | panel groups]
    int32_t n_pgroup;
    int32_t panel_width;             // columns per panel
    int32_t* pcol;                   // [nnz] panel-major copy (group ranges only)
    float* pval;                     // [nnz]
    int32_t* pstart;                 // [n_group * (npanels + 1)]
    uint16_t* poff;                  // [npanels * rows] row offset inside its panel block
    float* ypart;                    // [npanels * rows]
    // optional SELL-C-sigma copy of the group rows
    int32_t use_sell;
    int32_t sell_slices;
    const int64_t* sell_slice_ptr;   // [slices + 1]
    const int32_t* sell_perm;        // [rows]  sorted position -> row
    const int32_t* sell_len;         // [rows]  length at sorted position, -1 = row served elsewhere
    const int32_t* sell_col;         // [slots]
    const float* sell_val;           // [slots]
};

// ---- launchers (return hipError_t of the launch) ----
hipError_t launch_spmv(const DirDevice& d, float alpha, const float* x, float beta, float* y,
                       hipStream_t s);
hipError_t launch_spmm(const DirDevice& d, int32_t N, float alpha, const float* B, int64_t ldb,
                       float beta, float* C, int64_t ldc, hipStream_t s);
hipError_t launch_sell_fill(const DirDevice& d, int64_t slots, int32_t* sell_col, float* sell_val,
                            hipStream_t s);
hipError_t launch_panel_build(const DirDevice& d, int32_t* flag, hipStream_t s);

// Conversions: workspace sizes and the two builders (host driver in convert.hip).
size_t coo_build_bytes(int64_t m, int64_t n, int64_t nnz);
size_t csc_build_bytes(int64_t m, int64_t n, int64_t nnz);
int coo_to_csr_device(int64_t m, int64_t n, int64_t nnz, const int32_t* coo_row, const int32_t* coo_col,
                      const float* coo_val, int32_t* row_ptr, int32_t* col_idx, float* val, void* work,
                      size_t work_bytes, hipStream_t s);
int csr_to_csc_device(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                      const float* val, int32_t* col_ptr, int32_t* row_idx, float* cval, void* work,
                      size_t work_bytes, hipStream_t s);

// BSR SpMM (bsr.hip).
size_t bsr_work_bytes(int64_t mb, int64_t kb, int32_t bs, int64_t nnzb, int32_t N);
int bsr_spmm_device(int64_t mb, int64_t kb, int32_t bs, int64_t nnzb, const int32_t* brow_ptr,
                    const int32_t* bcol, const uint16_t* bval, int32_t N, const uint16_t* B, int64_t ldb,
                    float alpha, float beta, float* C, int64_t ldc, void* work, size_t work_bytes,
                    hipStream_t s);

}  // namespace spx
