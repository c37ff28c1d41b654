// extern "C" entry points of libspmm_csr_spmv.so and the host side of the plan.
//
// The plan is built once per matrix (「通用稀疏矩阵乘法CUDA算子实现」 §4: a light
// profile taken the first time the matrix is seen and cached with it): row
// lengths l_i = row_ptr[i+1] - row_ptr[i] with their mean, variance and tail
// (「CUDA LSMR 专栏（二）」 §5.3), then the row-to-kernel assignment.  Products
// only read the plan; they never allocate or synchronise.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cmath>
#include <cstring>
#include <new>
#include <vector>

#include "internal.h"
#include "spmm_csr_spmv.h"

namespace spx {
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);
hipError_t launch_check_indices(const int32_t* idx, int64_t nnz, int32_t n, int32_t* flag, hipStream_t s);
}

using spx::DirDevice;

namespace {
int check_options_impl(const sp_plan_options& o);
}

namespace spx {
int check_plan_options(const sp_plan_options& o) { return check_options_impl(o); }
}

namespace {

constexpr int64_t kI32Max = 2147483647;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Dir : spx::host::HostDir {
    bool present = false;
    const int32_t* ptr = nullptr;
    const int32_t* idx = nullptr;
    const float* val = nullptr;
    // phase-swept SpMM copy (see spmm.hip): decided per bind from max_N
    bool col_spread = false;           // sampled rows spread over > 1/4 of the columns
    mutable int32_t sw_pb = 0, sw_P = 0, sw_nblk = 0;
    mutable size_t off_sw_off = 0, off_sw_wrow = 0, off_sw_pk = 0, off_sw_pv = 0;
    DirDevice dev{};
    // workspace offsets (byte offsets into the bound workspace)
    mutable size_t off_tasks = 0, off_split_rows = 0, off_partials = 0, off_counters = 0;
    mutable size_t off_sell_ptr = 0, off_sell_perm = 0, off_sell_len = 0, off_sell_col = 0, off_sell_val = 0;
    mutable size_t off_ps_chunks = 0, off_ps_pk = 0, off_ps_pv = 0, off_ps_ypart = 0, off_ps_split_tasks = 0;
    mutable size_t off_ps_split_rows = 0, off_ps_partials = 0, off_ps_skip = 0;
    mutable size_t off_xw_pieces = 0, off_xw_wcol = 0, off_xw_wval = 0, off_xw_off = 0, off_xw_prod = 0;
    mutable size_t off_xw_chunks = 0, off_xw_chunk_q = 0, off_xw_runs = 0, off_xw_split_rows = 0, off_xw_partials = 0,
                   off_xw_counters = 0;
    mutable size_t off_xw_wm_runs = 0, off_xw_wm_tab = 0, off_xw_prod_ranges = 0;
};

}  // namespace

struct sp_plan {
    int64_t m = 0, n = 0, nnz = 0;
    sp_plan_options opt{};
    Dir fwd, tr;
    bool bound = false;
    int32_t bound_max_N = 0;
    uint64_t bind_gen = 0;              // bumped by every bind of a plan (not of a view)
    mutable std::atomic<int> views{0};  // views created on this plan and not yet destroyed
    // A view (base != nullptr) reads the bound tables of its base plan and owns
    // only the per-call scratch bound to it: its descriptors are the base's
    // with the scratch pointers replaced.
    const sp_plan* base = nullptr;
    uint64_t base_gen = 0;  // the base's bind_gen when the view was bound
    DirDevice vdev[2];
};

namespace {

int64_t ps_ystride(int64_t rows) { return (rows + 63) / 64 * 64; }

// Phase width (bits) of the phase-swept SpMM copy for a bind with max_N, or 0
// for none (the rule is in the public header, sp_plan_options).
int32_t sweep_bits(const Dir& d, const sp_plan_options& o, int32_t max_N) {
    if (!d.present || d.rows == 0 || d.nnz == 0 || o.spmm_phase_bits == 0) return 0;
    if (d.nnz > kI32Max) return 0;
    if (d.cols > (1 << spx::kSwColBits)) return 0;  // columns are stored in kSwColBits bits
    if (o.spmm_phase_bits > 0) return std::min(o.spmm_phase_bits, spx::kSwColBits);
    if (max_N < 4 || max_N > 16) return 0;
    if ((int64_t)d.cols * max_N * 4 <= ((int64_t)8 << 20)) return 0;
    if (d.prof.max_len > spx::kSwMaxRowLen || !d.col_spread) return 0;
    int32_t b = 5;
    while (b < spx::kSwColBits && ((int64_t)1 << (b + 1)) * max_N * 4 <= spx::kSwSliceBytes) ++b;
    return ((int64_t)d.cols + ((int64_t)1 << b) - 1) >> b >= 2 ? b : 0;
}

size_t dir_layout(const Dir& d, const sp_plan_options& o, int32_t max_N, size_t base, bool forward) {
    size_t off = base;
    d.sw_pb = forward ? sweep_bits(d, o, max_N) : 0;  // spmm runs on A only
    if (d.sw_pb > 0) {
        d.sw_P = (int32_t)(((int64_t)d.cols + ((int64_t)1 << d.sw_pb) - 1) >> d.sw_pb);
        d.sw_nblk = (int32_t)(((int64_t)d.rows + spx::kSwRows - 1) / spx::kSwRows);
        d.off_sw_off = off;
        off = align256(off + ((size_t)d.sw_nblk * d.sw_P * spx::kSwWaves + 1) * sizeof(int32_t));
        d.off_sw_wrow = off;
        off = align256(off + ((size_t)d.sw_nblk * spx::kSwWaves + 1) * sizeof(int32_t));
        d.off_sw_pk = off;
        off = align256(off + (size_t)d.nnz * sizeof(uint32_t));
        d.off_sw_pv = off;
        off = align256(off + (size_t)d.nnz * sizeof(float));
    } else {
        d.sw_P = d.sw_nblk = 0;
    }
    d.off_tasks = off;
    off = align256(off + d.tasks.size() * sizeof(int4));
    d.off_split_rows = off;
    off = align256(off + d.split_rows.size() * sizeof(int4));
    d.off_partials = off;
    off = align256(off + (size_t)d.n_partials * (size_t)std::max(1, max_N) * sizeof(float));
    const int64_t max_tiles = std::max<int64_t>(1, (max_N + 63) / 64);
    d.off_counters = off;
    off = align256(off + d.split_rows.size() * (size_t)max_tiles * sizeof(int32_t));
    if (d.ps_P > 0) {
        d.off_ps_chunks = off;
        off = align256(off + d.ps_chunks.size() * sizeof(int4));
        d.off_ps_pk = off;
        off = align256(off + (size_t)d.ps_total * sizeof(uint32_t));
        d.off_ps_pv = off;
        off = align256(off + (size_t)d.ps_total * sizeof(float));
        // panel row sums; at bind it first holds the [P][rows] stream starts
        d.off_ps_ypart = off;
        off = align256(off + (size_t)d.ps_P * (size_t)ps_ystride(d.rows) * sizeof(float));
        d.off_ps_split_tasks = off;
        off = align256(off + d.ps_split_tasks.size() * sizeof(int4));
        d.off_ps_split_rows = off;
        off = align256(off + d.ps_split_rows.size() * sizeof(int4));
        d.off_ps_partials = off;
        off = align256(off + d.ps_split_tasks.size() * sizeof(float));
        d.off_ps_skip = off;
        off = align256(off + d.ps_skip.size() * sizeof(uint32_t));
    }
    if (d.xw_bits > 0) {
        d.off_xw_pieces = off;
        off = align256(off + d.xw_pieces.size() * sizeof(int4));
        d.off_xw_prod_ranges = off;
        off = align256(off + d.xw_prod_ranges.size() * sizeof(int2));
        d.off_xw_wcol = off;
        off = align256(off + (size_t)d.xw_total * sizeof(uint16_t));
        d.off_xw_wval = off;
        off = align256(off + (size_t)d.xw_total * sizeof(float));
        d.off_xw_off = off;
        off = align256(off + (size_t)d.xw_total * sizeof(uint16_t));
        // products; at bind it first holds the stream position of every entry
        d.off_xw_prod = off;
        off = align256(off + (size_t)std::max<int64_t>(d.xw_total, d.nnz) * sizeof(float));
        d.off_xw_chunks = off;
        off = align256(off + d.xw_chunks.size() * sizeof(int4));
        d.off_xw_chunk_q = off;
        off = align256(off + d.xw_chunk_q.size() * sizeof(int2));
        d.off_xw_runs = off;
        off = align256(off + d.xw_runs.size() * sizeof(int32_t));
        d.off_xw_wm_runs = off;
        off = align256(off + d.xw_wm_runs.size() * sizeof(int32_t));
        d.off_xw_wm_tab = off;
        off = align256(off + d.xw_wm_tab.size() * sizeof(int2));
        d.off_xw_split_rows = off;
        off = align256(off + d.xw_split_rows.size() * sizeof(int4));
        d.off_xw_partials = off;
        off = align256(off + (size_t)d.xw_n_partials * sizeof(float));
        d.off_xw_counters = off;
        off = align256(off + d.xw_split_rows.size() * sizeof(int32_t));
    }
    if (d.use_sell) {
        d.off_sell_ptr = off;
        off = align256(off + d.sell_slice_ptr.size() * sizeof(int64_t));
        d.off_sell_perm = off;
        off = align256(off + d.sell_perm.size() * sizeof(int32_t));
        d.off_sell_len = off;
        off = align256(off + d.sell_len.size() * sizeof(int32_t));
        d.off_sell_col = off;
        off = align256(off + (size_t)d.sell_slots * sizeof(int32_t));
        d.off_sell_val = off;
        off = align256(off + (size_t)d.sell_slots * sizeof(float));
    }
    return off;
}

// The first 256 bytes of the workspace hold the index-check flag of bind.
constexpr size_t kMiscBytes = 256;

size_t plan_layout(const sp_plan* p, int32_t max_N) {
    size_t off = kMiscBytes;
    if (p->fwd.present) off = dir_layout(p->fwd, p->opt, max_N, off, true);
    if (p->tr.present) off = dir_layout(p->tr, p->opt, max_N, off, false);
    return off < 256 ? 256 : off;
}

// Per-call scratch of one direction, the part of the workspace every product
// writes: split-row partials and their arrival counters (row bins), the panel
// row sums and long-row partials (column-panel stream), the products and the
// long-row partials and counters (x-window stream).  A view holds its own copy.
struct ScratchOff {
    size_t partials = 0, counters = 0, ps_ypart = 0, ps_partials = 0, xw_prod = 0, xw_partials = 0, xw_counters = 0;
};

size_t view_dir_layout(const Dir& d, int32_t max_N, size_t base, ScratchOff& so) {
    size_t off = base;
    so.partials = off;
    off = align256(off + (size_t)d.n_partials * (size_t)std::max(1, max_N) * sizeof(float));
    const int64_t max_tiles = std::max<int64_t>(1, (max_N + 63) / 64);
    so.counters = off;
    off = align256(off + d.split_rows.size() * (size_t)max_tiles * sizeof(int32_t));
    if (d.ps_P > 0) {
        so.ps_ypart = off;
        off = align256(off + (size_t)d.ps_P * (size_t)ps_ystride(d.rows) * sizeof(float));
        so.ps_partials = off;
        off = align256(off + d.ps_split_tasks.size() * sizeof(float));
    }
    if (d.xw_bits > 0) {
        so.xw_prod = off;
        off = align256(off + (size_t)d.xw_total * sizeof(float));
        so.xw_partials = off;
        off = align256(off + (size_t)d.xw_n_partials * sizeof(float));
        so.xw_counters = off;
        off = align256(off + d.xw_split_rows.size() * sizeof(int32_t));
    }
    return off;
}

size_t view_layout(const sp_plan* base, int32_t max_N, ScratchOff so[2]) {
    size_t off = 0;
    if (base->fwd.present) off = view_dir_layout(base->fwd, max_N, off, so[0]);
    if (base->tr.present) off = view_dir_layout(base->tr, max_N, off, so[1]);
    return off < 256 ? 256 : off;
}

// The descriptors a product launches with: a plan's own, or a view's.
const DirDevice& dir_dev(const sp_plan* p, int transposed) {
    if (p->base) return p->vdev[transposed ? 1 : 0];
    return transposed ? p->tr.dev : p->fwd.dev;
}

// The plan that holds the tables (the base of a view, else the plan itself).
const sp_plan* tables_of(const sp_plan* p) { return p->base ? p->base : p; }

// A view may run only while its base is still bound to the workspace it had
// when the view was bound.
bool usable(const sp_plan* p) {
    if (!p->bound) return false;
    return !p->base || (p->base->bound && p->base->bind_gen == p->base_gen);
}

int check_options_impl(const sp_plan_options& o) {
    if (o.group_nnz < 64 || o.group_nnz > spx::kGroupMaxNnz) return SP_ERR_UNSUPPORTED;
    if (o.wave_min < 0 || o.wave_min > o.group_nnz) return SP_ERR_UNSUPPORTED;
    if (o.block_min < o.wave_min || o.split_min < o.block_min) return SP_ERR_UNSUPPORTED;
    if (o.split_seg < 16) return SP_ERR_UNSUPPORTED;
    if (o.use_sell < -1 || o.use_sell > 1) return SP_ERR_UNSUPPORTED;
    if (o.sell_sigma < 1) return SP_ERR_UNSUPPORTED;
    if (o.col_panels != -1 && o.col_panels != 0 && o.col_panels != 1 && o.col_panels != 2 && o.col_panels != 4 &&
        o.col_panels != 8)
        return SP_ERR_UNSUPPORTED;
    if (o.xcd_remap != 0 && o.xcd_remap != 1) return SP_ERR_UNSUPPORTED;
    if (o.x_window_bits != -1 && o.x_window_bits != 0 &&
        (o.x_window_bits < spx::kXwMinBits || o.x_window_bits > spx::kXwMaxBits))
        return SP_ERR_UNSUPPORTED;
    if (o.spmm_phase_bits != -1 && o.spmm_phase_bits != 0 && (o.spmm_phase_bits < 5 || o.spmm_phase_bits > 24))
        return SP_ERR_UNSUPPORTED;
    return SP_OK;
}

// Auto rule for the column-panel stream (8 panels, one per XCD): x must
// exceed 8 MiB (two L2s' worth), and a sample of up to 64 evenly spaced group
// tasks must show columns spread over more than a quarter of the column range
// (median over the sample of max col - min col).  Reads the sampled column
// ranges back: synchronises.
int column_spread(const Dir& d, hipStream_t s, bool* spread);

int scattered_columns(const Dir& d, hipStream_t s, int32_t* P) {
    *P = 0;
    if ((int64_t)d.cols * 4 <= (int64_t)8 << 20) return SP_OK;
    bool spread = false;
    const int rc = column_spread(d, s, &spread);
    if (rc == SP_OK && spread) *P = 8;
    return rc;
}

// A sample of up to 64 evenly spaced group tasks: is the median over the
// sample of (max col - min col) more than a quarter of the column range?
// Reads the sampled column ranges back: synchronises.
int column_spread(const Dir& d, hipStream_t s, bool* spread) {
    *spread = false;
    const int32_t first = d.n_split + d.n_block + d.n_wave;
    const int32_t nsample = std::min<int32_t>(64, d.n_group);
    std::vector<std::vector<int32_t>> cols((size_t)nsample);
    for (int32_t k = 0; k < nsample; ++k) {
        const auto t = d.tasks[(size_t)first + (size_t)((int64_t)k * d.n_group / nsample)];
        cols[(size_t)k].resize((size_t)(t.w - t.z));
        if (t.w > t.z && hipMemcpyAsync(cols[(size_t)k].data(), d.idx + t.z, (size_t)(t.w - t.z) * sizeof(int32_t),
                                        hipMemcpyDeviceToHost, s) != hipSuccess)
            return SP_ERR_HIP;
    }
    if (hipStreamSynchronize(s) != hipSuccess) return SP_ERR_HIP;
    std::vector<int64_t> spans;
    for (const auto& c : cols) {
        if (c.empty()) continue;
        const auto mm = std::minmax_element(c.begin(), c.end());
        spans.push_back((int64_t)*mm.second - *mm.first);
    }
    if (spans.empty()) return SP_OK;
    std::nth_element(spans.begin(), spans.begin() + spans.size() / 2, spans.end());
    *spread = spans[spans.size() / 2] * 4 > d.cols;
    return SP_OK;
}

// Copies the column indices of d to the host (synchronises) and checks that
// each lies in [0, cols).
int fetch_columns(const Dir& d, hipStream_t s, std::vector<int32_t>& hidx) {
    hidx.resize((size_t)d.nnz);
    if (d.nnz == 0) return SP_OK;
    if (hipMemcpyAsync(hidx.data(), d.idx, (size_t)d.nnz * sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess)
        return SP_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return SP_ERR_HIP;
    return spx::host::check_columns(hidx, d.cols);
}

// Column-panel stream (layout in plan_host.cpp); reads the column indices back.
int build_pstream(const std::vector<int32_t>& hptr, const sp_plan_options& o, int32_t P, Dir& d, hipStream_t s) {
    d.ps_P = 0;
    if (spx::host::pstream_bits(d.cols, P) < 0) return SP_OK;
    std::vector<int32_t> hidx;
    const int rc = fetch_columns(d, s, hidx);
    if (rc != SP_OK) return rc;
    return spx::host::build_pstream_layout(hptr, hidx, o, P, d);
}

// x-window stream (layout in plan_host.cpp); reads the column indices back.
// SP_ERR_UNSUPPORTED (stream off) when x needs more than kXwMaxWindows windows.
int build_xwin(const std::vector<int32_t>& hptr, int32_t bits, Dir& d, hipStream_t s) {
    d.xw_bits = 0;
    const int64_t nw = std::max<int64_t>(1, ((int64_t)d.cols + ((int64_t)1 << bits) - 1) >> bits);
    if (nw > spx::kXwMaxWindows) return SP_ERR_UNSUPPORTED;
    std::vector<int32_t> hidx;
    const int rc = fetch_columns(d, s, hidx);
    if (rc != SP_OK) return rc;
    return spx::host::build_xwin_layout(hptr, hidx, bits, d);
}

int setup_dir(Dir& d, int64_t rows, int64_t cols, int64_t nnz, const int32_t* ptr, const int32_t* idx, const float* val,
              const sp_plan_options& o, hipStream_t s, bool forward) {
    d.present = true;
    d.rows = (int32_t)rows;
    d.cols = (int32_t)cols;
    d.nnz = nnz;
    d.ptr = ptr;
    d.idx = idx;
    d.val = val;
    std::vector<int32_t> hptr((size_t)rows + 1);
    if (hipMemcpyAsync(hptr.data(), ptr, ((size_t)rows + 1) * sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess)
        return SP_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return SP_ERR_HIP;
    if (hptr[0] != 0 || (int64_t)hptr[(size_t)rows] != nnz) return SP_ERR_SIZE;
    for (int64_t i = 0; i < rows; ++i)
        if (hptr[(size_t)i + 1] < hptr[(size_t)i]) return SP_ERR_SIZE;
    spx::host::profile_rows(hptr, d);
    spx::host::assign_bins(hptr, o, d);
    d.use_sell = o.use_sell == 1;
    if (o.use_sell < 0) {
        // SELL-C-sigma pays when rows are short and similar in length
        // (「通用稀疏矩阵乘法CUDA算子实现」 §4 rule table: check the padding first).
        // Rule: no row above 64 entries among the rows it would serve, and the
        // padded slots exceed the real entries by at most 20 %.
        if (d.prof.p99 <= 64 && d.prof.max_len <= o.wave_min && d.prof.mean >= 4.0) {
            spx::host::build_sell(hptr, o, d);
            int64_t sell_nnz = d.prof.group_nnz;
            d.use_sell = d.sell_slots <= sell_nnz + sell_nnz / 5;
        }
    }
    if (d.use_sell) {
        if (d.sell_perm.empty() && d.rows > 0) spx::host::build_sell(hptr, o, d);
    } else {
        d.sell_perm.clear();
        d.sell_len.clear();
        d.sell_slice_ptr.clear();
        d.sell_slots = 0;
        d.prof.sell_slots = 0;
    }
    d.ps_P = 0;
    d.xw_bits = 0;
    if (!d.use_sell && d.rows > 0) {
        // x windows (explicit or auto) take precedence over column panels;
        // explicit panels rule out automatic windows
        int32_t bits = o.x_window_bits, P = o.col_panels;
        if (bits < 0 && P > 0) bits = 0;
        if (bits < 0 || P < 0) {
            int32_t scattered = 0;
            const int rc = scattered_columns(d, s, &scattered);
            if (rc != SP_OK) return rc;
            if (bits < 0) bits = scattered > 0 ? spx::kXwMaxBits : 0;
            if (P < 0) P = scattered;
        }
        if (bits > 0) {
            const int rc = build_xwin(hptr, bits, d, s);
            if (rc == SP_OK) {
                P = 0;
            } else if (!(rc == SP_ERR_UNSUPPORTED && o.x_window_bits < 0)) {
                return rc;  // an explicit request that cannot be met, or a failure
            }
        }
        if (P > 0) {
            const int rc = build_pstream(hptr, o, P, d, s);
            if (rc != SP_OK) return rc;
        }
    }
    d.prof.col_panels = d.ps_P;
    d.prof.x_window_bits = d.xw_bits;
    // column spread for the phase-swept SpMM's automatic rule (B of 8 MiB at
    // N = 16 at the least)
    d.col_spread = false;
    if (forward && o.spmm_phase_bits == -1 && d.rows > 0 && d.n_group > 0 && d.prof.max_len <= spx::kSwMaxRowLen &&
        (int64_t)d.cols * 16 * 4 > ((int64_t)8 << 20)) {
        const int rc = column_spread(d, s, &d.col_spread);
        if (rc != SP_OK) return rc;
    }
    return SP_OK;
}

// Phase-swept SpMM copy (spmm.hip) of d for the bind's layout: the table of
// first entries of every (block, wave, phase) and, in d.sw_pk, the CSR entry
// of every stream slot, which the build kernel turns into the packed words
// and values.  Reads the row pointer and column indices back (synchronises).
int build_sweep(Dir& d, char* ws, hipStream_t s) {
    std::vector<int32_t> hptr((size_t)d.rows + 1), hidx;
    if (hipMemcpyAsync(hptr.data(), d.ptr, hptr.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess)
        return SP_ERR_HIP;
    int rc = fetch_columns(d, s, hidx);  // synchronises
    if (rc != SP_OK) return rc;
    std::vector<int32_t> wrow, off, src;
    spx::host::build_sweep_layout(hptr, hidx, d.rows, d.sw_pb, d.sw_P, d.sw_nblk, wrow, off, src);
    // the uploads must not outlive the host vectors: synchronise after the build
    if (hipMemcpyAsync(ws + d.off_sw_off, off.data(), off.size() * sizeof(int32_t), hipMemcpyHostToDevice, s) !=
            hipSuccess ||
        hipMemcpyAsync(ws + d.off_sw_wrow, wrow.data(), wrow.size() * sizeof(int32_t), hipMemcpyHostToDevice, s) !=
            hipSuccess ||
        hipMemcpyAsync(ws + d.off_sw_pk, src.data(), src.size() * sizeof(int32_t), hipMemcpyHostToDevice, s) !=
            hipSuccess)
        return SP_ERR_HIP;
    if (spx::launch_sweep_build(d.dev, d.nnz, s) != hipSuccess) return SP_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return SP_ERR_HIP;
    return SP_OK;
}

int upload_dir(Dir& d, char* ws, const sp_plan_options& o, hipStream_t s) {
    DirDevice& v = d.dev;
    v = DirDevice{};
    v.rows = d.rows;
    v.cols = d.cols;
    v.ptr = d.ptr;
    v.idx = d.idx;
    v.val = d.val;
    v.tasks = reinterpret_cast<const int4*>(ws + d.off_tasks);
    v.n_split = d.n_split;
    v.n_block = d.n_block;
    v.n_wave = d.n_wave;
    v.n_group = d.n_group;
    v.split_rows = reinterpret_cast<const int4*>(ws + d.off_split_rows);
    v.n_split_rows = (int32_t)d.split_rows.size();
    v.partials = reinterpret_cast<float*>(ws + d.off_partials);
    v.counters = reinterpret_cast<int32_t*>(ws + d.off_counters);
    v.xcd_remap = o.xcd_remap;
    v.group_cap = o.group_nnz;
    if (!d.tasks.empty() &&
        hipMemcpyAsync(ws + d.off_tasks, d.tasks.data(), d.tasks.size() * sizeof(int4), hipMemcpyHostToDevice, s) !=
            hipSuccess)
        return SP_ERR_HIP;
    if (!d.split_rows.empty() &&
        hipMemcpyAsync(ws + d.off_split_rows, d.split_rows.data(), d.split_rows.size() * sizeof(int4),
                       hipMemcpyHostToDevice, s) != hipSuccess)
        return SP_ERR_HIP;
    v.ps_P = d.ps_P;
    if (d.ps_P > 0) {
        v.ps_cb = d.ps_cb;
        for (int k = 0; k <= spx::kXcds; ++k) v.ps_coff[k] = d.ps_coff[k];
        v.ps_chunks = reinterpret_cast<const int4*>(ws + d.off_ps_chunks);
        v.ps_pk = reinterpret_cast<uint32_t*>(ws + d.off_ps_pk);
        v.ps_pv = reinterpret_cast<float*>(ws + d.off_ps_pv);
        v.ps_ypart = reinterpret_cast<float*>(ws + d.off_ps_ypart);
        v.ps_ystride = ps_ystride(d.rows);
        v.ps_n_split_tasks = (int32_t)d.ps_split_tasks.size();
        v.ps_split_tasks = reinterpret_cast<const int4*>(ws + d.off_ps_split_tasks);
        v.ps_n_split_rows = (int32_t)d.ps_split_rows.size();
        v.ps_split_rows = reinterpret_cast<const int4*>(ws + d.off_ps_split_rows);
        v.ps_partials = reinterpret_cast<float*>(ws + d.off_ps_partials);
        v.ps_skip = reinterpret_cast<const uint32_t*>(ws + d.off_ps_skip);
        auto up = [&](size_t off, const void* src, size_t bytes) {
            return bytes == 0 || hipMemcpyAsync(ws + off, src, bytes, hipMemcpyHostToDevice, s) == hipSuccess;
        };
        // the stream starts go to the panel-sum area, which the build kernel reads before any product runs
        if (!up(d.off_ps_chunks, d.ps_chunks.data(), d.ps_chunks.size() * sizeof(int4)) ||
            !up(d.off_ps_split_tasks, d.ps_split_tasks.data(), d.ps_split_tasks.size() * sizeof(int4)) ||
            !up(d.off_ps_split_rows, d.ps_split_rows.data(), d.ps_split_rows.size() * sizeof(int4)) ||
            !up(d.off_ps_skip, d.ps_skip.data(), d.ps_skip.size() * sizeof(uint32_t)) ||
            !up(d.off_ps_ypart, d.ps_start.data(), d.ps_start.size() * sizeof(int32_t)))
            return SP_ERR_HIP;
        if (spx::launch_pstream_build(v, reinterpret_cast<const int32_t*>(ws + d.off_ps_ypart), s) != hipSuccess)
            return SP_ERR_HIP;
    }
    v.xw_bits = d.xw_bits;
    if (d.xw_bits > 0) {
        v.xw_nw = d.xw_nw;
        v.xw_n_pieces = (int32_t)d.xw_pieces.size();
        v.xw_prod_ranges = reinterpret_cast<const int2*>(ws + d.off_xw_prod_ranges);
        v.xw_pieces = reinterpret_cast<const int4*>(ws + d.off_xw_pieces);
        v.xw_wcol = reinterpret_cast<uint16_t*>(ws + d.off_xw_wcol);
        v.xw_wval = reinterpret_cast<float*>(ws + d.off_xw_wval);
        v.xw_off = reinterpret_cast<uint16_t*>(ws + d.off_xw_off);
        v.xw_prod = reinterpret_cast<float*>(ws + d.off_xw_prod);
        v.xw_total = d.xw_total;
        v.xw_n_chunks = (int32_t)d.xw_chunks.size();
        v.xw_chunks = reinterpret_cast<const int4*>(ws + d.off_xw_chunks);
        v.xw_chunk_q = reinterpret_cast<const int2*>(ws + d.off_xw_chunk_q);
        v.xw_runs = reinterpret_cast<const int32_t*>(ws + d.off_xw_runs);
        v.xw_wm_runs = reinterpret_cast<const int32_t*>(ws + d.off_xw_wm_runs);
        v.xw_wm_tab = reinterpret_cast<const int2*>(ws + d.off_xw_wm_tab);
        // the row kernel keeps two workgroups per CU, each taking every grid-th chunk
        v.xw_row_grid = (int32_t)std::min<int64_t>((int64_t)d.xw_chunks.size(), 2 * 256);
        v.xw_n_split_rows = (int32_t)d.xw_split_rows.size();
        v.xw_split_rows = reinterpret_cast<const int4*>(ws + d.off_xw_split_rows);
        v.xw_partials = reinterpret_cast<float*>(ws + d.off_xw_partials);
        v.xw_counters = reinterpret_cast<int32_t*>(ws + d.off_xw_counters);
        auto up = [&](size_t off, const void* src, size_t bytes) {
            return bytes == 0 || hipMemcpyAsync(ws + off, src, bytes, hipMemcpyHostToDevice, s) == hipSuccess;
        };
        // the entry positions go to the product area, which the build kernel reads before any product runs
        if (!up(d.off_xw_pieces, d.xw_pieces.data(), d.xw_pieces.size() * sizeof(int4)) ||
            !up(d.off_xw_prod_ranges, d.xw_prod_ranges.data(), d.xw_prod_ranges.size() * sizeof(int2)) ||
            !up(d.off_xw_chunks, d.xw_chunks.data(), d.xw_chunks.size() * sizeof(int4)) ||
            !up(d.off_xw_chunk_q, d.xw_chunk_q.data(), d.xw_chunk_q.size() * sizeof(int2)) ||
            !up(d.off_xw_runs, d.xw_runs.data(), d.xw_runs.size() * sizeof(int32_t)) ||
            !up(d.off_xw_wm_runs, d.xw_wm_runs.data(), d.xw_wm_runs.size() * sizeof(int32_t)) ||
            !up(d.off_xw_wm_tab, d.xw_wm_tab.data(), d.xw_wm_tab.size() * sizeof(int2)) ||
            !up(d.off_xw_split_rows, d.xw_split_rows.data(), d.xw_split_rows.size() * sizeof(int4)) ||
            !up(d.off_xw_prod, d.xw_pos.data(), d.xw_pos.size() * sizeof(int32_t)))
            return SP_ERR_HIP;
        if (spx::launch_xwin_build(v, reinterpret_cast<const int32_t*>(ws + d.off_xw_prod), s) != hipSuccess)
            return SP_ERR_HIP;
        // the long rows' arrival counters start at zero; the row kernel puts them back to zero
        if (!d.xw_split_rows.empty() &&
            spx::launch_fill_i32(v.xw_counters, (int64_t)d.xw_split_rows.size(), 0, s) != hipSuccess)
            return SP_ERR_HIP;
    }
    v.sw_pb = d.sw_pb;
    if (d.sw_pb > 0) {
        v.sw_P = d.sw_P;
        v.sw_nblk = d.sw_nblk;
        v.sw_off = reinterpret_cast<const int32_t*>(ws + d.off_sw_off);
        v.sw_wrow = reinterpret_cast<const int32_t*>(ws + d.off_sw_wrow);
        v.sw_pk = reinterpret_cast<uint32_t*>(ws + d.off_sw_pk);
        v.sw_pv = reinterpret_cast<float*>(ws + d.off_sw_pv);
    }
    if (d.use_sell) {
        v.use_sell = 1;
        v.sell_slices = (int32_t)(d.sell_slice_ptr.size() - 1);
        v.sell_slice_ptr = reinterpret_cast<const int64_t*>(ws + d.off_sell_ptr);
        v.sell_perm = reinterpret_cast<const int32_t*>(ws + d.off_sell_perm);
        v.sell_len = reinterpret_cast<const int32_t*>(ws + d.off_sell_len);
        v.sell_col = reinterpret_cast<const int32_t*>(ws + d.off_sell_col);
        v.sell_val = reinterpret_cast<const float*>(ws + d.off_sell_val);
        if (hipMemcpyAsync(ws + d.off_sell_ptr, d.sell_slice_ptr.data(), d.sell_slice_ptr.size() * sizeof(int64_t),
                           hipMemcpyHostToDevice, s) != hipSuccess)
            return SP_ERR_HIP;
        if (d.rows > 0 &&
            (hipMemcpyAsync(ws + d.off_sell_perm, d.sell_perm.data(), d.sell_perm.size() * sizeof(int32_t),
                            hipMemcpyHostToDevice, s) != hipSuccess ||
             hipMemcpyAsync(ws + d.off_sell_len, d.sell_len.data(), d.sell_len.size() * sizeof(int32_t),
                            hipMemcpyHostToDevice, s) != hipSuccess))
            return SP_ERR_HIP;
        // int16 column offsets when every SELL column lies within 32767 of its row
        // (the slot area is sized for int32 columns either way)
        int32_t* most = reinterpret_cast<int32_t*>(ws + 64);
        int32_t hmost = 0;
        if (spx::launch_fill_i32(most, 1, 0, s) != hipSuccess || spx::launch_sell_offset(v, most, s) != hipSuccess ||
            hipMemcpyAsync(&hmost, most, sizeof hmost, hipMemcpyDeviceToHost, s) != hipSuccess ||
            hipStreamSynchronize(s) != hipSuccess)
            return SP_ERR_HIP;
        v.sell_narrow = hmost <= 32767 ? 1 : 0;
        if (spx::launch_sell_fill(v, d.sell_slots, reinterpret_cast<int32_t*>(ws + d.off_sell_col),
                                  reinterpret_cast<float*>(ws + d.off_sell_val), s) != hipSuccess)
            return SP_ERR_HIP;
    }
    return SP_OK;
}

}  // namespace

extern "C" {

const char* sp_status_string(int status) {
    switch (status) {
        case SP_OK: return "SP_OK";
        case SP_ERR_NULL: return "SP_ERR_NULL: a required pointer is NULL";
        case SP_ERR_SIZE: return "SP_ERR_SIZE: a size is negative, too large or inconsistent";
        case SP_ERR_INDEX: return "SP_ERR_INDEX: an index is outside its dimension";
        case SP_ERR_WORKSPACE: return "SP_ERR_WORKSPACE: workspace missing or too small";
        case SP_ERR_UNSUPPORTED: return "SP_ERR_UNSUPPORTED: option, shape or layout not supported";
        case SP_ERR_HIP: return "SP_ERR_HIP: a HIP call or kernel launch failed";
        case SP_ERR_STATE: return "SP_ERR_STATE: plan not bound to a workspace";
        case SP_ERR_FILL: return "SP_ERR_FILL: block fill ratio below the requested minimum";
        default: return "unknown status";
    }
}

int sp_version(void) { return 100; }

// ------------------------------------------------------------------ conversions
static int check_dims(int64_t m, int64_t n, int64_t nnz) {
    if (m < 0 || n < 0 || nnz < 0 || m > kI32Max || n > kI32Max || nnz > kI32Max) return SP_ERR_SIZE;
    // row_ptr entries and positions must fit int32 (m + 1 included)
    if (m + 1 > kI32Max || n + 1 > kI32Max) return SP_ERR_SIZE;
    return SP_OK;
}

int csr_build_from_coo_bufsize(int64_t m, int64_t n, int64_t nnz, size_t* bytes) {
    if (!bytes) return SP_ERR_NULL;
    const int rc = check_dims(m, n, nnz);
    if (rc) return rc;
    *bytes = spx::coo_build_bytes(m, n, nnz);
    return SP_OK;
}

int csr_build_from_coo(int64_t m, int64_t n, int64_t nnz, const int32_t* coo_row, const int32_t* coo_col,
                       const float* coo_val, int32_t* row_ptr, int32_t* col_idx, float* val, void* work,
                       size_t work_bytes, void* stream) {
    int rc = check_dims(m, n, nnz);
    if (rc) return rc;
    if (!row_ptr || (nnz > 0 && (!coo_row || !coo_col || !coo_val || !col_idx || !val))) return SP_ERR_NULL;
    if (!work) return SP_ERR_WORKSPACE;
    return spx::coo_to_csr_device(m, n, nnz, coo_row, coo_col, coo_val, row_ptr, col_idx, val, work, work_bytes,
                                  (hipStream_t)stream);
}

int csr_build_from_coo_noalloc(int64_t m, int64_t n, int64_t nnz, const int32_t* coo_row, const int32_t* coo_col,
                               const float* coo_val, int32_t* row_ptr, int32_t* col_idx, float* val, void* stream) {
    int rc = check_dims(m, n, nnz);
    if (rc) return rc;
    if (!row_ptr || (nnz > 0 && (!coo_row || !coo_col || !coo_val || !col_idx || !val))) return SP_ERR_NULL;
    return spx::coo_to_csr_noalloc(m, n, nnz, coo_row, coo_col, coo_val, row_ptr, col_idx, val, (hipStream_t)stream);
}

int csr_to_csc_bufsize(int64_t m, int64_t n, int64_t nnz, size_t* bytes) {
    if (!bytes) return SP_ERR_NULL;
    const int rc = check_dims(m, n, nnz);
    if (rc) return rc;
    *bytes = spx::csc_build_bytes(m, n, nnz);
    return SP_OK;
}

int csr_to_csc(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx, const float* val,
               int32_t* col_ptr, int32_t* row_idx, float* cval, void* work, size_t work_bytes, void* stream) {
    int rc = check_dims(m, n, nnz);
    if (rc) return rc;
    if (!row_ptr || !col_ptr || (nnz > 0 && (!col_idx || !val || !row_idx || !cval))) return SP_ERR_NULL;
    if (!work) return SP_ERR_WORKSPACE;
    return spx::csr_to_csc_device(m, n, nnz, row_ptr, col_idx, val, col_ptr, row_idx, cval, work, work_bytes,
                                  (hipStream_t)stream);
}

// ------------------------------------------------------------------ plan
int sp_plan_options_default(sp_plan_options* o) {
    if (!o) return SP_ERR_NULL;
    o->group_nnz = 2048;
    o->wave_min = 256;
    o->block_min = 4096;
    o->split_min = 32768;
    o->split_seg = 8192;
    o->use_sell = -1;
    o->col_panels = -1;
    o->x_window_bits = -1;
    o->spmm_phase_bits = -1;
    o->sell_sigma = 1024;
    o->xcd_remap = 1;
    return SP_OK;
}

int sp_plan_create(sp_plan** plan, int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                   const float* val, const int32_t* col_ptr, const int32_t* row_idx, const float* cval,
                   const sp_plan_options* opt, void* stream) {
    if (!plan) return SP_ERR_NULL;
    *plan = nullptr;
    int rc = check_dims(m, n, nnz);
    if (rc) return rc;
    if (!row_ptr || (nnz > 0 && (!col_idx || !val))) return SP_ERR_NULL;
    const bool has_t = col_ptr != nullptr;
    if (has_t && nnz > 0 && (!row_idx || !cval)) return SP_ERR_NULL;
    sp_plan_options o;
    if (opt) {
        o = *opt;
    } else {
        sp_plan_options_default(&o);
    }
    rc = check_options_impl(o);
    if (rc) return rc;
    // the kernels stream indices and values with 16-byte loads
    auto misaligned = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) != 0; };
    if (misaligned(col_idx) || misaligned(val) || (has_t && (misaligned(row_idx) || misaligned(cval))))
        return SP_ERR_UNSUPPORTED;
    sp_plan* p = new (std::nothrow) sp_plan;
    if (!p) return SP_ERR_SIZE;
    p->m = m;
    p->n = n;
    p->nnz = nnz;
    p->opt = o;
    hipStream_t s = (hipStream_t)stream;
    rc = setup_dir(p->fwd, m, n, nnz, row_ptr, col_idx, val, o, s, true);
    if (rc == SP_OK && !opt) {
        // no options given: a tuned winner cached for this matrix's dispatch key
        // (SpMV, version 0) replaces the defaults
        sp_dispatch_key key;
        spx::make_dispatch_key(p->fwd.prof, 0, 1, 0, &key);
        sp_plan_options tuned;
        if (spx::tune_cache_find(key, &tuned) && check_options_impl(tuned) == SP_OK &&
            std::memcmp(&tuned, &o, sizeof o) != 0) {
            o = tuned;
            p->opt = o;
            p->fwd = Dir{};
            rc = setup_dir(p->fwd, m, n, nnz, row_ptr, col_idx, val, o, s, true);
        }
    }
    if (rc == SP_OK && has_t) rc = setup_dir(p->tr, n, m, nnz, col_ptr, row_idx, cval, o, s, false);
    if (rc != SP_OK) {
        delete p;
        return rc;
    }
    *plan = p;
    return SP_OK;
}

int sp_plan_workspace_size(const sp_plan* plan, int32_t max_N, size_t* bytes) {
    if (!plan || !bytes) return SP_ERR_NULL;
    if (max_N < 1) return SP_ERR_SIZE;
    if (plan->base) {
        ScratchOff so[2];
        *bytes = view_layout(plan->base, max_N, so);
    } else {
        *bytes = plan_layout(plan, max_N);
    }
    return SP_OK;
}

int sp_plan_view_create(const sp_plan* base, sp_plan** view) {
    if (!base || !view) return SP_ERR_NULL;
    *view = nullptr;
    if (base->base) base = base->base;  // a view of a view reads the same tables
    sp_plan* v = new (std::nothrow) sp_plan;
    if (!v) return SP_ERR_SIZE;
    v->m = base->m;
    v->n = base->n;
    v->nnz = base->nnz;
    v->opt = base->opt;
    v->base = base;
    base->views.fetch_add(1);
    *view = v;
    return SP_OK;
}

// Binds a view: its descriptors are the base's current ones with the scratch
// pointers moved into `work`; the arrival counters there are set to zero.
static int bind_view(sp_plan* view, void* work, size_t work_bytes, int32_t max_N, hipStream_t s) {
    const sp_plan* base = view->base;
    if (!base->bound) return SP_ERR_STATE;
    ScratchOff so[2];
    const size_t need = view_layout(base, max_N, so);
    if (!work || work_bytes < need) return SP_ERR_WORKSPACE;
    char* ws = static_cast<char*>(work);
    view->bound = false;
    const Dir* dirs[2] = {&base->fwd, &base->tr};
    for (int t = 0; t < 2; ++t) {
        const Dir& d = *dirs[t];
        DirDevice& v = view->vdev[t];
        v = d.dev;
        if (!d.present) continue;
        v.partials = reinterpret_cast<float*>(ws + so[t].partials);
        v.counters = reinterpret_cast<int32_t*>(ws + so[t].counters);
        if (d.ps_P > 0) {
            v.ps_ypart = reinterpret_cast<float*>(ws + so[t].ps_ypart);
            v.ps_partials = reinterpret_cast<float*>(ws + so[t].ps_partials);
        }
        if (d.xw_bits > 0) {
            v.xw_prod = reinterpret_cast<float*>(ws + so[t].xw_prod);
            v.xw_partials = reinterpret_cast<float*>(ws + so[t].xw_partials);
            v.xw_counters = reinterpret_cast<int32_t*>(ws + so[t].xw_counters);
            if (!d.xw_split_rows.empty() &&
                spx::launch_fill_i32(v.xw_counters, (int64_t)d.xw_split_rows.size(), 0, s) != hipSuccess)
                return SP_ERR_HIP;
        }
        const int64_t max_tiles = std::max<int64_t>(1, (max_N + 63) / 64);
        if (!d.split_rows.empty() &&
            spx::launch_fill_i32(v.counters, (int64_t)d.split_rows.size() * max_tiles, 0, s) != hipSuccess)
            return SP_ERR_HIP;
    }
    view->base_gen = base->bind_gen;
    view->bound = true;
    view->bound_max_N = max_N;
    return SP_OK;
}

int sp_plan_bind(sp_plan* plan, void* work, size_t work_bytes, int32_t max_N, void* stream) {
    if (!plan) return SP_ERR_NULL;
    if (max_N < 1) return SP_ERR_SIZE;
    if (plan->base) return bind_view(plan, work, work_bytes, max_N, (hipStream_t)stream);
    const size_t need = plan_layout(plan, max_N);
    if (!work || work_bytes < need) return SP_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    char* ws = static_cast<char*>(work);
    plan->bound = false;
    ++plan->bind_gen;  // views bound to the previous tables stop working
    // every stored index must lie inside its dimension before any product runs
    int32_t* flag = reinterpret_cast<int32_t*>(ws);
    if (spx::launch_fill_i32(flag, 4, 0, s) != hipSuccess) return SP_ERR_HIP;
    for (const Dir* d : {&plan->fwd, &plan->tr}) {
        if (d->present && spx::launch_check_indices(d->idx, d->nnz, d->cols, flag, s) != hipSuccess)
            return SP_ERR_HIP;
    }
    int32_t bad = 0;
    if (hipMemcpyAsync(&bad, flag, sizeof bad, hipMemcpyDeviceToHost, s) != hipSuccess) return SP_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return SP_ERR_HIP;
    if (bad) return SP_ERR_INDEX;
    int rc = SP_OK;
    if (plan->fwd.present) rc = upload_dir(plan->fwd, ws, plan->opt, s);
    if (rc == SP_OK && plan->tr.present) rc = upload_dir(plan->tr, ws, plan->opt, s);
    if (rc == SP_OK && plan->fwd.present && plan->fwd.sw_pb > 0) rc = build_sweep(plan->fwd, ws, s);
    if (rc != SP_OK) return rc;
    plan->fwd.prof.spmm_phase_bits = plan->fwd.sw_pb;
    // arrival counters start at zero; the kernels put them back to zero
    for (Dir* d : {&plan->fwd, &plan->tr}) {
        if (!d->present || d->split_rows.empty()) continue;
        const int64_t max_tiles = std::max<int64_t>(1, (max_N + 63) / 64);
        if (spx::launch_fill_i32(d->dev.counters, (int64_t)d->split_rows.size() * max_tiles, 0, s) != hipSuccess)
            return SP_ERR_HIP;
    }
    plan->bound = true;
    plan->bound_max_N = max_N;
    return SP_OK;
}

int sp_plan_profile(const sp_plan* plan, int32_t transposed, sp_profile* out) {
    if (!plan || !out) return SP_ERR_NULL;
    plan = tables_of(plan);
    const Dir& d = transposed ? plan->tr : plan->fwd;
    if (!d.present) return SP_ERR_UNSUPPORTED;
    *out = d.prof;
    return SP_OK;
}

int sp_plan_destroy(sp_plan* plan) {
    if (!plan) return SP_OK;
    if (plan->views.load() != 0) return SP_ERR_STATE;  // its views still read its tables
    if (plan->base) plan->base->views.fetch_sub(1);
    delete plan;
    return SP_OK;
}

// ------------------------------------------------------------------ products
int spmv(const sp_plan* plan, float alpha, const float* x, float beta, float* y, void* stream) {
    if (!plan) return SP_ERR_NULL;
    if (!usable(plan)) return SP_ERR_STATE;
    if ((plan->n > 0 && !x) || (plan->m > 0 && !y)) return SP_ERR_NULL;
    if (plan->m == 0) return SP_OK;
    return spx::launch_spmv(dir_dev(plan, 0), alpha, x, beta, y, (hipStream_t)stream) == hipSuccess ? SP_OK
                                                                                                    : SP_ERR_HIP;
}

int spmv_t(const sp_plan* plan, float alpha, const float* u, float beta, float* z, void* stream) {
    if (!plan) return SP_ERR_NULL;
    if (!tables_of(plan)->tr.present) return SP_ERR_UNSUPPORTED;
    if (!usable(plan)) return SP_ERR_STATE;
    if ((plan->m > 0 && !u) || (plan->n > 0 && !z)) return SP_ERR_NULL;
    if (plan->n == 0) return SP_OK;
    return spx::launch_spmv(dir_dev(plan, 1), alpha, u, beta, z, (hipStream_t)stream) == hipSuccess ? SP_OK
                                                                                                    : SP_ERR_HIP;
}

int spmm(const sp_plan* plan, int32_t N, float alpha, const float* B, int64_t ldb, float beta, float* C, int64_t ldc,
         void* stream) {
    if (!plan) return SP_ERR_NULL;
    if (!usable(plan)) return SP_ERR_STATE;
    if (N < 1 || ldb < N || ldc < N) return SP_ERR_SIZE;
    if (!tables_of(plan)->fwd.split_rows.empty() && N > plan->bound_max_N) return SP_ERR_SIZE;
    if ((plan->n > 0 && !B) || (plan->m > 0 && !C)) return SP_ERR_NULL;
    if (plan->m == 0) return SP_OK;
    const DirDevice& d = dir_dev(plan, 0);
    hipError_t e = spx::spmm_sweep_ok(d, N, B, ldb, C, ldc)
                       ? spx::launch_spmm_sweep(d, N, alpha, B, ldb, beta, C, ldc, (hipStream_t)stream)
                       : spx::launch_spmm(d, N, alpha, B, ldb, beta, C, ldc, (hipStream_t)stream);
    return e == hipSuccess ? SP_OK : SP_ERR_HIP;
}

// ------------------------------------------------------------------ CSR -> BSR, BSR SpMV
static bool bsr_block_ok(int32_t bs) { return bs == 1 || bs == 2 || bs == 4 || bs == 8 || bs == 16 || bs == 32 || bs == 64; }

int csr_to_bsr_bufsize(int64_t m, int64_t n, int64_t nnz, int32_t bs, size_t* bytes) {
    if (!bytes) return SP_ERR_NULL;
    const int rc = check_dims(m, n, nnz);
    if (rc) return rc;
    if (!bsr_block_ok(bs)) return SP_ERR_UNSUPPORTED;
    *bytes = spx::bsr_convert_work_bytes(m, bs);
    return SP_OK;
}

int csr_to_bsr_analyze(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx, int32_t bs,
                       double min_fill, int32_t* brow_ptr, int64_t* nnzb, double* fill, void* work, size_t work_bytes,
                       void* stream) {
    int rc = check_dims(m, n, nnz);
    if (rc) return rc;
    if (!bsr_block_ok(bs)) return SP_ERR_UNSUPPORTED;
    if (!row_ptr || !brow_ptr || !nnzb || !fill || (nnz > 0 && !col_idx)) return SP_ERR_NULL;
    if (!work || work_bytes < spx::bsr_convert_work_bytes(m, bs)) return SP_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    int32_t flags = 0;
    rc = spx::csr_to_bsr_analyze_device(m, n, row_ptr, col_idx, bs, brow_ptr, work, s, &flags);
    if (rc != SP_OK) return rc;
    const int64_t mb = (m + bs - 1) / bs;
    int32_t tail[2] = {0, 0};
    if (hipMemcpyAsync(&tail[0], brow_ptr + mb, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipMemcpyAsync(&tail[1], row_ptr + m, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess)
        return SP_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return SP_ERR_HIP;
    if (flags & 1) return SP_ERR_INDEX;
    if (flags & 2) return SP_ERR_UNSUPPORTED;
    if ((int64_t)tail[1] != nnz) return SP_ERR_SIZE;
    *nnzb = tail[0];
    *fill = tail[0] > 0 ? (double)nnz / ((double)tail[0] * bs * bs) : 1.0;
    if (*fill < min_fill) return SP_ERR_FILL;
    return SP_OK;
}

int csr_to_bsr_fill(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx, const float* val,
                    int32_t bs, const int32_t* brow_ptr, int64_t nnzb, int32_t* bcol, void* bval, int32_t out_bf16,
                    void* stream) {
    int rc = check_dims(m, n, nnz);
    if (rc) return rc;
    if (!bsr_block_ok(bs) || (out_bf16 != 0 && out_bf16 != 1)) return SP_ERR_UNSUPPORTED;
    if (nnzb < 0 || nnzb > kI32Max || nnzb * bs * bs > ((int64_t)1 << 40)) return SP_ERR_SIZE;
    if (!row_ptr || !brow_ptr || (nnz > 0 && (!col_idx || !val)) || (nnzb > 0 && (!bcol || !bval))) return SP_ERR_NULL;
    if (!out_bf16 && bs % 4 == 0 && (reinterpret_cast<uintptr_t>(bval) & 15)) return SP_ERR_UNSUPPORTED;
    return spx::csr_to_bsr_fill_device(m, n, row_ptr, col_idx, val, bs, brow_ptr, bcol, bval, out_bf16,
                                       (hipStream_t)stream);
}

int bsr_spmv(int64_t m, int64_t n, int32_t bs, int64_t nnzb, const int32_t* brow_ptr, const int32_t* bcol,
             const float* bval, float alpha, const float* x, float beta, float* y, void* stream) {
    int rc = check_dims(m, n, 0);
    if (rc) return rc;
    if (!bsr_block_ok(bs)) return SP_ERR_UNSUPPORTED;
    if (nnzb < 0 || nnzb > kI32Max) return SP_ERR_SIZE;
    if (m == 0) return SP_OK;
    if (!brow_ptr || !y || (nnzb > 0 && (!bcol || !bval || (n > 0 && !x)))) return SP_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(bval) & 15) return SP_ERR_UNSUPPORTED;
    if (bs >= 4 && (reinterpret_cast<uintptr_t>(x) & 15)) return SP_ERR_UNSUPPORTED;
    return spx::bsr_spmv_device(m, n, bs, nnzb, brow_ptr, bcol, bval, alpha, x, beta, y, (hipStream_t)stream);
}

int bsr_spmv_rowwise(int64_t m, int64_t n, int32_t bs, int64_t nnzb, const int32_t* brow_ptr, const int32_t* bcol,
                     const float* bval, float alpha, const float* x, float beta, float* y, void* stream) {
    int rc = check_dims(m, n, 0);
    if (rc) return rc;
    if (!bsr_block_ok(bs)) return SP_ERR_UNSUPPORTED;
    if (nnzb < 0 || nnzb > kI32Max) return SP_ERR_SIZE;
    if (m == 0) return SP_OK;
    if (!brow_ptr || !y || (nnzb > 0 && (!bcol || !bval || (n > 0 && !x)))) return SP_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(bval) & 15) return SP_ERR_UNSUPPORTED;
    if (bs >= 4 && (reinterpret_cast<uintptr_t>(x) & 15)) return SP_ERR_UNSUPPORTED;
    return spx::bsr_spmv_rows_device(m, n, bs, nnzb, brow_ptr, bcol, bval, alpha, x, beta, y, (hipStream_t)stream);
}

// ------------------------------------------------------------------ CSR -> WCSR, windowed SpMM
static bool wcsr_pad_ok(int32_t pad) { return pad == 1 || pad == 2 || pad == 4 || pad == 8 || pad == 16 || pad == 32; }

int csr_to_wcsr_bufsize(int64_t m, int64_t n, int64_t nnz, size_t* bytes) {
    if (!bytes) return SP_ERR_NULL;
    const int rc = check_dims(m, n, nnz);
    if (rc) return rc;
    *bytes = spx::wcsr_convert_work_bytes(m);
    return SP_OK;
}

int csr_to_wcsr_analyze(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx, int32_t pad,
                        int32_t* window_ptr, int64_t* total_cols, double* fill, void* work, size_t work_bytes,
                        void* stream) {
    int rc = check_dims(m, n, nnz);
    if (rc) return rc;
    if (!wcsr_pad_ok(pad)) return SP_ERR_UNSUPPORTED;
    if (!row_ptr || !window_ptr || !total_cols || !fill || (nnz > 0 && !col_idx)) return SP_ERR_NULL;
    if (!work || work_bytes < spx::wcsr_convert_work_bytes(m)) return SP_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    int32_t flags = 0;
    rc = spx::csr_to_wcsr_analyze_device(m, n, row_ptr, col_idx, pad, window_ptr, work, s, &flags);
    if (rc != SP_OK) return rc;
    const int64_t nw = (m + 63) / 64;
    int32_t tail[2] = {0, 0};
    if (hipMemcpyAsync(&tail[0], window_ptr + nw, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipMemcpyAsync(&tail[1], row_ptr + m, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess)
        return SP_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return SP_ERR_HIP;
    if (flags & 1) return SP_ERR_INDEX;
    if (flags & 2) return SP_ERR_UNSUPPORTED;
    if ((int64_t)tail[1] != nnz) return SP_ERR_SIZE;
    *total_cols = tail[0];
    *fill = tail[0] > 0 ? (double)nnz / ((double)tail[0] * 64.0) : 1.0;
    return SP_OK;
}

int csr_to_wcsr_fill(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                     const float* val, const int32_t* window_ptr, int64_t total_cols, int32_t* window_col,
                     float* values, void* stream) {
    int rc = check_dims(m, n, nnz);
    if (rc) return rc;
    if (total_cols < 0 || total_cols > kI32Max) return SP_ERR_SIZE;
    if (!row_ptr || !window_ptr || (nnz > 0 && (!col_idx || !val)) || (total_cols > 0 && (!window_col || !values)))
        return SP_ERR_NULL;
    return spx::csr_to_wcsr_fill_device(m, n, row_ptr, col_idx, val, window_ptr, window_col, values,
                                        (hipStream_t)stream);
}

int wcsr_spmm(int64_t m, int64_t n, const int32_t* window_ptr, const int32_t* window_col, const float* values,
              int32_t N, float alpha, const float* B, int64_t ldb, float beta, float* C, int64_t ldc, void* stream) {
    int rc = check_dims(m, n, 0);
    if (rc) return rc;
    if (N < 0 || ldb < N || ldc < N) return SP_ERR_SIZE;
    if (m == 0 || N == 0) return SP_OK;
    // window_col / values may be NULL when every window is empty (they are then never read)
    if (!window_ptr || !C || (n > 0 && !B)) return SP_ERR_NULL;
    if (N % 4 != 0 || ldb % 4 != 0) return SP_ERR_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(B) & 15) || (reinterpret_cast<uintptr_t>(values) & 15)) return SP_ERR_UNSUPPORTED;
    return spx::wcsr_spmm_device(m, window_ptr, window_col, values, N, B, ldb, alpha, beta, C, ldc,
                                 (hipStream_t)stream);
}

static int wcsr_task_args(int64_t m, int64_t total_cols, int32_t task_cols) {
    if (m < 0 || m > kI32Max || total_cols < 0 || total_cols > kI32Max) return SP_ERR_SIZE;
    if (task_cols < 32 || task_cols % 32 != 0) return SP_ERR_UNSUPPORTED;
    return SP_OK;
}

int wcsr_tasks_bufsize(int64_t m, int64_t total_cols, int32_t task_cols, size_t* bytes) {
    if (!bytes) return SP_ERR_NULL;
    const int rc = wcsr_task_args(m, total_cols, task_cols);
    if (rc) return rc;
    *bytes = spx::wcsr_task_table_bytes(m, total_cols, task_cols);
    return SP_OK;
}

int wcsr_tasks_build(int64_t m, const int32_t* window_ptr, int64_t total_cols, int32_t task_cols, void* table,
                     size_t table_bytes, int64_t* ntasks, int64_t* nslots, void* stream) {
    const int rc = wcsr_task_args(m, total_cols, task_cols);
    if (rc) return rc;
    if (!ntasks || !nslots) return SP_ERR_NULL;
    *ntasks = *nslots = 0;
    if (m == 0) return SP_OK;
    if (!window_ptr || !table) return SP_ERR_NULL;
    if (table_bytes < spx::wcsr_task_table_bytes(m, total_cols, task_cols)) return SP_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(table) & 15) return SP_ERR_UNSUPPORTED;
    int32_t head[4] = {0, 0, 0, 0};
    const int r = spx::wcsr_tasks_build_device(m, window_ptr, total_cols, task_cols, table, (hipStream_t)stream, head);
    if (r != SP_OK) return r;
    *ntasks = head[0];
    *nslots = head[1];
    return SP_OK;
}

// nslots partial tiles of 64 x N floats must be addressable in size_t
static bool wcsr_slots_fit(int64_t nslots, int32_t N) {
    return nslots == 0 || N == 0 || (uint64_t)N <= (uint64_t)SIZE_MAX / (256u * (uint64_t)nslots);
}

int wcsr_spmm_tasks_bufsize(int64_t nslots, int32_t N, size_t* bytes) {
    if (!bytes) return SP_ERR_NULL;
    if (nslots < 0 || nslots > kI32Max || N < 0 || !wcsr_slots_fit(nslots, N)) return SP_ERR_SIZE;
    *bytes = spx::wcsr_spmm_tasks_work_bytes(nslots, N);
    return SP_OK;
}

int wcsr_spmm_tasks(int64_t m, int64_t n, const void* table, int64_t ntasks, int64_t nslots,
                    const int32_t* window_col, const float* values, int32_t N, float alpha, const float* B,
                    int64_t ldb, float beta, float* C, int64_t ldc, void* work, size_t work_bytes, void* stream) {
    int rc = check_dims(m, n, 0);
    if (rc) return rc;
    if (N < 0 || ldb < N || ldc < N) return SP_ERR_SIZE;
    if (m == 0 || N == 0) return SP_OK;
    // every window is at least one task
    if (ntasks < (m + 63) / 64 || ntasks > kI32Max || nslots < 0 || nslots > kI32Max || !wcsr_slots_fit(nslots, N))
        return SP_ERR_SIZE;
    if (!table || !C || (n > 0 && !B) || (nslots > 0 && !work)) return SP_ERR_NULL;
    if (work_bytes < spx::wcsr_spmm_tasks_work_bytes(nslots, N)) return SP_ERR_WORKSPACE;
    if (N % 4 != 0 || ldb % 4 != 0) return SP_ERR_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(B) & 15) || (reinterpret_cast<uintptr_t>(values) & 15) ||
        (reinterpret_cast<uintptr_t>(table) & 15) || (reinterpret_cast<uintptr_t>(work) & 15))
        return SP_ERR_UNSUPPORTED;
    return spx::wcsr_spmm_tasks_device(m, table, ntasks, nslots, window_col, values, N, B, ldb, alpha, beta, C, ldc,
                                       work, (hipStream_t)stream);
}

// ------------------------------------------------------------------ BSR
int bsr_spmm_bufsize(int64_t mb, int64_t kb, int32_t bs, int64_t nnzb, int32_t N, size_t* bytes) {
    if (!bytes) return SP_ERR_NULL;
    if (mb < 0 || kb < 0 || nnzb < 0 || N < 0 || mb > kI32Max || kb > kI32Max || nnzb > kI32Max) return SP_ERR_SIZE;
    if (bs != 64) return SP_ERR_UNSUPPORTED;
    *bytes = spx::bsr_work_bytes(mb, kb, bs, nnzb, N);
    return SP_OK;
}

int bsr_spmm(int64_t mb, int64_t kb, int32_t bs, int64_t nnzb, const int32_t* brow_ptr, const int32_t* bcol,
             const uint16_t* bval, int32_t N, const uint16_t* B, int64_t ldb, float alpha, float beta, float* C,
             int64_t ldc, void* work, size_t work_bytes, void* stream) {
    if (mb < 0 || kb < 0 || nnzb < 0 || N < 0 || mb > kI32Max || kb > kI32Max || nnzb > kI32Max) return SP_ERR_SIZE;
    if (bs != 64) return SP_ERR_UNSUPPORTED;
    if (mb * 64 > kI32Max || kb * 64 > kI32Max) return SP_ERR_SIZE;
    if (ldb < N || ldc < N) return SP_ERR_SIZE;
    if (N % 8 != 0 || ldb % 8 != 0 || ldc % 4 != 0) return SP_ERR_UNSUPPORTED;
    if (mb > 0 && N > 0 && (!brow_ptr || !C)) return SP_ERR_NULL;
    if (nnzb > 0 && N > 0 && (!bcol || !bval || !B)) return SP_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(B) & 15) || (reinterpret_cast<uintptr_t>(C) & 15) ||
        (reinterpret_cast<uintptr_t>(bval) & 15))
        return SP_ERR_UNSUPPORTED;
    const size_t need = spx::bsr_work_bytes(mb, kb, bs, nnzb, N);
    if (need > 0 && (!work || work_bytes < need)) return SP_ERR_WORKSPACE;
    return spx::bsr_spmm_device(mb, kb, bs, nnzb, brow_ptr, bcol, bval, N, B, ldb, alpha, beta, C, ldc, work,
                                work_bytes, (hipStream_t)stream);
}

}  // extern "C"
