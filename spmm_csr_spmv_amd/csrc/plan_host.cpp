// Host side of the plan (declarations and the layout of each structure in
// layout.h): row profile, row bins, SELL-C-sigma order, column-panel and
// x-window streams, phase-swept SpMM copy; and the WCSR task table.  Plain
// C++ without HIP, so that it runs under the host sanitizers; api.cpp and
// wcsr.hip move the arrays to and from the device.
//
// 「通用稀疏矩阵乘法CUDA算子实现」 §4: the profile of the matrix (row lengths with
// their mean, variance and tail, 「CUDA LSMR 专栏（二）」 §5.3) decides which kernel
// serves which rows.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include "layout.h"

namespace spx {
namespace host {

namespace {
constexpr int64_t kI32Max = 2147483647;
}  // namespace

// Nearest-rank q-th percentile of the lengths: the (ceil(q m / 100))-th
// smallest.  hist[l] counts the rows of length l for l < hist.size(); a rank
// beyond the histogram is found by selection on a copy.
int64_t nearest_rank(const std::vector<int32_t>& len, const std::vector<int64_t>& hist, int q) {
    const int64_t m = (int64_t)len.size();
    const int64_t k = (q * m + 99) / 100 - 1;
    int64_t below = 0;
    for (size_t l = 0; l < hist.size(); ++l) {
        below += hist[l];
        if (below > k) return (int64_t)l;
    }
    std::vector<int32_t> c(len);
    std::nth_element(c.begin(), c.begin() + k, c.end());
    return c[(size_t)k];
}

void profile_rows(const std::vector<int32_t>& hptr, HostDir& d) {
    sp_profile& p = d.prof;
    std::memset(&p, 0, sizeof p);
    p.rows = d.rows;
    p.cols = d.cols;
    p.nnz = d.nnz;
    const int64_t m = d.rows;
    if (m == 0) return;
    std::vector<int32_t> len((size_t)m);
    double sum = 0.0;
    int64_t mx = 0, empty = 0;
    for (int64_t i = 0; i < m; ++i) {
        len[(size_t)i] = hptr[(size_t)i + 1] - hptr[(size_t)i];
        sum += len[(size_t)i];
        mx = std::max<int64_t>(mx, len[(size_t)i]);
        empty += len[(size_t)i] == 0;
    }
    const double mean = sum / (double)m;
    double var = 0.0;
    for (int64_t i = 0; i < m; ++i) var += (len[(size_t)i] - mean) * (len[(size_t)i] - mean);
    var /= (double)m;
    p.mean = mean;
    p.var = var;
    p.cv = mean > 0.0 ? std::sqrt(var) / mean : 0.0;
    p.max_len = mx;
    p.empty_rows = empty;
    std::vector<int64_t> hist((size_t)std::min<int64_t>(mx + 1, (int64_t)1 << 20), 0);
    for (const int32_t l : len)
        if ((size_t)l < hist.size()) hist[(size_t)l] += 1;
    p.p95 = nearest_rank(len, hist, 95);
    p.p99 = nearest_rank(len, hist, 99);
}

// Row-to-bin assignment (see the sp_plan_options comment in the public header).
void assign_bins(const std::vector<int32_t>& hptr, const sp_plan_options& o, HostDir& d) {
    std::vector<int4> split, block, wave, group;
    sp_profile& p = d.prof;
    p.group_tasks = p.group_rows = p.group_nnz = 0;
    p.wave_rows = p.wave_nnz = p.block_rows = p.block_nnz = 0;
    p.split_rows = p.split_segments = p.split_nnz = 0;
    d.split_rows.clear();
    d.n_partials = 0;
    int32_t g_r0 = 0, g_rows = 0;
    int64_t g_nnz = 0;
    auto close_group = [&](int32_t next_row) {
        if (g_rows > 0) {
            group.push_back(make_int4(g_r0, g_r0 + g_rows, hptr[(size_t)g_r0], hptr[(size_t)(g_r0 + g_rows)]));
            p.group_tasks += 1;
            p.group_rows += g_rows;
            p.group_nnz += g_nnz;
        }
        g_r0 = next_row;
        g_rows = 0;
        g_nnz = 0;
    };
    for (int32_t r = 0; r < d.rows; ++r) {
        const int32_t b = hptr[(size_t)r], e = hptr[(size_t)r + 1];
        const int32_t l = e - b;
        if (l > o.split_min) {
            close_group(r + 1);
            const int32_t nseg = (int32_t)((l + (int64_t)o.split_seg - 1) / o.split_seg);
            const int32_t id = (int32_t)d.split_rows.size();
            d.split_rows.push_back(make_int4(r, (int32_t)d.n_partials, nseg, 0));
            for (int32_t s = 0; s < nseg; ++s) {
                const int32_t sb = b + s * o.split_seg;
                const int32_t se = std::min<int64_t>(e, (int64_t)sb + o.split_seg);
                split.push_back(make_int4(id, s, sb, se));
            }
            d.n_partials += nseg;
            p.split_rows += 1;
            p.split_segments += nseg;
            p.split_nnz += l;
        } else if (l > o.block_min) {
            close_group(r + 1);
            block.push_back(make_int4(r, b, e, 0));
            p.block_rows += 1;
            p.block_nnz += l;
        } else if (l > o.wave_min) {
            close_group(r + 1);
            wave.push_back(make_int4(r, b, e, 0));
            p.wave_rows += 1;
            p.wave_nnz += l;
        } else {
            if (g_rows > 0 && (g_nnz + l > o.group_nnz || g_rows == spx::kGroupMaxRows)) close_group(r);
            if (g_rows == 0) g_r0 = r;
            g_rows += 1;
            g_nnz += l;
        }
    }
    close_group(d.rows);
    d.tasks.clear();
    d.tasks.reserve(split.size() + block.size() + wave.size() + group.size());
    d.tasks.insert(d.tasks.end(), split.begin(), split.end());
    d.tasks.insert(d.tasks.end(), block.begin(), block.end());
    d.tasks.insert(d.tasks.end(), wave.begin(), wave.end());
    d.tasks.insert(d.tasks.end(), group.begin(), group.end());
    d.n_split = (int32_t)split.size();
    d.n_block = (int32_t)block.size();
    d.n_wave = (int32_t)wave.size();
    d.n_group = (int32_t)group.size();
}

// SELL-C-sigma layout of the group rows (C = 64): windows of sigma rows sorted
// by decreasing length (ties by row index); rows served by another bin keep
// their place in the window order with length -1 (sorted after every group
// row) and contribute no slots.
void build_sell(const std::vector<int32_t>& hptr, const sp_plan_options& o, HostDir& d) {
    const int64_t m = d.rows;
    std::vector<int32_t> len((size_t)m);
    for (int64_t i = 0; i < m; ++i) {
        const int32_t l = hptr[(size_t)i + 1] - hptr[(size_t)i];
        len[(size_t)i] = l <= o.wave_min ? l : -1;
    }
    d.sell_perm.resize((size_t)m);
    for (int64_t i = 0; i < m; ++i) d.sell_perm[(size_t)i] = (int32_t)i;
    // each window of sigma rows sorted on its own (windows in parallel)
    parallel_for((m + o.sell_sigma - 1) / o.sell_sigma, [&](int64_t i) {
        const int64_t w = i * o.sell_sigma, e = std::min<int64_t>(m, w + o.sell_sigma);
        std::stable_sort(d.sell_perm.begin() + w, d.sell_perm.begin() + e,
                         [&](int32_t a, int32_t b) { return len[(size_t)a] > len[(size_t)b]; });
    });
    d.sell_len.resize((size_t)m);
    for (int64_t k = 0; k < m; ++k) d.sell_len[(size_t)k] = len[(size_t)d.sell_perm[(size_t)k]];
    const int64_t slices = (m + 63) / 64;
    d.sell_slice_ptr.assign((size_t)slices + 1, 0);
    int64_t slots = 0;
    for (int64_t s = 0; s < slices; ++s) {
        int32_t width = 0;
        for (int64_t k = s * 64; k < std::min<int64_t>(m, s * 64 + 64); ++k) width = std::max(width, d.sell_len[(size_t)k]);
        d.sell_slice_ptr[(size_t)s] = slots;
        slots += (int64_t)width * 64;
    }
    d.sell_slice_ptr[(size_t)slices] = slots;
    d.sell_slots = slots;
    d.prof.sell_slots = slots;
}

int check_columns(const std::vector<int32_t>& hidx, int64_t cols) {
    const int64_t nnz = (int64_t)hidx.size();
    // blocks small enough that parallel_for spreads them over its threads
    // (it takes at most one thread per 64 blocks)
    constexpr int64_t kBlockEntries = 1 << 14;
    const int64_t blocks = (nnz + kBlockEntries - 1) / kBlockEntries;
    std::vector<char> bad((size_t)blocks, 0);
    parallel_for(blocks, [&](int64_t b) {
        const int64_t e = std::min<int64_t>(nnz, (b + 1) * kBlockEntries);
        for (int64_t q = b * kBlockEntries; q < e; ++q)
            if (hidx[(size_t)q] < 0 || hidx[(size_t)q] >= cols) bad[(size_t)b] = 1;
    });
    for (const char f : bad)
        if (f) return SP_ERR_INDEX;
    return SP_OK;
}

int pstream_bits(int64_t cols, int32_t P) {
    const int64_t w = std::max<int64_t>(32, (cols + P - 1) / P);
    int cb = 0;
    while (((int64_t)1 << cb) < w) ++cb;
    return cb > 22 ? -1 : cb;
}

// Column-panel stream (pstream.hip): panel width W = 2^cb, the smallest power
// of two >= cols / P (at least 32); rows longer than S = min(split_min,
// kPsEntries - 64) are cut out and split into segments of split_seg entries.
// Each panel's rows are packed greedily into chunks of at most kPsEntries
// entries (chunk starts padded to multiples of 4) and at most
// min(kPsMaxRows, 2^(32 - cb)) rows, a long row ending the chunk before it.
// Leaves d.ps_P = 0 (no stream) when the panel width would exceed 2^22
// columns or the stream would not fit int32 positions.
int build_pstream_layout(const std::vector<int32_t>& hptr, const std::vector<int32_t>& hidx, const sp_plan_options& o,
                         int32_t P, HostDir& d) {
    d.ps_P = 0;
    d.ps_chunks.clear();
    d.ps_start.clear();
    d.ps_split_tasks.clear();
    d.ps_split_rows.clear();
    d.ps_skip.clear();
    const int64_t rows = d.rows;
    const int cb = pstream_bits(d.cols, P);
    if (cb < 0) return SP_OK;
    const int64_t rmax = std::min<int64_t>(spx::kPsMaxRows, (int64_t)1 << (32 - cb));
    const int64_t S = std::min<int64_t>(o.split_min, spx::kPsEntries - 64);
    // entries of each stream row in each panel (a stream row has at most S <= 4032 entries)
    std::vector<uint16_t> cnt((size_t)P * (size_t)rows, 0);
    std::vector<char> longrow((size_t)rows, 0);
    int64_t n_partials = 0;
    for (int64_t r = 0; r < rows; ++r) {
        const int32_t b = hptr[(size_t)r], e = hptr[(size_t)r + 1];
        if (e - b > S) {
            longrow[(size_t)r] = 1;
            const int32_t nseg = (int32_t)(((int64_t)(e - b) + o.split_seg - 1) / o.split_seg);
            d.ps_split_rows.push_back(make_int4((int32_t)r, (int32_t)n_partials, nseg, 0));
            for (int32_t k = 0; k < nseg; ++k) {
                const int32_t sb = b + k * o.split_seg;
                const int32_t se = (int32_t)std::min<int64_t>(e, (int64_t)sb + o.split_seg);
                d.ps_split_tasks.push_back(make_int4((int32_t)(n_partials + k), 0, sb, se));
            }
            n_partials += nseg;
            continue;
        }
        for (int32_t k = b; k < e; ++k) {
            const int32_t p = hidx[(size_t)k] >> cb;
            cnt[(size_t)p * (size_t)rows + (size_t)r] += 1;
        }
    }
    d.ps_start.assign((size_t)P * (size_t)rows, 0);
    int64_t pos = 0;
    for (int32_t p = 0; p < P; ++p) {
        d.ps_coff[p] = (int32_t)d.ps_chunks.size();
        int64_t rb = -1, n = 0;
        auto close = [&](int64_t re) {
            if (rb >= 0) {
                d.ps_chunks.push_back(make_int4((int32_t)pos, (int32_t)(pos + n), (int32_t)rb, (int32_t)re));
                pos += (n + 3) & ~(int64_t)3;
            }
            rb = -1;
            n = 0;
        };
        const uint16_t* cp = cnt.data() + (size_t)p * (size_t)rows;
        int32_t* sp = d.ps_start.data() + (size_t)p * (size_t)rows;
        for (int64_t r = 0; r < rows; ++r) {
            if (longrow[(size_t)r]) {
                close(r);
                continue;
            }
            const int64_t c = cp[r];
            if (rb >= 0 && (r - rb + 1 > rmax || ((n + c + 3) & ~(int64_t)3) > spx::kPsEntries)) close(r);
            if (rb < 0) rb = r;
            if (pos + n > kI32Max) return SP_OK;
            sp[r] = (int32_t)(pos + n);
            n += c;
        }
        close(rows);
        if (pos > kI32Max) return SP_OK;
    }
    for (int32_t p = P; p <= spx::kXcds; ++p) d.ps_coff[p] = (int32_t)d.ps_chunks.size();
    d.ps_skip.assign((size_t)((rows + 31) / 32), 0u);
    for (const int4& sr : d.ps_split_rows) d.ps_skip[(size_t)sr.x / 32] |= 1u << (sr.x % 32);
    d.ps_total = pos;
    d.ps_P = P;
    d.ps_cb = cb;
    return SP_OK;
}

// x-window stream (xwin.hip): windows of 2^bits columns; rows cut greedily
// into chunks of at most kXwChunk entries and kXwMaxRows rows, a row longer
// than kXwChunk entries forming segments of its own; the stream holds the
// chunks in order, each chunk's entries window by window (CSR order inside a
// window) with every window's run padded to a multiple of 8 slots; a product
// workgroup takes the runs of one window over at most kXwPieceRuns chunks
// and kXwPiece slots, window w on XCD w mod 8.  Needs the column indices on
// the host (the caller's hidx).  Returns SP_ERR_UNSUPPORTED,
// leaving the stream off, when x needs more than kXwMaxWindows windows,
// positions would not fit int32 or the run table would exceed 2^26 entries.
int build_xwin_layout(const std::vector<int32_t>& hptr, const std::vector<int32_t>& hidx, int32_t bits, HostDir& d) {
    d.xw_bits = 0;
    d.xw_chunks.clear();
    d.xw_chunk_q.clear();
    d.xw_runs.clear();
    d.xw_wm_runs.clear();
    d.xw_wm_tab.clear();
    d.xw_pieces.clear();
    d.xw_prod_ranges.clear();
    d.xw_split_rows.clear();
    d.xw_pos.clear();
    d.xw_total = 0;
    d.xw_n_partials = 0;
    const int64_t rows = d.rows, nnz = d.nnz;
    const int64_t nw = std::max<int64_t>(1, ((int64_t)d.cols + ((int64_t)1 << bits) - 1) >> bits);
    if (nw > spx::kXwMaxWindows) return SP_ERR_UNSUPPORTED;
    // row chunks, in CSR order: {q_begin, q_end, row_begin or long row, row_end or -(partial + 1)}
    std::vector<int4> chunks;
    std::vector<int4> split_rows;
    int64_t n_partials = 0;
    {
        int64_t rb = -1, n = 0;
        auto close = [&](int64_t re) {
            if (rb >= 0)
                chunks.push_back(make_int4(hptr[(size_t)rb], hptr[(size_t)re], (int32_t)rb, (int32_t)re));
            rb = -1;
            n = 0;
        };
        for (int64_t r = 0; r < rows; ++r) {
            const int64_t b = hptr[(size_t)r], e = hptr[(size_t)r + 1], len = e - b;
            if (len > spx::kXwChunk) {
                close(r);
                const int64_t nseg = (len + spx::kXwChunk - 1) / spx::kXwChunk;
                const int32_t j = (int32_t)split_rows.size();
                split_rows.push_back(make_int4((int32_t)r, (int32_t)n_partials, (int32_t)nseg, 0));
                for (int64_t k = 0; k < nseg; ++k) {
                    const int64_t sb = b + k * spx::kXwChunk, se = std::min<int64_t>(e, sb + spx::kXwChunk);
                    chunks.push_back(make_int4((int32_t)sb, (int32_t)se, j, (int32_t)(-(n_partials + k) - 1)));
                }
                n_partials += nseg;
                continue;
            }
            if (rb >= 0 && (n + len > spx::kXwChunk || r - rb + 1 > spx::kXwMaxRows)) close(r);
            if (rb < 0) rb = r;
            n += len;
        }
        close(rows);
    }
    const int64_t n_chunks = (int64_t)chunks.size();
    if (n_chunks * (nw + 1) > ((int64_t)1 << 26)) return SP_ERR_UNSUPPORTED;
    // runs (padded to multiples of 8) and the stream position of every entry;
    // chunks are independent but for where each starts: their padded sizes
    // in parallel, the starts in order, then runs and positions in parallel
    std::vector<int32_t> runs((size_t)(n_chunks * (nw + 1)));
    std::vector<int32_t> pos((size_t)nnz);
    std::vector<int2> chunk_q((size_t)n_chunks);
    std::vector<int64_t> first((size_t)n_chunks + 1);
    parallel_for(n_chunks, [&](int64_t c) {
        const int4 ch = chunks[(size_t)c];
        int32_t cnt[spx::kXwMaxWindows] = {};
        for (int32_t q = ch.x; q < ch.y; ++q) cnt[hidx[(size_t)q] >> bits] += 1;
        int32_t* row = runs.data() + (size_t)(c * (nw + 1));
        int64_t span = 0;
        for (int64_t w = 0; w < nw; ++w) {
            row[w] = (cnt[w] + 7) & ~7;  // padded length for now
            span += row[w];
        }
        first[(size_t)c + 1] = span;
    });
    first[0] = 0;
    for (int64_t c = 0; c < n_chunks; ++c) first[(size_t)c + 1] += first[(size_t)c];
    const int64_t total = first[(size_t)n_chunks];
    if (total > kI32Max) return SP_ERR_UNSUPPORTED;
    parallel_for(n_chunks, [&](int64_t c) {
        const int4 ch = chunks[(size_t)c];
        int32_t* row = runs.data() + (size_t)(c * (nw + 1));
        int32_t cur[spx::kXwMaxWindows];
        int64_t at = first[(size_t)c];
        for (int64_t w = 0; w < nw; ++w) {
            const int32_t len = row[w];
            row[w] = (int32_t)at;
            cur[w] = (int32_t)at;
            at += len;
        }
        row[nw] = (int32_t)at;
        for (int32_t q = ch.x; q < ch.y; ++q) pos[(size_t)q] = cur[hidx[(size_t)q] >> bits]++;
        chunk_q[(size_t)c] = make_int2(ch.x, ch.y - ch.x);
        chunks[(size_t)c].x = (int32_t)first[(size_t)c];
        chunks[(size_t)c].y = (int32_t)at;
    });
    // window-major run starts: window after window, runs in chunk order
    std::vector<int32_t> wm_runs((size_t)(n_chunks * nw));
    {
        int64_t at = 0;
        for (int64_t w = 0; w < nw; ++w)
            for (int64_t c = 0; c < n_chunks; ++c) {
                wm_runs[(size_t)(c * nw + w)] = (int32_t)at;
                at += runs[(size_t)(c * (nw + 1) + w + 1)] - runs[(size_t)(c * (nw + 1) + w)];
            }
    }
    // the same run starts in window-major order, for the product kernel: the
    // runs of a piece are consecutive entries; a last entry closes the stream
    std::vector<int2> wm_tab((size_t)(n_chunks * nw + 1));
    for (int64_t w = 0; w < nw; ++w)
        for (int64_t c = 0; c < n_chunks; ++c)
            wm_tab[(size_t)(w * n_chunks + c)] =
                make_int2(runs[(size_t)(c * (nw + 1) + w)], wm_runs[(size_t)(c * nw + w)]);
    wm_tab[(size_t)(n_chunks * nw)] = make_int2(0, (int32_t)total);
    // pieces: the runs of one window over at most kXwPieceRuns chunks and
    // kXwPiece slots, {window | runs << 8, first chunk, window-major start,
    // groups of 8}; listed XCD by XCD (window w on XCD w mod 8), windows in
    // order.  Each XCD's run sequence is cut into kXwProdGrid / 8 contiguous
    // shares, one per product workgroup (workgroup b on XCD b mod 8), at the
    // run boundaries nearest to equal slot counts, or at a window boundary
    // within 2 % of a share of that (one x window fewer to load); no piece
    // crosses a share boundary
    constexpr int64_t kPerXcd = spx::kXwProdGrid / spx::kXcds;
    std::vector<int4> pieces;
    std::vector<int2> ranges((size_t)spx::kXwProdGrid, make_int2(0, 0));
    auto run_len = [&](int64_t c, int64_t w) {
        return (int64_t)(runs[(size_t)(c * (nw + 1) + w + 1)] - runs[(size_t)(c * (nw + 1) + w)]);
    };
    for (int64_t xcd = 0; xcd < spx::kXcds; ++xcd) {
        int64_t slots = 0;
        for (int64_t w = xcd; w < nw; w += spx::kXcds)
            for (int64_t c = 0; c < n_chunks; ++c) slots += run_len(c, w);
        int64_t share = 0, done = 0;  // current share, slots before the current run
        size_t share_first = pieces.size();
        auto close_share = [&]() {
            ranges[(size_t)(share * spx::kXcds + xcd)] = make_int2((int32_t)share_first, (int32_t)pieces.size());
            share_first = pieces.size();
            share += 1;
        };
        const int64_t snap = slots / kPerXcd / 50;  // a share may end at a window boundary this close to its target
        auto target = [&](int64_t i) { return slots * (i + 1) / kPerXcd; };
        for (int64_t w = xcd; w < nw; w += spx::kXcds) {
            int64_t w_end = done;
            for (int64_t c = 0; c < n_chunks; ++c) w_end += run_len(c, w);
            while (share < kPerXcd - 1 && std::llabs(target(share) - done) <= snap) close_share();
            int64_t ca = 0, acc = 0;
            auto emit = [&](int64_t cb) {
                if (acc > 0)
                    pieces.push_back(make_int4((int32_t)(w | ((cb - ca) << 8)), (int32_t)ca,
                                               wm_runs[(size_t)(ca * nw + w)], (int32_t)(acc / 8)));
                ca = cb;
                acc = 0;
            };
            for (int64_t c = 0; c < n_chunks; ++c) {
                const int64_t len = run_len(c, w);
                // share i ends at the run boundary nearest to (i + 1) / kPerXcd of the XCD's slots
                while (share < kPerXcd - 1 && 2 * done + len > 2 * target(share) && w_end - target(share) > snap) {
                    emit(c);
                    close_share();
                }
                if (c - ca == spx::kXwPieceRuns || (acc > 0 && acc + len > spx::kXwPiece)) emit(c);
                acc += len;
                done += len;
            }
            emit(n_chunks);
        }
        while (share < kPerXcd) close_share();
    }
    d.xw_pieces = std::move(pieces);
    d.xw_prod_ranges = std::move(ranges);
    d.xw_chunks = std::move(chunks);
    d.xw_chunk_q = std::move(chunk_q);
    d.xw_runs = std::move(runs);
    d.xw_wm_runs = std::move(wm_runs);
    d.xw_wm_tab = std::move(wm_tab);
    d.xw_split_rows = std::move(split_rows);
    d.xw_pos = std::move(pos);
    d.xw_total = total;
    d.xw_n_partials = n_partials;
    d.xw_nw = (int32_t)nw;
    d.xw_bits = bits;
    return SP_OK;
}

// Phase-swept SpMM copy (spmm.hip): wave row ranges, the first stream slot of
// every (block, wave, phase) cell and the CSR entry of every slot.
void build_sweep_layout(const std::vector<int32_t>& hptr, const std::vector<int32_t>& hidx, int64_t rows, int32_t pb,
                        int32_t P, int32_t nblk, std::vector<int32_t>& wrow, std::vector<int32_t>& off,
                        std::vector<int32_t>& src) {
    constexpr int W = spx::kSwWaves;
    const size_t ncell = (size_t)nblk * P * W;
    // wave row ranges: each block's rows cut into W contiguous ranges of about
    // equal entry counts (cut k at the first row whose entries before it in
    // the block reach k/W of the block's entries)
    wrow.assign((size_t)nblk * W + 1, 0);
    for (int64_t g = 0; g < nblk; ++g) {
        const int64_t rb = g * spx::kSwRows, re = std::min<int64_t>(rows, rb + spx::kSwRows);
        const int64_t base = hptr[(size_t)rb], tot = (int64_t)hptr[(size_t)re] - base;
        int64_t r = rb;
        for (int w = 0; w < W; ++w) {
            const int64_t goal = base + (tot * w + W - 1) / W;
            while (r < re && hptr[(size_t)r] < goal) ++r;
            wrow[(size_t)g * W + (size_t)w] = (int32_t)r;
        }
    }
    wrow[(size_t)nblk * W] = (int32_t)rows;
    off.assign(ncell + 1, 0);
    // counts of every (block, wave, phase) cell; blocks are independent
    parallel_for(nblk, [&](int64_t g) {
        for (int w = 0; w < W; ++w) {
            const int64_t r0 = wrow[(size_t)g * W + (size_t)w], r1 = wrow[(size_t)g * W + (size_t)w + 1];
            const size_t cell = ((size_t)g * W + (size_t)w) * P;
            for (int64_t r = r0; r < r1; ++r)
                for (int32_t q = hptr[(size_t)r]; q < hptr[(size_t)r + 1]; ++q)
                    ++off[cell + (size_t)(hidx[(size_t)q] >> pb) + 1];
        }
    });
    for (size_t k = 1; k <= ncell; ++k) off[k] += off[k - 1];
    src.assign(hidx.size(), 0);
    parallel_for(nblk, [&](int64_t g) {
        std::vector<int32_t> cur((size_t)P);
        for (int w = 0; w < W; ++w) {
            const size_t cell = ((size_t)g * W + (size_t)w) * P;
            for (size_t k = 0; k < cur.size(); ++k) cur[k] = off[cell + k];
            const int64_t r0 = wrow[(size_t)g * W + (size_t)w], r1 = wrow[(size_t)g * W + (size_t)w + 1];
            for (int64_t r = r0; r < r1; ++r)
                for (int32_t q = hptr[(size_t)r]; q < hptr[(size_t)r + 1]; ++q)
                    src[(size_t)cur[(size_t)(hidx[(size_t)q] >> pb)]++] = q;
        }
    });
}

// The AsyncSparse summary page §4.2: windows whose compressed columns pass a
// threshold are cut into pieces of a fixed width, one workgroup each.
// Workgroups start roughly in index order, so the widest tasks go first and
// the short ones fill in behind them.
int build_wcsr_tasks(const std::vector<int32_t>& wp, int64_t total_cols, int32_t task_cols, std::vector<int4>& tasks,
                     std::vector<int4>& splits, int32_t& slots) {
    const int64_t nw = (int64_t)wp.size() - 1;
    tasks.clear();
    splits.clear();
    slots = 0;
    for (int64_t w = 0; w < nw; ++w)
        if (wp[(size_t)w] < 0 || wp[(size_t)w + 1] < wp[(size_t)w] || wp[(size_t)w + 1] > total_cols)
            return SP_ERR_INDEX;
    tasks.reserve((size_t)(nw + total_cols / task_cols));
    for (int64_t w = 0; w < nw; ++w) {
        const int32_t q0 = wp[(size_t)w], q1 = wp[(size_t)w + 1];
        if (q1 - q0 <= task_cols) {
            tasks.push_back(make_int4((int32_t)w, q0, q1, -1));
            continue;
        }
        const int32_t nt = (int32_t)(((int64_t)q1 - q0 + task_cols - 1) / task_cols);
        splits.push_back(make_int4((int32_t)w, slots, nt, 0));
        for (int32_t t = 0; t < nt; ++t) {
            const int64_t b = q0 + (int64_t)t * task_cols;
            tasks.push_back(make_int4((int32_t)w, (int32_t)b, (int32_t)std::min<int64_t>(b + task_cols, q1), slots + t));
        }
        slots += nt;
    }
    std::stable_sort(tasks.begin(), tasks.end(), [](const int4& a, const int4& b) { return a.z - a.y > b.z - b.y; });
    return SP_OK;
}

}  // namespace host
}  // namespace spx
