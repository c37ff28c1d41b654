// Driver for the sanitizer run of the plan's host-side layout builders (test
// infrastructure; built by tests/test_plan_host_sanitize.py with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer, together with
// spmm_csr_spmv_amd/csrc/plan_host.cpp).
//
// On seeded random CSR matrices (empty rows, rows longer than a chunk, m != n)
// it runs the row profile, the row bins under several option sets, the
// SELL-C-sigma order, the column-panel stream (1, 2, 4, 8 panels), the x-window
// stream (several window widths), the phase-swept SpMM copy and the WCSR
// task table, and checks their structural invariants with plain loops
// written here: every row served once, every entry placed once inside its
// chunk, window run or cell, every window column in one task, tables
// monotone, sizes consistent.  A sanitizer report or a failed check ends the
// run with a non-zero status.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "layout.h"

using spx::host::HostDir;

static int g_fail = 0;
#define CHECK(c)                                                                  \
    do {                                                                          \
        if (!(c)) {                                                               \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++g_fail;                                                             \
            return;                                                               \
        }                                                                         \
    } while (0)

struct Csr {
    int32_t m = 0, n = 0;
    std::vector<int32_t> ptr, col;
};

static Csr random_csr(std::mt19937_64& rng, int32_t m, int32_t n, int32_t max_len, int nlong, int32_t long_len) {
    Csr a;
    a.m = m;
    a.n = n;
    a.ptr.assign((size_t)m + 1, 0);
    std::uniform_int_distribution<int32_t> len_d(0, max_len), col_d(0, n - 1), row_d(0, m - 1), coin(0, 4);
    std::vector<int32_t> len((size_t)m);
    for (int32_t i = 0; i < m; ++i) len[(size_t)i] = coin(rng) == 0 ? 0 : len_d(rng);
    for (int k = 0; k < nlong && m > 0; ++k) len[(size_t)row_d(rng)] = long_len;
    for (int32_t i = 0; i < m; ++i) a.ptr[(size_t)i + 1] = a.ptr[(size_t)i] + len[(size_t)i];
    a.col.resize((size_t)a.ptr[(size_t)m]);
    for (int32_t i = 0; i < m; ++i) {
        auto b = a.col.begin() + a.ptr[(size_t)i], e = a.col.begin() + a.ptr[(size_t)i + 1];
        for (auto it = b; it != e; ++it) *it = col_d(rng);
        std::sort(b, e);
    }
    return a;
}

static HostDir fresh(const Csr& a) {
    HostDir d;
    d.rows = a.m;
    d.cols = a.n;
    d.nnz = (int64_t)a.col.size();
    return d;
}

static sp_plan_options opts(int32_t group_nnz, int32_t wave_min, int32_t block_min, int32_t split_min,
                            int32_t split_seg, int32_t sigma) {
    sp_plan_options o{};
    o.group_nnz = group_nnz;
    o.wave_min = wave_min;
    o.block_min = block_min;
    o.split_min = split_min;
    o.split_seg = split_seg;
    o.use_sell = -1;
    o.sell_sigma = sigma;
    o.xcd_remap = 1;
    o.col_panels = -1;
    o.x_window_bits = -1;
    o.spmm_phase_bits = -1;
    return o;
}

static void check_profile(const Csr& a) {
    HostDir d = fresh(a);
    spx::host::profile_rows(a.ptr, d);
    if (a.m == 0) return;
    std::vector<int32_t> len((size_t)a.m);
    for (int32_t i = 0; i < a.m; ++i) len[(size_t)i] = a.ptr[(size_t)i + 1] - a.ptr[(size_t)i];
    std::vector<int32_t> s = len;
    std::sort(s.begin(), s.end());
    auto rank = [&](int q) { return (int64_t)s[(size_t)((q * (int64_t)a.m + 99) / 100 - 1)]; };
    CHECK(d.prof.p95 == rank(95) && d.prof.p99 == rank(99) && d.prof.max_len == s.back());
    CHECK(d.prof.empty_rows == (int64_t)std::count(len.begin(), len.end(), 0));
}

static void check_bins(const Csr& a, const sp_plan_options& o) {
    HostDir d = fresh(a);
    spx::host::profile_rows(a.ptr, d);
    spx::host::assign_bins(a.ptr, o, d);
    CHECK((int64_t)d.tasks.size() == (int64_t)d.n_split + d.n_block + d.n_wave + d.n_group);
    std::vector<int> served((size_t)a.m, 0);
    std::vector<int64_t> split_cov(d.split_rows.size(), 0);
    for (int32_t k = 0; k < d.n_split; ++k) {
        const auto t = d.tasks[(size_t)k];
        CHECK(t.x >= 0 && (size_t)t.x < d.split_rows.size());
        const auto sr = d.split_rows[(size_t)t.x];
        CHECK(t.z >= a.ptr[(size_t)sr.x] && t.w <= a.ptr[(size_t)sr.x + 1] && t.z < t.w);
        CHECK(t.y >= 0 && t.y < sr.z);
        split_cov[(size_t)t.x] += t.w - t.z;
    }
    for (size_t j = 0; j < d.split_rows.size(); ++j) {
        const auto sr = d.split_rows[j];
        CHECK(split_cov[j] == a.ptr[(size_t)sr.x + 1] - a.ptr[(size_t)sr.x]);
        CHECK(a.ptr[(size_t)sr.x + 1] - a.ptr[(size_t)sr.x] > o.split_min);
        served[(size_t)sr.x] += 1;
    }
    for (int32_t k = d.n_split; k < d.n_split + d.n_block + d.n_wave; ++k) {
        const auto t = d.tasks[(size_t)k];
        CHECK(t.x >= 0 && t.x < a.m && t.y == a.ptr[(size_t)t.x] && t.z == a.ptr[(size_t)t.x + 1]);
        served[(size_t)t.x] += 1;
    }
    for (int32_t k = d.n_split + d.n_block + d.n_wave; k < (int32_t)d.tasks.size(); ++k) {
        const auto t = d.tasks[(size_t)k];
        CHECK(t.x >= 0 && t.x < t.y && t.y <= a.m && t.z == a.ptr[(size_t)t.x] && t.w == a.ptr[(size_t)t.y]);
        CHECK(t.y - t.x <= spx::kGroupMaxRows);
        CHECK(t.w - t.z <= std::max(o.group_nnz, o.wave_min));
        for (int32_t r = t.x; r < t.y; ++r) served[(size_t)r] += 1;
    }
    for (int32_t r = 0; r < a.m; ++r) CHECK(served[(size_t)r] == 1);
}

static void check_sell(const Csr& a, const sp_plan_options& o) {
    HostDir d = fresh(a);
    spx::host::profile_rows(a.ptr, d);
    spx::host::assign_bins(a.ptr, o, d);
    spx::host::build_sell(a.ptr, o, d);
    std::vector<int> seen((size_t)a.m, 0);
    for (int32_t k = 0; k < a.m; ++k) {
        const int32_t r = d.sell_perm[(size_t)k];
        CHECK(r >= 0 && r < a.m);
        seen[(size_t)r] += 1;
        const int32_t l = a.ptr[(size_t)r + 1] - a.ptr[(size_t)r];
        CHECK(d.sell_len[(size_t)k] == (l <= o.wave_min ? l : -1));
        // windows of sigma rows, decreasing length inside a window
        if (k % o.sell_sigma != 0) CHECK(d.sell_len[(size_t)k - 1] >= d.sell_len[(size_t)k]);
    }
    for (int32_t r = 0; r < a.m; ++r) CHECK(seen[(size_t)r] == 1);
    const int64_t slices = (a.m + 63) / 64;
    CHECK((int64_t)d.sell_slice_ptr.size() == slices + 1 && d.sell_slice_ptr[(size_t)slices] == d.sell_slots);
    for (int64_t s = 0; s < slices; ++s) {
        const int64_t width = (d.sell_slice_ptr[(size_t)s + 1] - d.sell_slice_ptr[(size_t)s]) / 64;
        CHECK((d.sell_slice_ptr[(size_t)s + 1] - d.sell_slice_ptr[(size_t)s]) % 64 == 0);
        for (int64_t k = s * 64; k < std::min<int64_t>(a.m, s * 64 + 64); ++k) CHECK(d.sell_len[(size_t)k] <= width);
    }
}

static void check_pstream(const Csr& a, const sp_plan_options& o, int32_t P) {
    HostDir d = fresh(a);
    spx::host::profile_rows(a.ptr, d);
    CHECK(spx::host::build_pstream_layout(a.ptr, a.col, o, P, d) == SP_OK);
    if (d.ps_P == 0) return;
    const int cb = d.ps_cb;
    const int64_t S = std::min<int64_t>(o.split_min, spx::kPsEntries - 64);
    // long rows: split tasks cover their entries
    std::vector<char> longrow((size_t)a.m, 0);
    for (const auto& sr : d.ps_split_rows) {
        CHECK(sr.x >= 0 && sr.x < a.m && a.ptr[(size_t)sr.x + 1] - a.ptr[(size_t)sr.x] > S);
        longrow[(size_t)sr.x] = 1;
        CHECK((d.ps_skip[(size_t)sr.x / 32] >> (sr.x % 32)) & 1u);
    }
    int64_t covered = 0;
    for (const auto& t : d.ps_split_tasks) covered += t.w - t.z;
    int64_t long_nnz = 0, short_nnz = 0;
    for (int32_t r = 0; r < a.m; ++r) {
        const int64_t l = a.ptr[(size_t)r + 1] - a.ptr[(size_t)r];
        CHECK(longrow[(size_t)r] == (l > S ? 1 : 0));
        (l > S ? long_nnz : short_nnz) += l;
    }
    CHECK(covered == long_nnz);
    // panel p's chunks cover every short row's panel-p entries: the row's start
    // lies in its chunk and the next row (or the chunk end) closes it
    int64_t stream = 0;
    for (int32_t p = 0; p < P; ++p) {
        CHECK(d.ps_coff[p] <= d.ps_coff[p + 1]);
        for (int32_t c = d.ps_coff[p]; c < d.ps_coff[p + 1]; ++c) {
            const auto ch = d.ps_chunks[(size_t)c];
            CHECK(ch.x % 4 == 0 && ch.x <= ch.y && ch.y - ch.x <= spx::kPsEntries && ch.z < ch.w && ch.w <= a.m);
            stream += ch.y - ch.x;
            int64_t q = ch.x;
            for (int32_t r = ch.z; r < ch.w; ++r) {
                CHECK(!longrow[(size_t)r]);
                CHECK(d.ps_start[(size_t)p * a.m + r] == q);
                for (int32_t k = a.ptr[(size_t)r]; k < a.ptr[(size_t)r + 1]; ++k) q += (a.col[(size_t)k] >> cb) == p;
            }
            CHECK(q == ch.y);
        }
    }
    CHECK(stream == short_nnz);
    CHECK(d.ps_total >= stream);
}

static void check_xwin(const Csr& a, int32_t bits) {
    HostDir d = fresh(a);
    spx::host::profile_rows(a.ptr, d);
    const int rc = spx::host::build_xwin_layout(a.ptr, a.col, bits, d);
    CHECK(rc == SP_OK || rc == SP_ERR_UNSUPPORTED);
    if (rc != SP_OK) return;
    const int64_t nw = d.xw_nw, nc = (int64_t)d.xw_chunks.size();
    CHECK((int64_t)d.xw_runs.size() == nc * (nw + 1) && (int64_t)d.xw_pos.size() == d.nnz);
    std::vector<char> used((size_t)d.xw_total, 0);
    int64_t entries = 0;
    for (int64_t c = 0; c < nc; ++c) {
        const auto ch = d.xw_chunks[(size_t)c];
        const auto q = d.xw_chunk_q[(size_t)c];
        const int32_t* run = d.xw_runs.data() + c * (nw + 1);
        CHECK(run[0] == ch.x && run[nw] == ch.y);
        CHECK(q.y <= spx::kXwChunk);
        for (int64_t w = 0; w < nw; ++w) CHECK(run[w] <= run[w + 1] && (run[w + 1] - run[w]) % 8 == 0);
        for (int32_t k = q.x; k < q.x + q.y; ++k) {
            const int32_t w = a.col[(size_t)k] >> bits, p = d.xw_pos[(size_t)k];
            CHECK(p >= run[w] && p < run[w + 1]);
            CHECK(!used[(size_t)p]);
            used[(size_t)p] = 1;
        }
        entries += q.y;
        if (ch.w >= 0) {  // a chunk of whole rows
            CHECK(ch.z < ch.w && ch.w - ch.z <= spx::kXwMaxRows && q.x == a.ptr[(size_t)ch.z] &&
                  q.x + q.y == a.ptr[(size_t)ch.w]);
        } else {  // a segment of a long row
            CHECK(ch.z >= 0 && (size_t)ch.z < d.xw_split_rows.size());
        }
    }
    CHECK(entries == d.nnz);
    // product workgroups: their piece ranges tile the piece list, and the
    // pieces cover every slot once
    CHECK((int64_t)d.xw_prod_ranges.size() == spx::kXwProdGrid);
    int64_t slots = 0;
    std::vector<int> piece_seen(d.xw_pieces.size(), 0);
    for (const auto& r : d.xw_prod_ranges) {
        CHECK(r.x <= r.y && r.y <= (int32_t)d.xw_pieces.size());
        for (int32_t k = r.x; k < r.y; ++k) piece_seen[(size_t)k] += 1;
    }
    for (size_t k = 0; k < d.xw_pieces.size(); ++k) {
        CHECK(piece_seen[k] == 1);
        const auto pc = d.xw_pieces[k];
        const int32_t w = pc.x & 255, nr = pc.x >> 8;
        CHECK(w < nw && nr >= 1 && nr <= spx::kXwPieceRuns && pc.y >= 0 && pc.y + nr <= nc);
        slots += (int64_t)pc.w * 8;
    }
    CHECK(slots == d.xw_total);
}

static void check_sweep(const Csr& a, int32_t pb) {
    const int32_t P = (int32_t)(((int64_t)a.n + ((int64_t)1 << pb) - 1) >> pb);
    const int32_t nblk = (a.m + spx::kSwRows - 1) / spx::kSwRows;
    std::vector<int32_t> wrow, off, src;
    spx::host::build_sweep_layout(a.ptr, a.col, a.m, pb, P, nblk, wrow, off, src);
    const int W = spx::kSwWaves;
    CHECK((int64_t)wrow.size() == (int64_t)nblk * W + 1 && wrow.back() == a.m);
    CHECK((int64_t)off.size() == (int64_t)nblk * W * P + 1 && off.back() == (int32_t)a.col.size());
    std::vector<int32_t> rows_of(a.col.size());
    for (int32_t r = 0; r < a.m; ++r)
        for (int32_t k = a.ptr[(size_t)r]; k < a.ptr[(size_t)r + 1]; ++k) rows_of[(size_t)k] = r;
    std::vector<char> seen(a.col.size(), 0);
    for (int32_t g = 0; g < nblk; ++g)
        for (int w = 0; w < W; ++w) {
            const int32_t r0 = wrow[(size_t)g * W + w], r1 = wrow[(size_t)g * W + w + 1];
            CHECK(r0 <= r1 && r0 >= g * spx::kSwRows && r1 <= std::min(a.m, (g + 1) * spx::kSwRows));
            for (int32_t p = 0; p < P; ++p) {
                const size_t cell = ((size_t)g * W + w) * P + p;
                CHECK(off[cell] <= off[cell + 1]);
                int32_t prev_row = -1;
                for (int32_t s = off[cell]; s < off[cell + 1]; ++s) {
                    const int32_t q = src[(size_t)s], r = rows_of[(size_t)q];
                    CHECK(q >= 0 && (size_t)q < a.col.size() && !seen[(size_t)q]);
                    seen[(size_t)q] = 1;
                    CHECK(r >= r0 && r < r1 && (a.col[(size_t)q] >> pb) == p && r >= prev_row);
                    prev_row = r;
                }
            }
        }
    for (char f : seen) CHECK(f == 1);
}

// WCSR task table: every window's range tiled once by its tasks in column
// order, each split window's tasks task_cols wide but the last, slots
// consecutive in window order, tasks sorted widest first with ties in
// (window, column) order; bad window pointers refused.
static void check_wcsr_tasks(std::mt19937_64& rng, int32_t task_cols) {
    std::uniform_int_distribution<int32_t> nwd(0, 300), wd(0, 3 * task_cols), big(0, 9);
    const int32_t nw = nwd(rng);
    std::vector<int32_t> wp(1, 0);
    for (int32_t w = 0; w < nw; ++w) wp.push_back(wp.back() + (big(rng) == 0 ? 10 * wd(rng) : wd(rng) / 4));
    std::vector<spx::host::int4> tasks, splits;
    int32_t slots = -1;
    CHECK(spx::host::build_wcsr_tasks(wp, wp.back(), task_cols, tasks, splits, slots) == SP_OK);
    for (size_t k = 1; k < tasks.size(); ++k) {
        const int32_t wa = tasks[k - 1].z - tasks[k - 1].y, wb = tasks[k].z - tasks[k].y;
        CHECK(wa > wb || (wa == wb && (tasks[k - 1].x < tasks[k].x ||
                                       (tasks[k - 1].x == tasks[k].x && tasks[k - 1].y < tasks[k].y))));
    }
    std::vector<std::vector<spx::host::int4>> by_window((size_t)nw);
    for (const auto& t : tasks) {
        CHECK(t.x >= 0 && t.x < nw);
        by_window[(size_t)t.x].push_back(t);
    }
    int32_t next_slot = 0;
    size_t si = 0;
    for (int32_t w = 0; w < nw; ++w) {
        auto& v = by_window[(size_t)w];
        std::sort(v.begin(), v.end(), [](const spx::host::int4& a, const spx::host::int4& b) { return a.y < b.y; });
        const int32_t c = wp[(size_t)w + 1] - wp[(size_t)w];
        CHECK(!v.empty() && v.front().y == wp[(size_t)w] && v.back().z == wp[(size_t)w + 1]);
        for (size_t k = 1; k < v.size(); ++k) CHECK(v[k].y == v[k - 1].z);
        if (c <= task_cols) {
            CHECK(v.size() == 1 && v[0].w == -1);
            continue;
        }
        CHECK((int64_t)v.size() == ((int64_t)c + task_cols - 1) / task_cols);
        for (size_t k = 0; k < v.size(); ++k) {
            CHECK(v[k].w == next_slot + (int32_t)k);
            CHECK(k + 1 == v.size() ? v[k].z - v[k].y >= 1 : v[k].z - v[k].y == task_cols);
        }
        CHECK(si < splits.size() && splits[si].x == w && splits[si].y == next_slot &&
              splits[si].z == (int32_t)v.size() && splits[si].w == 0);
        ++si;
        next_slot += (int32_t)v.size();
    }
    CHECK(si == splits.size() && slots == next_slot);
    CHECK((int64_t)tasks.size() <= (int64_t)nw + wp.back() / task_cols);
    if (nw >= 2) {
        std::vector<int32_t> bad(wp);
        std::swap(bad[1], bad[2]);
        if (bad[1] > bad[2]) CHECK(spx::host::build_wcsr_tasks(bad, wp.back(), task_cols, tasks, splits, slots) ==
                                   SP_ERR_INDEX);
        CHECK(spx::host::build_wcsr_tasks(wp, (int64_t)wp.back() - 1, task_cols, tasks, splits, slots) ==
              SP_ERR_INDEX);
    }
}

int main(int argc, char** argv) {
    const int cases = argc > 1 ? std::atoi(argv[1]) : 40;
    std::mt19937_64 rng(12345);
    for (int c = 0; c < cases; ++c) {
        std::uniform_int_distribution<int32_t> md(0, 6000), nd(1, 70000), ld(1, 120);
        const int32_t m = md(rng), n = nd(rng);
        const Csr a = random_csr(rng, m, n, ld(rng), c % 3, c % 2 ? 20000 : 600);
        check_profile(a);
        const sp_plan_options o1 = opts(2048, 256, 4096, 32768, 8192, 1024);
        const sp_plan_options o2 = opts(64, 8, 40, 100, 32, 128);
        const sp_plan_options o3 = opts(4096, 0, 0, 0, 16, 1);
        for (const auto& o : {o1, o2, o3}) {
            check_bins(a, o);
            check_sell(a, o);
        }
        for (int32_t P : {1, 2, 4, 8}) check_pstream(a, c % 2 ? o1 : o2, P);
        for (int32_t bits : {5, 8, 11, 15}) check_xwin(a, bits);
        for (int32_t pb : {5, 9, 16}) check_sweep(a, pb);
        for (int32_t T : {32, 64, 2048}) check_wcsr_tasks(rng, T);
        if (g_fail) {
            std::fprintf(stderr, "case %d (m=%d n=%d nnz=%zu) failed\n", c, m, n, a.col.size());
            return 1;
        }
    }
    std::printf("ok %d cases\n", cases);
    return 0;
}
