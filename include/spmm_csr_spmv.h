/*
 * spmm_csr_spmv -- sparse x dense products on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libspmm_csr_spmv.so.  Every pointer argument named as "device" is
 * a device (HBM) address; every call that takes `stream` enqueues its work on
 * that HIP stream (a hipStream_t passed as void*, NULL = the null stream) and
 * returns without waiting, unless its comment says it synchronises.
 *
 * Pages the operations follow (title, then section):
 *   [FMT]  「稀疏矩阵存储格式:COO、CSR、ELL、Hybrid 与块稀疏,SpMV 的容量与带宽账」
 *   [LSMR] 「CUDA LSMR 专栏（二）：用 CSR/CSC 双存储压榨双向 SpMV」
 *   [GEN]  「通用稀疏矩阵乘法CUDA算子实现」
 *   [BCSR] 「GPU加速实战用BCSR格式优化稀疏矩阵乘法附CUDA代码」
 *   [ASYNC] the AsyncSparse summary page (capital-peak.com, news 566)
 *
 * Conventions shared by all entry points
 *   - Indices are zero-based int32 ([LSMR] §5.1 uses zero-based indices).
 *     Sizes that do not fit int32 (m, n, nnz > INT32_MAX) are rejected with
 *     SP_ERR_SIZE, never truncated ([LSMR] §8).
 *   - Products use the BLAS axpby form  out = alpha * op(A) * in + beta * out
 *     ([LSMR] §5.2 folds the previous vector into the product through beta).
 *     beta == 0 means `out` is write-only: its old contents are not read.
 *   - The caller owns every buffer.  The library allocates no device memory in
 *     any call: scratch comes from a caller-provided workspace whose size is
 *     queried first ([GEN] §6: scratch belongs to the framework allocator).
 *   - Floating-point results are deterministic run to run: no floating-point
 *     atomics, fixed reduction order ([GEN] §2.4).
 *   - Errors are returned as status codes; nothing is thrown across the ABI.
 *     A failed HIP launch is reported as SP_ERR_HIP.
 */
#ifndef SPMM_CSR_SPMV_H
#define SPMM_CSR_SPMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
enum {
    SP_OK = 0,
    SP_ERR_NULL = 1,        /* a required pointer is NULL                    */
    SP_ERR_SIZE = 2,        /* a size is negative, too large or inconsistent */
    SP_ERR_INDEX = 3,       /* an input index is outside its dimension       */
    SP_ERR_WORKSPACE = 4,   /* workspace missing or smaller than queried     */
    SP_ERR_UNSUPPORTED = 5, /* option, shape or layout not supported         */
    SP_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed    */
    SP_ERR_STATE = 7,       /* plan used before sp_plan_bind, or similar     */
    SP_ERR_FILL = 8         /* block fill ratio below the requested minimum  */
};

/* Static string naming a status code (never NULL). */
const char* sp_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int sp_version(void);

/* --------------------------------------------------------- COO -> CSR
 * [FMT] §3 (and §2): count the entries of every row, prefix-sum the counts
 * into row_ptr, move each entry into its row's range; [GEN] §1.2 asks for
 * the result ordered by (row, col).
 *
 * Input: coo_row/coo_col/coo_val, nnz entries each, device, in any order.
 * Output (device, caller-allocated): row_ptr[m+1], col_idx[nnz], val[nnz].
 * Within a row, entries are ordered by column; entries with equal (row, col)
 * are kept as separate entries (duplicates are not summed) in their input
 * order.  The result is therefore unique and bit-exact.
 * work: device scratch of at least csr_build_from_coo_bufsize() bytes.
 * Synchronises `stream` once (to report SP_ERR_INDEX and to size the sort).
 * Errors: SP_ERR_NULL, SP_ERR_SIZE, SP_ERR_INDEX (some row not in [0,m) or
 * col not in [0,n); outputs are then unspecified), SP_ERR_WORKSPACE, SP_ERR_HIP.
 */
int csr_build_from_coo_bufsize(int64_t m, int64_t n, int64_t nnz, size_t* bytes);
int csr_build_from_coo(int64_t m, int64_t n, int64_t nnz,
                       const int32_t* coo_row, const int32_t* coo_col, const float* coo_val,
                       int32_t* row_ptr, int32_t* col_idx, float* val,
                       void* work, size_t work_bytes, void* stream);

/* COO -> CSR as csr_build_from_coo, for callers that cannot allocate device
 * memory (code whose harness forbids hipMalloc, loops that must not allocate):
 * no workspace argument; the scratch is a static 64 MiB device array that the
 * library holds on every GPU it runs on until the process ends.  Sizes whose
 * csr_build_from_coo_bufsize() exceeds 64 MiB (about 3.5 M entries with
 * m = 1 M rows; 16 bytes per entry plus 24 per row) are refused with
 * SP_ERR_WORKSPACE before any work is enqueued.  Every call on one GPU uses
 * the same array: calls that overlap in time on one GPU (on other streams or
 * from other host threads) race and must be ordered by the caller.
 * Synchronises `stream` once, as csr_build_from_coo.  Allocates nothing.
 * Errors: those of csr_build_from_coo, SP_ERR_WORKSPACE as above. */
int csr_build_from_coo_noalloc(int64_t m, int64_t n, int64_t nnz,
                               const int32_t* coo_row, const int32_t* coo_col, const float* coo_val,
                               int32_t* row_ptr, int32_t* col_idx, float* val, void* stream);

/* --------------------------------------------------------- CSR -> CSC
 * [LSMR] §2 and §4: the CSC of A is, array for array, the CSR of A^T; it is
 * built once, when the matrix is constructed.  Reading a CSC input as the
 * CSR of A^T and calling this again turns it back into the CSR of A.
 *
 * Input: CSR of an m x n matrix (device).  Output (device, caller-allocated):
 * col_ptr[n+1], row_idx[nnz], cval[nnz].  Within a column, entries are ordered
 * by row, and entries with equal (row, col) keep their CSR order; the result
 * is unique and bit-exact.  nnz must equal row_ptr[m].
 * work: at least csr_to_csc_bufsize() bytes.  Synchronises `stream` once.
 * Errors: SP_ERR_NULL, SP_ERR_SIZE, SP_ERR_INDEX, SP_ERR_WORKSPACE, SP_ERR_HIP.
 */
int csr_to_csc_bufsize(int64_t m, int64_t n, int64_t nnz, size_t* bytes);
int csr_to_csc(int64_t m, int64_t n, int64_t nnz,
               const int32_t* row_ptr, const int32_t* col_idx, const float* val,
               int32_t* col_ptr, int32_t* row_idx, float* cval,
               void* work, size_t work_bytes, void* stream);

/* --------------------------------------------------------- plan
 * [GEN] §4: a light profile of the matrix, taken the first time the matrix is
 * seen and kept with it, decides which kernel serves which rows; [LSMR] §5.3
 * names the statistics (row length l_i = row_ptr[i+1] - row_ptr[i], its mean,
 * variance and tail).  The plan holds the profile, the row-to-kernel
 * assignment for A (and for A^T when a CSC is given) and pointers to the
 * caller's arrays; it owns no device memory.
 *
 * Rows are assigned by length l:
 *   l <= wave_min            consecutive rows packed into groups of at most
 *                            group_nnz entries and 256 rows; a group is staged
 *                            through LDS and reduced by 1..64 lanes per row
 *                            (thread-per-row up to wave-per-row, [GEN] §2.1-2.2)
 *   wave_min < l <= block_min    one wave64 per row ([GEN] §2.2)
 *   block_min < l <= split_min   one 256-thread workgroup per row ([GEN] §2.3)
 *   l > split_min            split into segments of split_seg entries, one
 *                            workgroup each, partial sums reduced in fixed
 *                            order by the last segment to finish ([GEN] §2.4)
 * With use_sell = 1 the group rows are served instead from a SELL-C-sigma
 * copy ([GEN] §1.4) built in the workspace (C = 64 lanes, window sell_sigma);
 * use_sell = -1 (the default) picks SELL when every row has at most 64
 * entries, rows average at least 4 entries and the padded slots exceed the
 * entries by at most 20 % ([GEN] §4 rule table: short regular rows, padding
 * checked first); use_sell = 0 never uses it.  sp_plan_bind stores the SELL
 * columns as int16 offsets from the row when every SELL entry lies within
 * 32767 of its row (banded matrices: 6 instead of 8 bytes per slot), else
 * as int32 columns.
 *
 * Column-panel stream ([GEN] §2.5: random x gathers are the real cost once
 * x is much larger than the cache; §2.4: split long rows, reduce the pieces in
 * a fixed order): with col_panels = P in {1, 2, 4, 8} spmv and spmv_t use,
 * instead of the bins above, a copy of the matrix built at bind in which
 * the columns are cut into P panels of a power-of-two width and every row of
 * at most min(split_min, 4032) entries is stored panel by panel, cut into
 * row-aligned chunks of at most 4096 entries.  Panel p is served only by the
 * XCDs p, p + P, ..., so its gathers stay in one L2-sized slice of x; the
 * per-panel row sums are added in panel order.  Longer rows are summed in
 * segments of split_seg entries whose partials are added in segment order.
 * The default (-1) uses 8 panels when x exceeds 8 MiB and a sample of groups
 * shows columns spread over more than a quarter of the column range, else
 * none; SELL and panels exclude each other.  The copy costs 8 bytes per
 * entry plus 4 bytes per row and panel of workspace, and sp_plan_create
 * reads the column indices back to the host once to cut the chunks.
 *
 * x-window stream ([GEN] §2.5 as above; §2.1: stage through on-chip memory;
 * §2.4: long rows in pieces reduced in a fixed order): with x_window_bits =
 * b in 5..15, spmv and spmv_t instead cut x into windows of 2^b columns (at
 * most 256 windows).  A first kernel holds one window of x in LDS and forms
 * the product of every entry of that window from a window-major copy of the
 * matrix (column within the window as uint16, value); a second kernel reads
 * the products of a row chunk (at most 15360 entries and 1536 rows, in order)
 * back into LDS in CSR order and forms the row sums; rows longer than a
 * chunk are summed in chunk-sized segments added in segment order.  No
 * gather of x leaves LDS.  The default (-1) uses 2^15-column windows where
 * the column-panel rule above would pick 8 panels and x has at most 2^23
 * columns; explicit col_panels > 0 turns the automatic choice off; an
 * explicit b wins over col_panels; SELL excludes both.  The copy costs 14
 * bytes per entry (the products are rewritten by every call) plus small
 * tables; sp_plan_create reads the column indices back to the host once, and
 * returns SP_ERR_UNSUPPORTED for an explicit b that needs more than 256
 * windows.  Column indices outside [0, n) make sp_plan_create return
 * SP_ERR_INDEX whenever either stream is built.
 *
 * Phase-swept SpMM ([GEN] §3.1: with few right-hand sides the cost is the
 * B-row reads; §2.5: gathers that leave the cache are the real cost): with
 * spmm_phase_bits = b, sp_plan_bind builds a copy of A in which the columns
 * are cut into phases of 2^b columns and, for every block of 2048 rows cut
 * into 8 row ranges of about equal entry counts, each range's entries are
 * stored phase by phase (at most 2^21 columns).  spmm with
 * N in {4, 8, 16} (B and C rows 16-byte aligned) then runs one workgroup per
 * block that keeps the block's C rows in LDS and sweeps the phases in order,
 * so the B rows every XCD reads at a time form one slice of 2^b rows that
 * stays in its L2; each C row is summed by one wave in a fixed order.  The
 * default (-1) builds it when max_N (of the bind) is 4..16, B (n * max_N
 * floats) exceeds 8 MiB, no row is longer than 8192 entries and a sample of
 * rows shows columns spread over more than a quarter of the range and the
 * matrix has at most 2^21 columns, with 2^b * max_N * 4 bytes = 512 KiB
 * slices.
 * An explicit b above 21 is taken as 21.  The copy costs 8 bytes per entry
 * plus 4 bytes per (block, range, phase); sp_plan_bind reads the row pointer
 * and column indices back once to lay it out.
 */
typedef struct sp_plan sp_plan;

typedef struct sp_plan_options {
    int32_t group_nnz;   /* entries per group, 64..4096 (default 2048)        */
    int32_t wave_min;    /* default 256; must be <= group_nnz                 */
    int32_t block_min;   /* default 4096; >= wave_min                         */
    int32_t split_min;   /* default 32768; >= block_min                       */
    int32_t split_seg;   /* entries per split segment, >= 16 (default 8192)   */
    int32_t use_sell;    /* -1 auto (default), 0 off, 1 on                     */
    int32_t sell_sigma;  /* sorting window in rows for SELL, >= 1 (default 1024) */
    int32_t xcd_remap;   /* 1 (default): consecutive groups go to one XCD     */
    int32_t col_panels;  /* -1 auto (default), 0 off, or 1, 2, 4, 8 panels    */
    int32_t x_window_bits; /* -1 auto (default), 0 off, or 5..15: x windows of 2^bits columns */
    int32_t spmm_phase_bits; /* -1 auto (default), 0 off, or 5..24: SpMM phases of 2^bits columns */
} sp_plan_options;

/* Row-length profile and bin sizes of one direction of a plan. */
typedef struct sp_profile {
    int64_t rows, cols, nnz;
    double mean, var, cv;        /* population variance, cv = sqrt(var)/mean  */
    int64_t p95, p99, max_len;   /* nearest-rank percentiles of l_i           */
    int64_t empty_rows;
    int64_t group_tasks, group_rows, group_nnz;
    int64_t wave_rows, wave_nnz;
    int64_t block_rows, block_nnz;
    int64_t split_rows, split_segments, split_nnz;
    int64_t sell_slots;          /* padded SELL slots (0 without SELL)         */
    int64_t col_panels;          /* panels of the column-panel stream (0: off)  */
    int64_t x_window_bits;       /* window bits of the x-window stream (0: off) */
    int64_t spmm_phase_bits;     /* phase bits of the phase-swept SpMM copy, set by
                                    sp_plan_bind (0: off)                       */
} sp_profile;

/* Fills *opt with the defaults listed above. */
int sp_plan_options_default(sp_plan_options* opt);

/* Creates a plan for the m x n CSR matrix (row_ptr, col_idx, val: device).
 * opt == NULL: the defaults, or the options the tuning cache holds for this
 * matrix's dispatch key (see sp_autotune_spmv below).
 * When col_ptr/row_idx/cval (the CSC, e.g. from csr_to_csc) are non-NULL the
 * plan also serves spmv_t ([LSMR] §4: both directions run as non-transposed
 * CSR products); otherwise spmv_t returns SP_ERR_UNSUPPORTED.  opt may be NULL
 * (defaults).  Copies row_ptr (and col_ptr) to the host once: synchronises
 * `stream`.  The arrays must stay alive and unchanged until sp_plan_destroy.
 * Errors: SP_ERR_NULL, SP_ERR_SIZE, SP_ERR_UNSUPPORTED (bad option or an
 * explicit x window width that does not fit), SP_ERR_INDEX (a column index
 * outside [0, n) seen while building a stream), SP_ERR_HIP. */
int sp_plan_create(sp_plan** plan, int64_t m, int64_t n, int64_t nnz,
                   const int32_t* row_ptr, const int32_t* col_idx, const float* val,
                   const int32_t* col_ptr, const int32_t* row_idx, const float* cval,
                   const sp_plan_options* opt, void* stream);

/* Bytes of device workspace the plan needs to serve spmv/spmv_t and spmm with
 * up to max_N right-hand-side columns ([LSMR] §5.1: one query covering both
 * directions).  For a view (below): the bytes of its per-call scratch only. */
int sp_plan_workspace_size(const sp_plan* plan, int32_t max_N, size_t* bytes);

/* Attaches a device workspace of at least the queried size and uploads the
 * plan's task tables into it (enqueued on `stream`).  The workspace must stay
 * alive until sp_plan_destroy or the next bind.  Binding a view attaches its
 * scratch instead (no upload, no synchronisation; SP_ERR_STATE when its base
 * is not bound).  Errors: SP_ERR_NULL, SP_ERR_SIZE (max_N < 1),
 * SP_ERR_WORKSPACE, SP_ERR_INDEX (a stored index outside its dimension),
 * SP_ERR_STATE, SP_ERR_HIP.
 *
 * Concurrency ([LSMR] §5.1: the matrix is set up once, and each call only
 * supplies its vectors).  After bind the task tables and matrix copies are
 * read-only; what a product writes besides its output (split-row partials and
 * arrival counters, panel row sums, x-window products) lives in the per-call
 * scratch of the plan or view it is called on.  So calls on one plan or view
 * must be ordered (one stream at a time), and calls on different views of a
 * plan, or on the plan and its views, may run concurrently on different
 * streams when their outputs are disjoint. */
int sp_plan_bind(sp_plan* plan, void* work, size_t work_bytes, int32_t max_N, void* stream);

/* Creates a view of `base` (a plan, or a view: then of its plan): an sp_plan
 * that every product entry point accepts, which reads the base's bound tables
 * and owns only a per-call scratch, attached with sp_plan_bind after
 * sp_plan_workspace_size (with its own max_N).  Host-only: allocates the small
 * host struct, no device memory.  A view stops working (SP_ERR_STATE) when
 * its base is bound again; bind the view again then.  Destroy the views of a
 * plan before the plan (sp_plan_destroy of a plan with live views returns
 * SP_ERR_STATE and frees nothing).  Errors: SP_ERR_NULL, SP_ERR_SIZE (out of
 * host memory). */
int sp_plan_view_create(const sp_plan* base, sp_plan** view);

/* Profile of A (transposed = 0) or of A^T (transposed = 1); a view reports its
 * base's. */
int sp_plan_profile(const sp_plan* plan, int32_t transposed, sp_profile* out);

/* Frees the host-side plan or view (NULL is accepted).  SP_ERR_STATE, freeing
 * nothing, for a plan whose views are not all destroyed. */
int sp_plan_destroy(sp_plan* plan);

/* --------------------------------------------------------- dispatch key, tuning cache, autotune
 * [GEN] §4: the first time a matrix is seen, a light profile gives a stable
 * dispatch key; a small autotune times 2-4 candidate kernels with events on
 * the stream, caches the fastest configuration and never benchmarks on every
 * call; a version number invalidates the cache for a matrix that changes.
 *
 * The key: format (0 = CSR), dtype (0 = fp32 values), index_bits (32),
 * transposed (0: A, 1: A^T through the CSC), rows, cols, nnz, N (right-hand
 * sides; 1 = SpMV), arch (950 = gfx950), the row-length profile quantised as
 * floor(4 log2(1 + v)) for the mean, p95 and maximum row length and
 * floor(8 cv) for the coefficient of variation, and the caller's version.
 * Keys compare field by field (the struct is zero-filled by the library).
 *
 * The cache is process-wide (all devices, all threads; a mutex guards it) and
 * maps a key to plan options.  sp_plan_create with opt == NULL builds the key
 * of A (N = 1, version 0) and, when the cache holds options for it, uses them
 * for both directions instead of the defaults.
 *
 * sp_autotune_spmv: for each of the ncand (1..16) candidate option sets,
 * creates a plan on the CSR (row_ptr, col_idx, val: device), binds it to `work`
 * (at least sp_autotune_workspace_size() bytes), runs one warm-up spmv and
 * times `reps` spmv calls y = A x between two events on `stream`; writes the
 * mean milliseconds per call to ms[i], the fastest index to *best (ties: the
 * lower index) and stores that candidate under the key of A (N = 1, the given
 * version).  Overwrites y.  Synchronises; allocates no device memory (the
 * plans are created and destroyed on the host).  Errors: those of
 * sp_plan_create / sp_plan_bind / spmv, SP_ERR_SIZE (ncand or reps out of
 * range), SP_ERR_WORKSPACE.
 */
typedef struct sp_dispatch_key {
    int32_t format, dtype, index_bits, transposed;
    int64_t rows, cols, nnz;
    int32_t N, arch;
    int32_t avg_len_q, p95_len_q, max_len_q, cv_q;
    uint64_t version;
} sp_dispatch_key;

int sp_plan_dispatch_key(const sp_plan* plan, int32_t transposed, int32_t N, uint64_t version,
                         sp_dispatch_key* key);
int sp_tune_cache_store(const sp_dispatch_key* key, const sp_plan_options* opt);  /* SP_ERR_UNSUPPORTED: bad options */
int sp_tune_cache_lookup(const sp_dispatch_key* key, sp_plan_options* opt, int32_t* found);
int sp_tune_cache_clear(void);
int sp_tune_cache_size(int64_t* entries);
int sp_autotune_workspace_size(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                               const float* val, const sp_plan_options* candidates, int32_t ncand,
                               size_t* bytes, void* stream);
int sp_autotune_spmv(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                     const float* val, const sp_plan_options* candidates, int32_t ncand, const float* x, float* y,
                     int32_t reps, uint64_t version, void* work, size_t work_bytes, int32_t* best, float* ms,
                     void* stream);

/* --------------------------------------------------------- products
 * spmv:   y = alpha * A x + beta * y     x: n floats, y: m floats (device)
 *         ([LSMR] §2, (Av)_i as a sum over the row's entries; [LSMR] §5.2)
 * spmv_t: z = alpha * A^T u + beta * z   u: m floats, z: n floats (device),
 *         computed on the CSC held by the plan ([LSMR] §2, §4)
 * spmm:   C = alpha * A B + beta * C     B: n x N row-major with leading
 *         dimension ldb >= N, C: m x N row-major with ldc >= N (device)
 *         ([GEN] §3, C[i,n] sums A[i,k] B[k,n] over the row's entries)
 * `plan` is a bound plan or a bound view (see sp_plan_view_create).
 * Never allocate, never synchronise.  x/u/B must not alias y/z/C.
 * Errors: SP_ERR_NULL, SP_ERR_SIZE (N < 1, ld < N, N above the bound max_N),
 * SP_ERR_STATE (not bound, or a view whose base was bound again since),
 * SP_ERR_UNSUPPORTED (spmv_t without CSC), SP_ERR_HIP.
 */
int spmv(const sp_plan* plan, float alpha, const float* x, float beta, float* y, void* stream);
int spmv_t(const sp_plan* plan, float alpha, const float* u, float beta, float* z, void* stream);
int spmm(const sp_plan* plan, int32_t N, float alpha, const float* B, int64_t ldb,
         float beta, float* C, int64_t ldc, void* stream);

/* --------------------------------------------------------- CSR -> BSR
 * [BCSR] §1: a block is stored when it holds at least one entry; the format is
 * brow_ptr[mb+1] (block row pointer), bcol[nnzb] (block column of each stored
 * block, increasing within a block row) and the nnzb dense bs x bs blocks one
 * after another, each row-major ([BCSR] §2.1).  [ASYNC] §2.2.1 measures the
 * layout's waste by the fill ratio nnz / (nnzb * bs * bs); [GEN] §6 warns that
 * a conversion only pays when it is reused, so the analysis step reports the
 * fill ratio and can refuse the conversion.
 *
 * Square blocks, bs in {1, 2, 4, 8, 16, 32, 64}; mb = ceil(m / bs),
 * kb = ceil(n / bs) (the last block row / column is padded with zeros).
 * Input: a CSR whose rows are sorted by column (as csr_build_from_coo
 * returns it), device arrays.  The value at in-block position (r, c) of block
 * (I, J) is the sum of the CSR entries at element (I*bs + r, J*bs + c), added
 * in CSR order in fp32 starting from the first; other positions are +0.
 * bf16 output is that sum rounded once to nearest-even.  Bit-exact and unique.
 *
 * csr_to_bsr_analyze: writes brow_ptr (device, mb+1 entries), returns nnzb and
 * the fill ratio (host; 1.0 when nnzb == 0) and synchronises `stream` once.
 * work: at least csr_to_bsr_bufsize() bytes.  Errors: SP_ERR_NULL,
 * SP_ERR_SIZE (row_ptr[m] != nnz, sizes beyond int32), SP_ERR_INDEX (a column
 * outside [0, n)), SP_ERR_UNSUPPORTED (bs not supported, or a row not sorted),
 * SP_ERR_WORKSPACE, SP_ERR_FILL (fill ratio < min_fill: *nnzb and *fill are
 * still set, brow_ptr is written), SP_ERR_HIP.
 * csr_to_bsr_fill: writes bcol (device, nnzb) and bval (device, nnzb*bs*bs
 * fp32, or bf16 bit patterns when out_bf16 = 1) for the brow_ptr of the
 * analysis; fp32 output needs bval 16-byte aligned when bs % 4 == 0.  Never
 * synchronises; never writes outside the ranges brow_ptr gives.
 */
int csr_to_bsr_bufsize(int64_t m, int64_t n, int64_t nnz, int32_t bs, size_t* bytes);
int csr_to_bsr_analyze(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                       int32_t bs, double min_fill, int32_t* brow_ptr, int64_t* nnzb, double* fill,
                       void* work, size_t work_bytes, void* stream);
int csr_to_bsr_fill(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                    const float* val, int32_t bs, const int32_t* brow_ptr, int64_t nnzb, int32_t* bcol,
                    void* bval, int32_t out_bf16, void* stream);

/* --------------------------------------------------------- BSR SpMV
 * [BCSR] §2 (block sparse matrix-vector product over the BCSR layout above):
 * y = alpha * A x + beta * y for the m x n matrix A given as bs x bs fp32
 * blocks (layout of csr_to_bsr), x: n floats, y: m floats (device).  Element
 * rows >= m and columns >= n of the padded last block row / column are not
 * read through x nor written.  A block whose column index lies outside
 * [0, kb) contributes nothing; block pointers are clamped to [0, nnzb].
 * bval must be 16-byte aligned, and x too when bs >= 4.  bs in {1, 2, 4, 8,
 * 16, 32, 64}.  Never allocates, never synchronises; deterministic.
 * Errors: SP_ERR_NULL, SP_ERR_SIZE, SP_ERR_UNSUPPORTED, SP_ERR_HIP.
 */
int bsr_spmv(int64_t m, int64_t n, int32_t bs, int64_t nnzb, const int32_t* brow_ptr, const int32_t* bcol,
             const float* bval, float alpha, const float* x, float beta, float* y, void* stream);

/* The same product by the other thread mapping of [BCSR] §2 (§2.2, a warp
 * covers whole columns, where bsr_spmv follows §2.1, a warp covers whole
 * blocks): each block row is served by bs lanes, lane r owning element row r,
 * which walks the row's blocks reading its own row of each block and ends
 * with the row's whole sum (no reduction across lanes).  [BCSR] §3 compares
 * the two; bench.py reports both on the 64 x 64-block workload.  Arguments,
 * layout, alignment and errors as bsr_spmv; deterministic. */
int bsr_spmv_rowwise(int64_t m, int64_t n, int32_t bs, int64_t nnzb, const int32_t* brow_ptr, const int32_t* bcol,
                     const float* bval, float alpha, const float* x, float beta, float* y, void* stream);

/* --------------------------------------------------------- windowed rows (WCSR), windowed SpMM
 * [ASYNC] §2.2.2: rows are grouped into windows of a fixed height; per window
 * the union of its rows' column indices is kept (padding columns carry -1)
 * and the values of those columns are stored densely, so that a row of B is
 * fetched once per window; [ASYNC] §4: the window's B rows are gathered into
 * on-chip memory and its dense tile is multiplied on the matrix units.
 *
 * Layout (windows of 64 rows, nw = ceil(m / 64)): window_ptr[nw+1] (first
 * compressed column of each window), window_col[total_cols] (the window's
 * distinct columns, ascending, then -1 up to a multiple of pad), values
 * [total_cols][64] fp32: values[q*64 + r] is row 64w + r of the window at
 * compressed column q (entries at one position added in CSR order in fp32,
 * starting from the first; 0 where there is none, padding included).
 * pad in {1, 2, 4, 8, 16, 32}.  Input: a CSR with rows sorted by column.
 *
 * csr_to_wcsr_analyze: writes window_ptr (device), returns total_cols and the
 * fill nnz / (total_cols * 64) (host; 1.0 when total_cols == 0); synchronises
 * once; work >= csr_to_wcsr_bufsize() bytes.  Errors as csr_to_bsr_analyze
 * (SP_ERR_INDEX, SP_ERR_UNSUPPORTED for unsorted rows or a bad pad, ...).
 * csr_to_wcsr_fill: writes window_col and values (device, caller-allocated:
 * total_cols ints and total_cols * 64 floats); never synchronises, never
 * writes outside the ranges window_ptr gives.
 * wcsr_spmm: C = alpha * A B + beta * C with B n x N and C m x N row-major
 * (fp32, device); N % 4 == 0, ldb % 4 == 0, B and values 16-byte aligned;
 * window_col and values may be NULL when total_cols == 0.  Deterministic;
 * never allocates, never synchronises.  The product runs over the stored
 * window tiles, zeros included (0 * Inf is NaN where a row of the window has
 * no entry at a column whose B row holds Inf or NaN); padding columns (-1)
 * are skipped and never read from B.
 */
int csr_to_wcsr_bufsize(int64_t m, int64_t n, int64_t nnz, size_t* bytes);
int csr_to_wcsr_analyze(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                        int32_t pad, int32_t* window_ptr, int64_t* total_cols, double* fill,
                        void* work, size_t work_bytes, void* stream);
int csr_to_wcsr_fill(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                     const float* val, const int32_t* window_ptr, int64_t total_cols, int32_t* window_col,
                     float* values, void* stream);
int wcsr_spmm(int64_t m, int64_t n, const int32_t* window_ptr, const int32_t* window_col, const float* values,
              int32_t N, float alpha, const float* B, int64_t ldb, float beta, float* C, int64_t ldc,
              void* stream);

/* Task split of the windowed SpMM ([ASYNC] §4.2): a window of more than
 * task_cols compressed columns is cut into tasks of task_cols columns (the
 * last one shorter); every other window is one task.  One workgroup per task
 * and column tile of C, so a few very wide windows no longer hold the tail of
 * the launch.  The tasks of a split window store partial tiles in slots of
 * the caller's workspace, and a second kernel adds each split window's
 * partials in task order and writes C.  The page adds the parts with
 * atomics; here the order is fixed: results are reproducible, equal bit for
 * bit to wcsr_spmm on windows that are not split, and within fp32 rounding
 * of it on the others.
 *
 * wcsr_tasks_bufsize: bytes of the task table for m rows, total_cols
 * compressed columns (from csr_to_wcsr_analyze) and task_cols, a positive
 * multiple of 32.
 * wcsr_tasks_build: reads window_ptr (device) back to the host, builds the
 * task table there and writes it to `table` (device, caller-allocated,
 * 16-byte aligned; built once per matrix, read-only afterwards); returns, on
 * the host, the number of tasks and of partial slots.  Synchronises `stream`.
 * SP_ERR_INDEX when window_ptr is not nondecreasing inside [0, total_cols].
 * Table layout, nw = ceil(m / 64): int32 {tasks, slots, 0, split windows} at
 * byte 0; int32 quadruples {window, first slot, tasks, 0} per split window,
 * in window order, at byte 256; int32 quadruples {window, first column, end
 * column, slot or -1} per task at byte 256 + 16 nw rounded up to a multiple
 * of 256.  A split window's tasks take consecutive slots in column order,
 * the split windows one after another in window order.  Tasks are stored
 * widest first (end - first column decreasing; equal widths in window order,
 * then column order): workgroups start roughly in index order, so the
 * longest tasks start first and the short ones fill in behind them.
 * wcsr_spmm_tasks_bufsize: workspace bytes of one call with nslots slots and
 * N columns (nslots * 64 * N * 4; 0 when nslots == 0).
 * wcsr_spmm_tasks: C = alpha * A B + beta * C as wcsr_spmm (same operands,
 * layouts and requirements), over a table built for the same m; ntasks and
 * nslots are the build's results.  work: device, 16-byte aligned, >=
 * wcsr_spmm_tasks_bufsize() bytes, may be NULL when nslots == 0; its contents
 * on entry do not matter, and calls that share one workspace must not
 * overlap.  Never allocates, never synchronises.  A table that needs more
 * slots than nslots makes the call write nothing.
 */
int wcsr_tasks_bufsize(int64_t m, int64_t total_cols, int32_t task_cols, size_t* bytes);
int wcsr_tasks_build(int64_t m, const int32_t* window_ptr, int64_t total_cols, int32_t task_cols, void* table,
                     size_t table_bytes, int64_t* ntasks, int64_t* nslots, void* stream);
int wcsr_spmm_tasks_bufsize(int64_t nslots, int32_t N, size_t* bytes);
int wcsr_spmm_tasks(int64_t m, int64_t n, const void* table, int64_t ntasks, int64_t nslots,
                    const int32_t* window_col, const float* values, int32_t N, float alpha, const float* B,
                    int64_t ldb, float beta, float* C, int64_t ldc, void* work, size_t work_bytes, void* stream);

/* --------------------------------------------------------- BSR SpMM
 * [BCSR] §1 and [ASYNC] §2.2.1: block row pointer brow_ptr[mb+1], block column
 * index bcol[nnzb] (increasing within a block row), and the nnzb dense
 * bs x bs blocks stored one after another, each row-major ([BCSR] §2.1 indexes
 * a block as row*bs + col).  [GEN] §3.4: each non-zero block is a small dense
 * GEMM, here on MFMA with bf16 inputs and fp32 accumulation ([GEN] §5).
 *
 * C (mb*bs x N fp32, row-major, ldc >= N) = alpha * A B + beta * C, with
 * B (kb*bs x N bf16 bit patterns, row-major, ldb >= N).  Supported: bs == 64,
 * N % 8 == 0, ldb % 8 == 0, ldc % 4 == 0, B and C 16-byte aligned.  Widths
 * that are multiples of 256 (or of 128) take the pipelined kernels; other
 * widths a plain 64-column-tile kernel whose last tile reads no B column and
 * writes no C column at or past N.
 * work: at least bsr_spmm_bufsize() bytes (may be 0 bytes: then NULL is fine).
 * The block structure is not validated (no synchronisation): block pointers
 * are clamped to [0, nnzb], and a block whose column index lies outside
 * [0, kb) contributes nothing; B is never read through such an index.
 * Never synchronises.
 * Errors: SP_ERR_NULL, SP_ERR_SIZE, SP_ERR_UNSUPPORTED, SP_ERR_WORKSPACE, SP_ERR_HIP.
 */
int bsr_spmm_bufsize(int64_t mb, int64_t kb, int32_t bs, int64_t nnzb, int32_t N, size_t* bytes);
int bsr_spmm(int64_t mb, int64_t kb, int32_t bs, int64_t nnzb,
             const int32_t* brow_ptr, const int32_t* bcol, const uint16_t* bval,
             int32_t N, const uint16_t* B, int64_t ldb,
             float alpha, float beta, float* C, int64_t ldc,
             void* work, size_t work_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPMM_CSR_SPMV_H */
