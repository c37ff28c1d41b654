/*
 * CPU oracle for the sparse x dense products.  TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, the smoke check of __graft_entry__ and the cpu_baseline leg of
 * bench.py may load this file's library.  It shares no code, header, table or
 * helper with the HIP library in spmm_csr_spmv_amd/; neither side includes or
 * links the other.  Everything here is a plain, slow, single-threaded loop
 * written for readability; floating point is accumulated in fp64.
 *
 * Pages cited (title, then section):
 *   [FMT]  「稀疏矩阵存储格式:COO、CSR、ELL、Hybrid 与块稀疏,SpMV 的容量与带宽账」
 *   [LSMR] 「CUDA LSMR 专栏（二）：用 CSR/CSC 双存储压榨双向 SpMV」
 *   [GEN]  「通用稀疏矩阵乘法CUDA算子实现」
 *   [BCSR] 「GPU加速实战用BCSR格式优化稀疏矩阵乘法附CUDA代码」
 *   [ASYNC] the AsyncSparse summary page (capital-peak.com, news 566)
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository as well):
 *   - COO duplicates are kept as separate CSR entries (no summation).
 *   - Inside a CSR row, entries are ordered by column; equal columns keep the
 *     order in which they appear in the COO input.
 *   - Inside a CSC column, entries are ordered by row; equal rows keep their
 *     CSR order.
 *   - y = alpha*A*x + beta*y; when beta == 0 the old y is not read.
 *   - BSR blocks are stored row-major inside each block.
 *   - CSR -> BSR: entries that share an element position are summed in CSR
 *     order in fp32; bf16 blocks are that sum rounded once to nearest-even.
 *   - CSR -> WCSR: the same duplicate rule; a window's compressed columns are
 *     ascending and padded with -1 to a multiple of `pad`; values are stored
 *     column by column inside a window.
 *   - SELL-C-sigma: windows of sigma rows sorted by decreasing length (ties by
 *     row index), slices of C rows padded to the slice's longest row, slot k of
 *     lane j stored at slice_ptr[s] + k*C + j; padded slots hold column -1.
 *
 * Parity pins: every function below is pinned by tests in tests/ that do not
 * call the function under test to produce their expected values (worked
 * example of [FMT] §2-§4, dense brute force, invariants).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

#define ORACLE_OK 0
#define ORACLE_ERR_SIZE 2
#define ORACLE_ERR_INDEX 3

/* ------------------------------------------------------------------------ */
/* COO -> CSR  ([FMT] §3: count entries per row, prefix-sum the counts into   */
/* the row pointer, then move column/value into each row's range; [GEN] §1.2 */
/* asks for rows ordered by (row, col)).                                     */
/* ------------------------------------------------------------------------ */

typedef struct { int32_t col; int64_t pos; } col_pos;

static int cmp_col_pos(const void* a, const void* b)
{
    const col_pos* p = (const col_pos*)a;
    const col_pos* q = (const col_pos*)b;
    if (p->col != q->col) return p->col < q->col ? -1 : 1;
    if (p->pos != q->pos) return p->pos < q->pos ? -1 : 1;
    return 0;
}

int oracle_coo_to_csr(int64_t m, int64_t n, int64_t nnz,
                      const int32_t* row, const int32_t* col, const float* val,
                      int32_t* row_ptr, int32_t* col_out, float* val_out)
{
    if (m < 0 || n < 0 || nnz < 0 || m > INT32_MAX || n > INT32_MAX || nnz > INT32_MAX)
        return ORACLE_ERR_SIZE;
    for (int64_t i = 0; i < nnz; ++i)
        if (row[i] < 0 || row[i] >= m || col[i] < 0 || col[i] >= n) return ORACLE_ERR_INDEX;

    /* 1. count entries of each row */
    int64_t* count = (int64_t*)calloc((size_t)m + 1, sizeof(int64_t));
    for (int64_t i = 0; i < nnz; ++i) count[row[i]] += 1;

    /* 2. exclusive prefix sum -> row pointer */
    int64_t run = 0;
    for (int64_t r = 0; r < m; ++r) { row_ptr[r] = (int32_t)run; run += count[r]; }
    row_ptr[m] = (int32_t)run;

    /* 3. place every entry, in input order, at the next free slot of its row */
    int64_t* next = (int64_t*)malloc(((size_t)m + 1) * sizeof(int64_t));
    for (int64_t r = 0; r < m; ++r) next[r] = row_ptr[r];
    col_pos* slot = (col_pos*)malloc(((size_t)nnz + 1) * sizeof(col_pos));
    for (int64_t i = 0; i < nnz; ++i) {
        int64_t p = next[row[i]]++;
        slot[p].col = col[i];
        slot[p].pos = i;
    }

    /* 4. order each row by (column, input position) */
    for (int64_t r = 0; r < m; ++r) {
        int64_t b = row_ptr[r], e = row_ptr[r + 1];
        if (e - b > 1) qsort(slot + b, (size_t)(e - b), sizeof(col_pos), cmp_col_pos);
    }
    for (int64_t p = 0; p < nnz; ++p) {
        col_out[p] = slot[p].col;
        val_out[p] = val[slot[p].pos];
    }
    free(slot); free(next); free(count);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* CSR -> CSC  ([LSMR] §2 and §4: CSC(A) has the memory layout of CSR(A^T);   */
/* built once by counting entries per column, prefix sum, and walking the    */
/* rows in order so that each column receives its rows in ascending order).  */
/* ------------------------------------------------------------------------ */
int oracle_csr_to_csc(int64_t m, int64_t n, const int32_t* row_ptr, const int32_t* col,
                      const float* val, int32_t* col_ptr, int32_t* row_idx, float* val_out)
{
    if (m < 0 || n < 0 || m > INT32_MAX || n > INT32_MAX) return ORACLE_ERR_SIZE;
    int64_t nnz = row_ptr[m];
    for (int64_t p = 0; p < nnz; ++p)
        if (col[p] < 0 || col[p] >= n) return ORACLE_ERR_INDEX;

    int64_t* count = (int64_t*)calloc((size_t)n + 1, sizeof(int64_t));
    for (int64_t p = 0; p < nnz; ++p) count[col[p]] += 1;
    int64_t run = 0;
    for (int64_t c = 0; c < n; ++c) { col_ptr[c] = (int32_t)run; run += count[c]; }
    col_ptr[n] = (int32_t)run;

    int64_t* next = (int64_t*)malloc(((size_t)n + 1) * sizeof(int64_t));
    for (int64_t c = 0; c < n; ++c) next[c] = col_ptr[c];
    for (int64_t r = 0; r < m; ++r) {
        for (int64_t p = row_ptr[r]; p < row_ptr[r + 1]; ++p) {
            int64_t q = next[col[p]]++;
            row_idx[q] = (int32_t)r;
            val_out[q] = val[p];
        }
    }
    free(next); free(count);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* SpMV  y = alpha*A*x + beta*y  ([LSMR] §2: (Av)_i is the sum over the row's */
/* entries of value times x at the entry's column; [LSMR] §5.2: the old       */
/* vector is folded in through beta).                                        */
/* scale_i = |alpha| * sum_p |val_p * x[col_p]| + |beta| * |y_i|  is the      */
/* magnitude a rounding error of the GPU result is measured against.         */
/* rows == NULL computes every row; otherwise only rows[0..nrows) and the    */
/* results go to y_out[k], scale_out[k] for k-th listed row.                  */
/* ------------------------------------------------------------------------ */
void oracle_spmv(int64_t m, const int32_t* row_ptr, const int32_t* col, const float* val,
                 const float* x, double alpha, double beta, const float* y_in,
                 const int64_t* rows, int64_t nrows, double* y_out, double* scale_out)
{
    int64_t count = rows ? nrows : m;
    for (int64_t k = 0; k < count; ++k) {
        int64_t i = rows ? rows[k] : k;
        double s = 0.0, a = 0.0;
        for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) {
            double t = (double)val[p] * (double)x[col[p]];
            s += t;
            a += fabs(t);
        }
        double y = alpha * s;
        double sc = fabs(alpha) * a;
        if (beta != 0.0) {
            y += beta * (double)y_in[i];
            sc += fabs(beta) * fabs((double)y_in[i]);
        }
        y_out[k] = y;
        if (scale_out) scale_out[k] = sc;
    }
}

/* A second, independent route to z = alpha*A^T*u + beta*z: scatter every CSR
 * entry (i, j, v) into z_j += v * u_i.  Used only to cross-check the CSC route
 * on small inputs. */
void oracle_spmv_t_scatter(int64_t m, int64_t n, const int32_t* row_ptr, const int32_t* col,
                           const float* val, const float* u, double alpha, double beta,
                           const float* z_in, double* z_out, double* scale_out)
{
    double* acc = (double*)calloc((size_t)n + 1, sizeof(double));
    double* mag = (double*)calloc((size_t)n + 1, sizeof(double));
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) {
            double t = (double)val[p] * (double)u[i];
            acc[col[p]] += t;
            mag[col[p]] += fabs(t);
        }
    }
    for (int64_t j = 0; j < n; ++j) {
        double z = alpha * acc[j];
        double sc = fabs(alpha) * mag[j];
        if (beta != 0.0) {
            z += beta * (double)z_in[j];
            sc += fabs(beta) * fabs((double)z_in[j]);
        }
        z_out[j] = z;
        if (scale_out) scale_out[j] = sc;
    }
    free(acc); free(mag);
}

/* ------------------------------------------------------------------------ */
/* SpMM  C = alpha*A*B + beta*C  ([GEN] §3: C[i,n] sums A[i,k]*B[k,n] over the */
/* columns k present in row i).  B is K x N row-major with leading dimension  */
/* ldb, C is M x N row-major with leading dimension ldc.  The outputs of the  */
/* listed rows (or all rows) are written densely: out[k*N + n].               */
/* ------------------------------------------------------------------------ */
void oracle_spmm(int64_t m, const int32_t* row_ptr, const int32_t* col, const float* val,
                 int64_t N, const float* B, int64_t ldb, double alpha, double beta,
                 const float* C_in, int64_t ldc, const int64_t* rows, int64_t nrows,
                 double* C_out, double* scale_out)
{
    int64_t count = rows ? nrows : m;
    for (int64_t k = 0; k < count; ++k) {
        int64_t i = rows ? rows[k] : k;
        for (int64_t c = 0; c < N; ++c) {
            double s = 0.0, a = 0.0;
            for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) {
                double t = (double)val[p] * (double)B[(int64_t)col[p] * ldb + c];
                s += t;
                a += fabs(t);
            }
            double y = alpha * s;
            double sc = fabs(alpha) * a;
            if (beta != 0.0) {
                double old = (double)C_in[i * ldc + c];
                y += beta * old;
                sc += fabs(beta) * fabs(old);
            }
            C_out[k * N + c] = y;
            if (scale_out) scale_out[k * N + c] = sc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* BSR ([BCSR] §1: block row pointer, block column index, dense blocks stored  */
/* one after another; the page's code indexes a block as row*bs + col, i.e.   */
/* row-major).  bf16 is the upper half of an IEEE binary32 word, so widening  */
/* it to double is exact.                                                     */
/* ------------------------------------------------------------------------ */
double oracle_bf16_to_double(uint16_t h)
{
    uint32_t w = (uint32_t)h << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* Expand BSR to CSR keeping every in-block entry (explicit zeros included):
 * element row I*bs + r holds, for each block b of block-row I in stored order,
 * the bs entries (bcol[b]*bs + c, A_b[r][c]) for c = 0..bs-1. */
int oracle_bsr_to_csr(int64_t mb, int64_t bs, const int32_t* brow_ptr, const int32_t* bcol,
                      const uint16_t* bval, int32_t* row_ptr, int32_t* col, double* val)
{
    int64_t p = 0;
    for (int64_t I = 0; I < mb; ++I) {
        for (int64_t r = 0; r < bs; ++r) {
            row_ptr[I * bs + r] = (int32_t)p;
            for (int64_t b = brow_ptr[I]; b < brow_ptr[I + 1]; ++b) {
                for (int64_t c = 0; c < bs; ++c) {
                    col[p] = (int32_t)((int64_t)bcol[b] * bs + c);
                    val[p] = oracle_bf16_to_double(bval[(b * bs + r) * bs + c]);
                    ++p;
                }
            }
        }
    }
    row_ptr[mb * bs] = (int32_t)p;
    return ORACLE_OK;
}

/* SpMM over a CSR with fp64 values and a bf16 right-hand side (the expanded
 * BSR route).  Same output convention as oracle_spmm. */
void oracle_spmm_bf16(int64_t m, const int32_t* row_ptr, const int32_t* col, const double* val,
                      int64_t N, const uint16_t* B, int64_t ldb, double alpha, double beta,
                      const float* C_in, int64_t ldc, const int64_t* rows, int64_t nrows,
                      double* C_out, double* scale_out)
{
    int64_t count = rows ? nrows : m;
    for (int64_t k = 0; k < count; ++k) {
        int64_t i = rows ? rows[k] : k;
        for (int64_t c = 0; c < N; ++c) {
            double s = 0.0, a = 0.0;
            for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) {
                double t = val[p] * oracle_bf16_to_double(B[(int64_t)col[p] * ldb + c]);
                s += t;
                a += fabs(t);
            }
            double y = alpha * s;
            double sc = fabs(alpha) * a;
            if (beta != 0.0) {
                double old = (double)C_in[i * ldc + c];
                y += beta * old;
                sc += fabs(beta) * fabs(old);
            }
            C_out[k * N + c] = y;
            if (scale_out) scale_out[k * N + c] = sc;
        }
    }
}

/* Second route for BSR SpMM: loop over the blocks of each listed element row
 * directly, C[I*bs + r, n] = alpha * sum_b sum_c A_b[r][c] * B[bcol_b*bs + c, n]
 * + beta * C.  rows are element rows. */
void oracle_bsr_spmm_direct(int64_t mb, int64_t bs, const int32_t* brow_ptr, const int32_t* bcol,
                            const uint16_t* bval, int64_t N, const uint16_t* B, int64_t ldb,
                            double alpha, double beta, const float* C_in, int64_t ldc,
                            const int64_t* rows, int64_t nrows, double* C_out)
{
    int64_t count = rows ? nrows : mb * bs;
    for (int64_t k = 0; k < count; ++k) {
        int64_t i = rows ? rows[k] : k;
        int64_t I = i / bs, r = i % bs;
        for (int64_t c = 0; c < N; ++c) {
            double s = 0.0;
            for (int64_t b = brow_ptr[I]; b < brow_ptr[I + 1]; ++b)
                for (int64_t q = 0; q < bs; ++q)
                    s += oracle_bf16_to_double(bval[(b * bs + r) * bs + q]) *
                         oracle_bf16_to_double(B[((int64_t)bcol[b] * bs + q) * ldb + c]);
            double y = alpha * s;
            if (beta != 0.0) y += beta * (double)C_in[i * ldc + c];
            C_out[k * N + c] = y;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* CSR -> BSR with square bs x bs blocks ([BCSR] §1: only blocks holding at   */
/* least one entry are stored; block row pointer, block column index and the */
/* dense blocks one after another, each row-major).  mb = ceil(m / bs) block  */
/* rows, kb = ceil(n / bs) block columns; the last block row / column is     */
/* padded.  Blocks of a block row are ordered by block column.  The value at */
/* in-block position (r, c) of block (I, J) is the sum of the CSR entries at */
/* element (I*bs + r, J*bs + c) taken in CSR order and added left to right in */
/* fp32, starting from the first of them; positions without entries hold +0. */
/* ------------------------------------------------------------------------ */

/* Number of stored blocks per block row, as a row pointer brow_ptr[mb + 1];
 * returns nnzb. */
int64_t oracle_csr_to_bsr_count(int64_t m, int64_t n, const int32_t* row_ptr, const int32_t* col, int64_t bs,
                                int32_t* brow_ptr)
{
    int64_t mb = (m + bs - 1) / bs, kb = (n + bs - 1) / bs;
    char* seen = (char*)calloc((size_t)(kb > 0 ? kb : 1), 1);
    int64_t total = 0;
    brow_ptr[0] = 0;
    for (int64_t I = 0; I < mb; ++I) {
        int64_t i_end = (I + 1) * bs < m ? (I + 1) * bs : m;
        int64_t count = 0;
        for (int64_t i = I * bs; i < i_end; ++i)
            for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p)
                if (!seen[col[p] / bs]) {
                    seen[col[p] / bs] = 1;
                    ++count;
                }
        for (int64_t i = I * bs; i < i_end; ++i)
            for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) seen[col[p] / bs] = 0;
        total += count;
        brow_ptr[I + 1] = (int32_t)total;
    }
    free(seen);
    return total;
}

static int cmp_i32(const void* a, const void* b)
{
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/* Block columns and fp32 block values for the row pointer from
 * oracle_csr_to_bsr_count. */
void oracle_csr_to_bsr_fill(int64_t m, const int32_t* row_ptr, const int32_t* col, const float* val, int64_t bs,
                            const int32_t* brow_ptr, int32_t* bcol, float* bval)
{
    int64_t mb = (m + bs - 1) / bs;
    int64_t nnzb = brow_ptr[mb];
    char* filled = (char*)calloc((size_t)(nnzb * bs * bs > 0 ? nnzb * bs * bs : 1), 1);
    for (int64_t q = 0; q < nnzb * bs * bs; ++q) bval[q] = 0.0f;
    for (int64_t I = 0; I < mb; ++I) {
        int64_t i_end = (I + 1) * bs < m ? (I + 1) * bs : m;
        /* the distinct block columns of the block row, ascending */
        int64_t ne = row_ptr[i_end] - row_ptr[I * bs];
        int32_t* js = (int32_t*)malloc((size_t)(ne > 0 ? ne : 1) * sizeof(int32_t));
        for (int64_t p = row_ptr[I * bs]; p < row_ptr[i_end]; ++p) js[p - row_ptr[I * bs]] = col[p] / (int32_t)bs;
        qsort(js, (size_t)ne, sizeof(int32_t), cmp_i32);
        int64_t k = brow_ptr[I];
        for (int64_t e = 0; e < ne; ++e)
            if (e == 0 || js[e] != js[e - 1]) bcol[k++] = js[e];
        free(js);
        /* values, entry by entry in CSR order */
        for (int64_t i = I * bs; i < i_end; ++i) {
            for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) {
                int32_t J = col[p] / (int32_t)bs;
                int64_t lo = brow_ptr[I], hi = brow_ptr[I + 1] - 1;
                while (lo < hi) {
                    int64_t mid = (lo + hi) / 2;
                    if (bcol[mid] < J) lo = mid + 1; else hi = mid;
                }
                int64_t slot = (lo * bs + (i - I * bs)) * bs + col[p] % bs;
                if (!filled[slot]) {
                    bval[slot] = val[p];
                    filled[slot] = 1;
                } else {
                    bval[slot] = bval[slot] + val[p];
                }
            }
        }
    }
    free(filled);
}

/* fp32 -> bf16 bit pattern, round to nearest, ties to even: add 0x7fff plus
 * the lowest kept bit to the 32-bit pattern and keep the upper half (a
 * carry into the exponent is the correct rounding, up to infinity).  NaN
 * keeps its sign and upper payload and is made quiet. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

/* BSR SpMV with fp32 blocks: y_i = alpha * sum over the blocks b of block
 * row i / bs and in-block columns c of A_b[i % bs][c] * x[bcol_b * bs + c]
 * + beta * y_i, for element rows i < m; columns >= n (padding) are skipped.
 * Sums in fp64; scale_i = |alpha| sum |A x| + |beta| |y_i| as in oracle_spmv. */
void oracle_bsr_spmv(int64_t m, int64_t n, int64_t bs, const int32_t* brow_ptr, const int32_t* bcol,
                     const float* bval, const float* x, double alpha, double beta, const float* y_in,
                     double* y_out, double* scale_out)
{
    for (int64_t i = 0; i < m; ++i) {
        int64_t I = i / bs, r = i % bs;
        double s = 0.0, a = 0.0;
        for (int64_t b = brow_ptr[I]; b < brow_ptr[I + 1]; ++b) {
            for (int64_t c = 0; c < bs; ++c) {
                int64_t j = (int64_t)bcol[b] * bs + c;
                if (j >= n) continue;
                double t = (double)bval[(b * bs + r) * bs + c] * (double)x[j];
                s += t;
                a += fabs(t);
            }
        }
        double y = alpha * s, sc = fabs(alpha) * a;
        if (beta != 0.0) {
            y += beta * (double)y_in[i];
            sc += fabs(beta) * fabs((double)y_in[i]);
        }
        y_out[i] = y;
        if (scale_out) scale_out[i] = sc;
    }
}

/* ------------------------------------------------------------------------ */
/* CSR -> WCSR ([ASYNC] §2.2.2: rows grouped into windows of fixed height; for */
/* each window the union of the column indices of its rows, with the values   */
/* of those columns stored densely; padding columns carry index -1).  Window  */
/* w holds rows [w*H, w*H + H); its compressed columns are the distinct column */
/* indices of those rows, ascending, followed by -1 up to a multiple of pad.  */
/* window_ptr[w] is the first compressed column of window w.  Values are      */
/* stored column by column: values[q*H + r] is the element (w*H + r,          */
/* window_col[q]), the CSR entries at that position added in CSR order in    */
/* fp32 starting from the first; 0 where there is none (padding included).   */
/* ------------------------------------------------------------------------ */
int64_t oracle_csr_to_wcsr_count(int64_t m, int64_t n, const int32_t* row_ptr, const int32_t* col, int64_t H,
                                 int64_t pad, int32_t* window_ptr)
{
    int64_t nw = (m + H - 1) / H;
    char* seen = (char*)calloc((size_t)(n > 0 ? n : 1), 1);
    int64_t total = 0;
    window_ptr[0] = 0;
    for (int64_t w = 0; w < nw; ++w) {
        int64_t i_end = (w + 1) * H < m ? (w + 1) * H : m;
        int64_t count = 0;
        for (int64_t i = w * H; i < i_end; ++i)
            for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p)
                if (!seen[col[p]]) {
                    seen[col[p]] = 1;
                    ++count;
                }
        for (int64_t i = w * H; i < i_end; ++i)
            for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) seen[col[p]] = 0;
        total += (count + pad - 1) / pad * pad;
        window_ptr[w + 1] = (int32_t)total;
    }
    free(seen);
    return total;
}

void oracle_csr_to_wcsr_fill(int64_t m, const int32_t* row_ptr, const int32_t* col, const float* val, int64_t H,
                             const int32_t* window_ptr, int32_t* window_col, float* values)
{
    int64_t nw = (m + H - 1) / H;
    int64_t total = window_ptr[nw];
    char* filled = (char*)calloc((size_t)(total * H > 0 ? total * H : 1), 1);
    for (int64_t q = 0; q < total * H; ++q) values[q] = 0.0f;
    for (int64_t w = 0; w < nw; ++w) {
        int64_t i_end = (w + 1) * H < m ? (w + 1) * H : m;
        int64_t ne = row_ptr[i_end] - row_ptr[w * H];
        int32_t* cs = (int32_t*)malloc((size_t)(ne > 0 ? ne : 1) * sizeof(int32_t));
        for (int64_t p = row_ptr[w * H]; p < row_ptr[i_end]; ++p) cs[p - row_ptr[w * H]] = col[p];
        qsort(cs, (size_t)ne, sizeof(int32_t), cmp_i32);
        int64_t q = window_ptr[w];
        for (int64_t e = 0; e < ne; ++e)
            if (e == 0 || cs[e] != cs[e - 1]) window_col[q++] = cs[e];
        int64_t used = q;
        while (q < window_ptr[w + 1]) window_col[q++] = -1;
        free(cs);
        for (int64_t i = w * H; i < i_end; ++i) {
            for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) {
                int64_t lo = window_ptr[w], hi = used - 1;
                while (lo < hi) {
                    int64_t mid = (lo + hi) / 2;
                    if (window_col[mid] < col[p]) lo = mid + 1; else hi = mid;
                }
                int64_t slot = lo * H + (i - w * H);
                if (!filled[slot]) {
                    values[slot] = val[p];
                    filled[slot] = 1;
                } else {
                    values[slot] = values[slot] + val[p];
                }
            }
        }
    }
    free(filled);
}

/* SpMM over the WCSR layout: C[i, c] = alpha * sum over the compressed columns
 * q of window i / H with window_col[q] >= 0 of values[q*H + i % H] *
 * B[window_col[q], c] + beta * C[i, c], for rows i < m; fp64 sums, scale as
 * in oracle_spmm. */
void oracle_wcsr_spmm(int64_t m, int64_t H, const int32_t* window_ptr, const int32_t* window_col,
                      const float* values, int64_t N, const float* B, int64_t ldb, double alpha, double beta,
                      const float* C_in, int64_t ldc, double* C_out, double* scale_out)
{
    for (int64_t i = 0; i < m; ++i) {
        int64_t w = i / H, r = i % H;
        for (int64_t c = 0; c < N; ++c) {
            double s = 0.0, a = 0.0;
            for (int64_t q = window_ptr[w]; q < window_ptr[w + 1]; ++q) {
                if (window_col[q] < 0) continue;
                double t = (double)values[q * H + r] * (double)B[(int64_t)window_col[q] * ldb + c];
                s += t;
                a += fabs(t);
            }
            double y = alpha * s, sc = fabs(alpha) * a;
            if (beta != 0.0) {
                double old = (double)C_in[i * ldc + c];
                y += beta * old;
                sc += fabs(beta) * fabs(old);
            }
            C_out[i * N + c] = y;
            if (scale_out) scale_out[i * N + c] = sc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* WCSR task split ([ASYNC] §4.2: a window whose compressed columns exceed a  */
/* threshold is cut along its columns into pieces of a fixed width, and a     */
/* workgroup is launched per piece; each piece names its window, its first    */
/* compressed column and its width).  A window of c <= T columns is one task  */
/* covering [window_ptr[w], window_ptr[w+1]); a window of c > T columns is    */
/* ceil(c / T) tasks of T columns each, the last one shorter.  Tasks are      */
/* numbered window by window.  The tasks of the split windows take partial    */
/* slots 0, 1, 2, ... in task order; a task of an unsplit window has slot -1.  */
/* tasks[4k .. 4k+3] = {window, first column, end column, slot};              */
/* winfo[2w], winfo[2w+1] = first slot of window w (-1 if not split), tasks. */
/* Returns the number of tasks and stores the number of slots in *nslots;     */
/* with tasks == NULL and winfo == NULL it only counts.                       */
/* ------------------------------------------------------------------------ */
int64_t oracle_wcsr_tasks(int64_t nw, const int32_t* window_ptr, int64_t T, int32_t* tasks, int32_t* winfo,
                          int64_t* nslots)
{
    int64_t k = 0, slot = 0;
    for (int64_t w = 0; w < nw; ++w) {
        int64_t q0 = window_ptr[w], q1 = window_ptr[w + 1];
        int64_t c = q1 - q0;
        int64_t nt = c <= T ? 1 : (c + T - 1) / T;
        if (winfo) {
            winfo[2 * w] = nt > 1 ? (int32_t)slot : -1;
            winfo[2 * w + 1] = (int32_t)nt;
        }
        for (int64_t t = 0; t < nt; ++t, ++k) {
            if (!tasks) continue;
            int64_t b = nt > 1 ? q0 + t * T : q0;
            int64_t e = nt > 1 ? (b + T < q1 ? b + T : q1) : q1;
            tasks[4 * k] = (int32_t)w;
            tasks[4 * k + 1] = (int32_t)b;
            tasks[4 * k + 2] = (int32_t)e;
            tasks[4 * k + 3] = nt > 1 ? (int32_t)(slot + t) : -1;
        }
        if (nt > 1) slot += nt;
    }
    *nslots = slot;
    return k;
}

/* ------------------------------------------------------------------------ */
/* Row-length profile ([GEN] §4 dispatch key: average, p95 and maximum row    */
/* length and the coefficient of variation; [LSMR] §5.3: l_i = row_ptr[i+1] - */
/* row_ptr[i], its mean, variance and tail).  Percentiles use the nearest-    */
/* rank rule: the smallest length L such that at least q percent of the rows */
/* have length <= L.                                                         */
/* out: [0] mean, [1] population variance, [2] cv = sqrt(var)/mean (0 when   */
/* mean == 0), [3] p95, [4] p99, [5] max, [6] number of empty rows.          */
/* ------------------------------------------------------------------------ */
static int cmp_i64(const void* a, const void* b)
{
    int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return (x > y) - (x < y);
}

void oracle_row_profile(int64_t m, const int32_t* row_ptr, double* out)
{
    for (int k = 0; k < 7; ++k) out[k] = 0.0;
    if (m <= 0) return;
    int64_t* len = (int64_t*)malloc((size_t)m * sizeof(int64_t));
    double sum = 0.0;
    int64_t empty = 0;
    for (int64_t i = 0; i < m; ++i) {
        len[i] = (int64_t)row_ptr[i + 1] - row_ptr[i];
        sum += (double)len[i];
        if (len[i] == 0) ++empty;
    }
    double mean = sum / (double)m;
    double var = 0.0;
    for (int64_t i = 0; i < m; ++i) var += ((double)len[i] - mean) * ((double)len[i] - mean);
    var /= (double)m;
    qsort(len, (size_t)m, sizeof(int64_t), cmp_i64);
    /* nearest rank: index ceil(q*m/100) - 1, computed in integers */
    int64_t i95 = (95 * m + 99) / 100 - 1;
    int64_t i99 = (99 * m + 99) / 100 - 1;
    out[0] = mean;
    out[1] = var;
    out[2] = mean > 0.0 ? sqrt(var) / mean : 0.0;
    out[3] = (double)len[i95];
    out[4] = (double)len[i99];
    out[5] = (double)len[m - 1];
    out[6] = (double)empty;
    free(len);
}

/* ------------------------------------------------------------------------ */
/* SELL-C-sigma  ([GEN] §1.4: sort rows by length inside windows of sigma     */
/* rows, cut the sorted order into slices of C rows and pad each slice;      */
/* [FMT] §4: ELL is the one-slice case, slot t of every row read together).  */
/* Outputs: perm[k] = original row at sorted position k; slice_ptr[s] =      */
/* first slot of slice s (nslices + 1 entries); slice_len[k] = length of the */
/* row at sorted position k; col/val in slot order with -1 / 0 padding.      */
/* Returns the total number of slots.  Sizes are queried by calling with    */
/* col == NULL first (then only perm, slice_ptr and slice_len are filled).   */
/* ------------------------------------------------------------------------ */
typedef struct { int64_t len; int64_t row; } len_row;

static int cmp_len_desc(const void* a, const void* b)
{
    const len_row* p = (const len_row*)a;
    const len_row* q = (const len_row*)b;
    if (p->len != q->len) return p->len > q->len ? -1 : 1;
    return (p->row > q->row) - (p->row < q->row);
}

int64_t oracle_sell_build(int64_t m, const int32_t* row_ptr, const int32_t* col, const float* val,
                          int64_t C, int64_t sigma, int32_t* perm, int64_t* slice_ptr,
                          int32_t* slice_len, int32_t* col_out, float* val_out)
{
    len_row* lr = (len_row*)malloc(((size_t)m + 1) * sizeof(len_row));
    for (int64_t i = 0; i < m; ++i) { lr[i].len = (int64_t)row_ptr[i + 1] - row_ptr[i]; lr[i].row = i; }
    for (int64_t w = 0; w < m; w += sigma) {
        int64_t e = w + sigma < m ? w + sigma : m;
        qsort(lr + w, (size_t)(e - w), sizeof(len_row), cmp_len_desc);
    }
    for (int64_t k = 0; k < m; ++k) { perm[k] = (int32_t)lr[k].row; slice_len[k] = (int32_t)lr[k].len; }
    int64_t nslices = (m + C - 1) / C;
    int64_t slots = 0;
    for (int64_t s = 0; s < nslices; ++s) {
        int64_t width = 0;
        for (int64_t j = 0; j < C && s * C + j < m; ++j)
            if (lr[s * C + j].len > width) width = lr[s * C + j].len;
        slice_ptr[s] = slots;
        if (col_out) {
            for (int64_t t = 0; t < width; ++t) {
                for (int64_t j = 0; j < C; ++j) {
                    int64_t k = s * C + j;
                    int64_t q = slots + t * C + j;
                    if (k < m && t < lr[k].len) {
                        int64_t p = row_ptr[lr[k].row] + t;
                        col_out[q] = col[p];
                        val_out[q] = val[p];
                    } else {
                        col_out[q] = -1;
                        val_out[q] = 0.0f;
                    }
                }
            }
        }
        slots += width * C;
    }
    slice_ptr[nslices] = slots;
    free(lr);
    return slots;
}

/* SpMV through a SELL-C-sigma layout: every lane of a slice walks its row's
 * slots t = 0 .. slice_len-1 (padding is skipped by the length, never
 * multiplied).  y_out is indexed by original row. */
void oracle_sell_spmv(int64_t m, int64_t C, const int32_t* perm, const int64_t* slice_ptr,
                      const int32_t* slice_len, const int32_t* col, const float* val,
                      const float* x, double alpha, double* y_out)
{
    int64_t nslices = (m + C - 1) / C;
    for (int64_t s = 0; s < nslices; ++s) {
        for (int64_t j = 0; j < C; ++j) {
            int64_t k = s * C + j;
            if (k >= m) break;
            double acc = 0.0;
            for (int64_t t = 0; t < slice_len[k]; ++t) {
                int64_t q = slice_ptr[s] + t * C + j;
                acc += (double)val[q] * (double)x[col[q]];
            }
            y_out[perm[k]] = alpha * acc;
        }
    }
}
