/* Driver for the sanitizer run of the CPU oracle (test infrastructure).
 *
 * Built by tests/test_oracle_sanitize.py together with oracle/oracle.c under
 * AddressSanitizer and UndefinedBehaviorSanitizer.  It calls every oracle
 * entry point the way the Python wrappers do, on seeded small matrices with
 * empty rows and duplicate entries, and cross-checks the routes against one
 * another (so a sanitizer report, a wrong size or an inconsistent result all
 * end the run with a non-zero status).  The arithmetic of the checks is plain
 * dense accumulation written here, not the oracle's. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_coo_to_csr(int64_t m, int64_t n, int64_t nnz, const int32_t* row, const int32_t* col, const float* val,
                      int32_t* row_ptr, int32_t* col_out, float* val_out);
int oracle_csr_to_csc(int64_t m, int64_t n, const int32_t* row_ptr, const int32_t* col, const float* val,
                      int32_t* col_ptr, int32_t* row_idx, float* val_out);
void oracle_spmv(int64_t m, const int32_t* row_ptr, const int32_t* col, const float* val, const float* x, double alpha,
                 double beta, const float* y_in, const int64_t* rows, int64_t nrows, double* y_out, double* scale_out);
void oracle_spmv_t_scatter(int64_t m, int64_t n, const int32_t* row_ptr, const int32_t* col, const float* val,
                           const float* u, double alpha, double beta, const float* z_in, double* z_out,
                           double* scale_out);
void oracle_spmm(int64_t m, const int32_t* row_ptr, const int32_t* col, const float* val, int64_t N, const float* B,
                 int64_t ldb, double alpha, double beta, const float* C_in, int64_t ldc, const int64_t* rows,
                 int64_t nrows, double* C_out, double* scale_out);
double oracle_bf16_to_double(uint16_t h);
int oracle_bsr_to_csr(int64_t mb, int64_t bs, const int32_t* brow_ptr, const int32_t* bcol, const uint16_t* bval,
                      int32_t* row_ptr, int32_t* col, double* val);
void oracle_spmm_bf16(int64_t m, const int32_t* row_ptr, const int32_t* col, const double* val, int64_t N,
                      const uint16_t* B, int64_t ldb, double alpha, double beta, const float* C_in, int64_t ldc,
                      const int64_t* rows, int64_t nrows, double* C_out, double* scale_out);
void oracle_bsr_spmm_direct(int64_t mb, int64_t bs, const int32_t* brow_ptr, const int32_t* bcol,
                            const uint16_t* bval, int64_t N, const uint16_t* B, int64_t ldb, double alpha, double beta,
                            const float* C_in, int64_t ldc, const int64_t* rows, int64_t nrows, double* C_out);
int64_t oracle_csr_to_bsr_count(int64_t m, int64_t n, const int32_t* row_ptr, const int32_t* col, int64_t bs,
                                int32_t* brow_ptr);
void oracle_csr_to_bsr_fill(int64_t m, const int32_t* row_ptr, const int32_t* col, const float* val, int64_t bs,
                            const int32_t* brow_ptr, int32_t* bcol, float* bval);
uint16_t oracle_f32_to_bf16(float f);
void oracle_bsr_spmv(int64_t m, int64_t n, int64_t bs, const int32_t* brow_ptr, const int32_t* bcol,
                     const float* bval, const float* x, double alpha, double beta, const float* y_in, double* y_out,
                     double* scale_out);
int64_t oracle_csr_to_wcsr_count(int64_t m, int64_t n, const int32_t* row_ptr, const int32_t* col, int64_t H,
                                 int64_t pad, int32_t* window_ptr);
void oracle_csr_to_wcsr_fill(int64_t m, const int32_t* row_ptr, const int32_t* col, const float* val, int64_t H,
                             const int32_t* window_ptr, int32_t* window_col, float* values);
void oracle_wcsr_spmm(int64_t m, int64_t H, const int32_t* window_ptr, const int32_t* window_col,
                      const float* values, int64_t N, const float* B, int64_t ldb, double alpha, double beta,
                      const float* C_in, int64_t ldc, double* C_out, double* scale_out);
void oracle_row_profile(int64_t m, const int32_t* row_ptr, double* out);
int64_t oracle_sell_build(int64_t m, const int32_t* row_ptr, const int32_t* col, const float* val, int64_t C,
                          int64_t sigma, int32_t* perm, int64_t* slice_ptr, int32_t* slice_len, int32_t* col_out,
                          float* val_out);
void oracle_sell_spmv(int64_t m, int64_t C, const int32_t* perm, const int64_t* slice_ptr, const int32_t* slice_len,
                      const int32_t* col, const float* val, const float* x, double alpha, double* y_out);

static uint64_t state;
static uint32_t next_u32(void) {
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(state >> 33);
}
static float uniform(void) { return (float)next_u32() / 2147483648.0f - 1.0f; }

static int failures;
static void check(int ok, const char* what, int seed) {
    if (!ok) {
        fprintf(stderr, "seed %d: %s\n", seed, what);
        ++failures;
    }
}
static int close_to(double a, double b) { return fabs(a - b) <= 1e-9 * (1.0 + fabs(a) + fabs(b)); }

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) exit(2);
    return p;
}

static void run(int seed) {
    state = 0x9e3779b97f4a7c15ull ^ (uint64_t)seed;
    const int64_t m = 1 + next_u32() % 17, n = 1 + next_u32() % 19;
    const int64_t nnz = next_u32() % (m * n + 3);
    int32_t* row = xmalloc(nnz * 4);
    int32_t* col = xmalloc(nnz * 4);
    float* val = xmalloc(nnz * 4);
    for (int64_t i = 0; i < nnz; ++i) {  /* duplicates arise naturally */
        row[i] = (int32_t)(next_u32() % m);
        col[i] = (int32_t)(next_u32() % n);
        val[i] = uniform();
    }
    /* dense reference, summed here */
    double* dense = calloc((size_t)(m * n), sizeof(double));
    for (int64_t i = 0; i < nnz; ++i) dense[row[i] * n + col[i]] += val[i];

    int32_t* rp = xmalloc((m + 1) * 4);
    int32_t* ci = xmalloc(nnz * 4);
    float* cv = xmalloc(nnz * 4);
    check(oracle_coo_to_csr(m, n, nnz, row, col, val, rp, ci, cv) == 0, "coo_to_csr", seed);
    check(rp[0] == 0 && rp[m] == nnz, "row_ptr ends", seed);
    if (nnz > 0) {  /* an index out of range is rejected */
        const int32_t keep = col[0];
        col[0] = (int32_t)n;
        check(oracle_coo_to_csr(m, n, nnz, row, col, val, rp, ci, cv) == 3, "index error", seed);
        col[0] = keep;
        check(oracle_coo_to_csr(m, n, nnz, row, col, val, rp, ci, cv) == 0, "coo_to_csr again", seed);
    }
    /* CSC, and the CSC of the CSC is the CSR */
    int32_t* cp = xmalloc((n + 1) * 4);
    int32_t* ri = xmalloc(nnz * 4);
    float* tv = xmalloc(nnz * 4);
    check(oracle_csr_to_csc(m, n, rp, ci, cv, cp, ri, tv) == 0, "csr_to_csc", seed);
    int32_t* rp2 = xmalloc((m + 1) * 4);
    int32_t* ci2 = xmalloc(nnz * 4);
    float* cv2 = xmalloc(nnz * 4);
    check(oracle_csr_to_csc(n, m, cp, ri, tv, rp2, ci2, cv2) == 0, "csc_to_csr", seed);
    check(memcmp(rp, rp2, (m + 1) * 4) == 0 && memcmp(ci, ci2, nnz * 4) == 0 && memcmp(cv, cv2, nnz * 4) == 0,
          "double transpose", seed);

    /* products against the dense matrix */
    float* x = xmalloc(n * 4);
    float* u = xmalloc(m * 4);
    float* y0 = xmalloc(m * 4);
    float* z0 = xmalloc(n * 4);
    for (int64_t j = 0; j < n; ++j) x[j] = uniform(), z0[j] = uniform();
    for (int64_t i = 0; i < m; ++i) u[i] = uniform(), y0[i] = uniform();
    double* y = xmalloc(m * 8);
    double* sc = xmalloc(m * 8);
    oracle_spmv(m, rp, ci, cv, x, 1.5, -0.5, y0, NULL, 0, y, sc);
    for (int64_t i = 0; i < m; ++i) {
        double r = 0.0;
        for (int64_t j = 0; j < n; ++j) r += dense[i * n + j] * x[j];
        check(fabs(1.5 * r - 0.5 * y0[i] - y[i]) <= 1e-5 * (sc[i] + 1e-30) + 1e-12, "spmv", seed);
    }
    int64_t rows[3] = {0, m - 1, m / 2};
    double ys[3], ss[3];
    oracle_spmv(m, rp, ci, cv, x, 1.5, -0.5, y0, rows, 3, ys, ss);
    for (int k = 0; k < 3; ++k) check(close_to(ys[k], y[rows[k]]), "spmv rows", seed);
    double* z = xmalloc(n * 8);
    double* zs = xmalloc(n * 8);
    double* z2 = xmalloc(n * 8);
    double* zs2 = xmalloc(n * 8);
    oracle_spmv_t_scatter(m, n, rp, ci, cv, u, 2.0, 0.25, z0, z, zs);
    oracle_spmv(n, cp, ri, tv, u, 2.0, 0.25, z0, NULL, 0, z2, zs2);
    for (int64_t j = 0; j < n; ++j) check(fabs(z[j] - z2[j]) <= 1e-9 * (zs2[j] + 1.0), "spmv_t", seed);

    const int64_t N = 3;
    float* B = xmalloc(n * N * 4);
    float* C0 = xmalloc(m * N * 4);
    for (int64_t i = 0; i < n * N; ++i) B[i] = uniform();
    for (int64_t i = 0; i < m * N; ++i) C0[i] = uniform();
    double* Cd = xmalloc(m * N * 8);
    double* Cs = xmalloc(m * N * 8);
    oracle_spmm(m, rp, ci, cv, N, B, N, 1.0, 0.5, C0, N, NULL, 0, Cd, Cs);
    for (int64_t i = 0; i < m; ++i)
        for (int64_t c = 0; c < N; ++c) {
            double r = 0.0;
            for (int64_t j = 0; j < n; ++j) r += dense[i * n + j] * B[j * N + c];
            check(fabs(r + 0.5 * C0[i * N + c] - Cd[i * N + c]) <= 1e-5 * (Cs[i * N + c] + 1e-30) + 1e-12, "spmm",
                  seed);
        }

    /* CSR -> BSR (bs 3), BSR SpMV; bf16 blocks -> CSR and both bf16 SpMM routes */
    const int64_t bs = 3, mb = (m + bs - 1) / bs;
    int32_t* brp = xmalloc((mb + 1) * 4);
    const int64_t nnzb = oracle_csr_to_bsr_count(m, n, rp, ci, bs, brp);
    int32_t* bcol = xmalloc(nnzb * 4);
    float* bval = xmalloc(nnzb * bs * bs * 4);
    oracle_csr_to_bsr_fill(m, rp, ci, cv, bs, brp, bcol, bval);
    double* yb = xmalloc(m * 8);
    double* sb = xmalloc(m * 8);
    oracle_bsr_spmv(m, n, bs, brp, bcol, bval, x, 1.5, -0.5, y0, yb, sb);
    for (int64_t i = 0; i < m; ++i) check(fabs(yb[i] - y[i]) <= 1e-5 * (sb[i] + 1e-30) + 1e-12, "bsr_spmv", seed);
    uint16_t* hb = xmalloc(nnzb * bs * bs * 2);
    for (int64_t i = 0; i < nnzb * bs * bs; ++i) {
        hb[i] = oracle_f32_to_bf16(bval[i]);
        check(fabs(oracle_bf16_to_double(hb[i]) - bval[i]) <= fabs(bval[i]) / 256.0, "bf16 rounding", seed);
    }
    const int64_t kbn = ((n + bs - 1) / bs) * bs;
    uint16_t* Bh = xmalloc(kbn * N * 2);
    for (int64_t i = 0; i < kbn * N; ++i) Bh[i] = oracle_f32_to_bf16(uniform());
    int32_t* erp = xmalloc((mb * bs + 1) * 4);
    int32_t* eci = xmalloc(nnzb * bs * bs * 4);
    double* ecv = xmalloc(nnzb * bs * bs * 8);
    check(oracle_bsr_to_csr(mb, bs, brp, bcol, hb, erp, eci, ecv) == 0, "bsr_to_csr", seed);
    double* C1 = xmalloc(mb * bs * N * 8);
    double* C1s = xmalloc(mb * bs * N * 8);
    double* C2 = xmalloc(mb * bs * N * 8);
    oracle_spmm_bf16(mb * bs, erp, eci, ecv, N, Bh, N, 1.0, 0.0, NULL, N, NULL, 0, C1, C1s);
    oracle_bsr_spmm_direct(mb, bs, brp, bcol, hb, N, Bh, N, 1.0, 0.0, NULL, N, NULL, 0, C2);
    for (int64_t i = 0; i < mb * bs * N; ++i) check(close_to(C1[i], C2[i]), "bsr spmm routes", seed);

    /* windowed rows (H 4, pad 2) against the CSR SpMM */
    const int64_t H = 4, nw = (m + H - 1) / H;
    int32_t* wp = xmalloc((nw + 1) * 4);
    const int64_t total = oracle_csr_to_wcsr_count(m, n, rp, ci, H, 2, wp);
    int32_t* wc = xmalloc(total * 4);
    float* wv = xmalloc(total * H * 4);
    oracle_csr_to_wcsr_fill(m, rp, ci, cv, H, wp, wc, wv);
    double* Cw = xmalloc(m * N * 8);
    double* Cws = xmalloc(m * N * 8);
    oracle_wcsr_spmm(m, H, wp, wc, wv, N, B, N, 1.0, 0.5, C0, N, Cw, Cws);
    for (int64_t i = 0; i < m * N; ++i) check(fabs(Cw[i] - Cd[i]) <= 1e-5 * (Cws[i] + 1e-30) + 1e-12, "wcsr", seed);

    /* profile and SELL */
    double prof[7];
    oracle_row_profile(m, rp, prof);
    check(fabs(prof[0] - (double)nnz / (double)m) < 1e-12, "profile mean", seed);
    const int64_t Cs_ = 4, ns = (m + Cs_ - 1) / Cs_;
    int32_t* perm = xmalloc(m * 4);
    int64_t* sp = xmalloc((ns + 1) * 8);
    int32_t* sl = xmalloc(m * 4);
    const int64_t slots = oracle_sell_build(m, rp, ci, cv, Cs_, 8, perm, sp, sl, NULL, NULL);
    int32_t* scol = xmalloc(slots * 4);
    float* sval = xmalloc(slots * 4);
    oracle_sell_build(m, rp, ci, cv, Cs_, 8, perm, sp, sl, scol, sval);
    double* ysell = xmalloc(m * 8);
    double* yplain = xmalloc(m * 8);
    double* splain = xmalloc(m * 8);
    oracle_sell_spmv(m, Cs_, perm, sp, sl, scol, sval, x, 1.0, ysell);
    oracle_spmv(m, rp, ci, cv, x, 1.0, 0.0, NULL, NULL, 0, yplain, splain);
    for (int64_t i = 0; i < m; ++i) check(fabs(ysell[i] - yplain[i]) <= 1e-12 * (splain[i] + 1.0), "sell", seed);

    void* all[] = {row, col, val, dense, rp, ci, cv, cp, ri, tv, rp2, ci2, cv2, x, u, y0, z0, y, sc, z, zs, z2, zs2,
                   B, C0, Cd, Cs, brp, bcol, bval, yb, sb, hb, Bh, erp, eci, ecv, C1, C1s, C2, wp, wc, wv, Cw, Cws,
                   perm, sp, sl, scol, sval, ysell, yplain, splain};
    for (size_t k = 0; k < sizeof all / sizeof all[0]; ++k) free(all[k]);
}

int main(int argc, char** argv) {
    const int count = argc > 1 ? atoi(argv[1]) : 200;
    for (int s = 0; s < count; ++s) run(s);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("ok %d cases\n", count);
    return 0;
}
