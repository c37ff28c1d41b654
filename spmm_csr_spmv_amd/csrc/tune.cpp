// Dispatch key, tuning cache and micro-autotune of the SpMV path.
//
// 「通用稀疏矩阵乘法CUDA算子实现」 §4: the first time a matrix is seen, a light
// profile gives a stable dispatch key (format, dtype, index width, M, K, N,
// average / p95 / maximum row length, row-length variation, ...); a rule table
// picks the kernel, and a small autotune times 2-4 candidates with events,
// caches the fastest configuration and never benchmarks on every call; for a
// matrix that changes, a version number invalidates what was cached.
//
// Here the candidates are plan option sets (row bins, SELL, column-panel
// stream).  The key quantises the row-length statistics (a quarter octave for
// lengths, 1/8 for the coefficient of variation) so that a re-loaded or
// re-valued matrix with the same shape and length profile hits the entry,
// while M, K, nnz, N and the caller's version number must match exactly.  The
// cache is process-wide and guarded by a mutex; sp_plan_create without
// options consults it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "internal.h"
#include "spmm_csr_spmv.h"

namespace {

auto key_fields(const sp_dispatch_key& k) {
    return std::make_tuple(k.format, k.dtype, k.index_bits, k.transposed, k.rows, k.cols, k.nnz, k.N, k.arch,
                           k.avg_len_q, k.p95_len_q, k.max_len_q, k.cv_q, k.version);
}

struct KeyLess {
    bool operator()(const sp_dispatch_key& a, const sp_dispatch_key& b) const { return key_fields(a) < key_fields(b); }
};

std::mutex& cache_mutex() {
    static std::mutex mu;
    return mu;
}

std::map<sp_dispatch_key, sp_plan_options, KeyLess>& cache() {
    static std::map<sp_dispatch_key, sp_plan_options, KeyLess> c;
    return c;
}

int32_t length_bucket(double v) { return (int32_t)std::floor(4.0 * std::log2(1.0 + std::max(0.0, v))); }

}  // namespace

namespace spx {

void make_dispatch_key(const sp_profile& p, int32_t transposed, int32_t N, uint64_t version, sp_dispatch_key* key) {
    std::memset(key, 0, sizeof *key);
    key->format = 0;       // CSR
    key->dtype = 0;        // fp32 values
    key->index_bits = 32;
    key->transposed = transposed;
    key->rows = p.rows;
    key->cols = p.cols;
    key->nnz = p.nnz;
    key->N = N;
    key->arch = 950;       // gfx950
    key->avg_len_q = length_bucket(p.mean);
    key->p95_len_q = length_bucket((double)p.p95);
    key->max_len_q = length_bucket((double)p.max_len);
    key->cv_q = (int32_t)std::min(4095.0, std::floor(8.0 * p.cv));
    key->version = version;
}

bool tune_cache_find(const sp_dispatch_key& key, sp_plan_options* out) {
    std::lock_guard<std::mutex> lock(cache_mutex());
    auto it = cache().find(key);
    if (it == cache().end()) return false;
    *out = it->second;
    return true;
}

}  // namespace spx

extern "C" {

int sp_plan_dispatch_key(const sp_plan* plan, int32_t transposed, int32_t N, uint64_t version, sp_dispatch_key* key) {
    if (!plan || !key) return SP_ERR_NULL;
    if (N < 1 || (transposed != 0 && transposed != 1)) return SP_ERR_SIZE;
    sp_profile p;
    const int rc = sp_plan_profile(plan, transposed, &p);
    if (rc != SP_OK) return rc;
    spx::make_dispatch_key(p, transposed, N, version, key);
    return SP_OK;
}

int sp_tune_cache_store(const sp_dispatch_key* key, const sp_plan_options* opt) {
    if (!key || !opt) return SP_ERR_NULL;
    if (spx::check_plan_options(*opt) != SP_OK) return SP_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(cache_mutex());
    cache()[*key] = *opt;
    return SP_OK;
}

int sp_tune_cache_lookup(const sp_dispatch_key* key, sp_plan_options* opt, int32_t* found) {
    if (!key || !opt || !found) return SP_ERR_NULL;
    *found = spx::tune_cache_find(*key, opt) ? 1 : 0;
    return SP_OK;
}

int sp_tune_cache_clear(void) {
    std::lock_guard<std::mutex> lock(cache_mutex());
    cache().clear();
    return SP_OK;
}

int sp_tune_cache_size(int64_t* entries) {
    if (!entries) return SP_ERR_NULL;
    std::lock_guard<std::mutex> lock(cache_mutex());
    *entries = (int64_t)cache().size();
    return SP_OK;
}

int sp_autotune_workspace_size(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                               const float* val, const sp_plan_options* cand, int32_t ncand, size_t* bytes,
                               void* stream) {
    if (!bytes || (ncand > 0 && !cand)) return SP_ERR_NULL;
    if (ncand < 1 || ncand > 16) return SP_ERR_SIZE;
    size_t most = 0;
    for (int32_t i = 0; i < ncand; ++i) {
        sp_plan* p = nullptr;
        int rc = sp_plan_create(&p, m, n, nnz, row_ptr, col_idx, val, nullptr, nullptr, nullptr, &cand[i], stream);
        if (rc != SP_OK) return rc;
        size_t b = 0;
        rc = sp_plan_workspace_size(p, 1, &b);
        sp_plan_destroy(p);
        if (rc != SP_OK) return rc;
        most = std::max(most, b);
    }
    *bytes = most;
    return SP_OK;
}

int sp_autotune_spmv(int64_t m, int64_t n, int64_t nnz, const int32_t* row_ptr, const int32_t* col_idx,
                     const float* val, const sp_plan_options* cand, int32_t ncand, const float* x, float* y,
                     int32_t reps, uint64_t version, void* work, size_t work_bytes, int32_t* best, float* ms,
                     void* stream) {
    if (!best || !ms || (ncand > 0 && !cand)) return SP_ERR_NULL;
    if (ncand < 1 || ncand > 16 || reps < 1) return SP_ERR_SIZE;
    hipStream_t s = (hipStream_t)stream;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess) return SP_ERR_HIP;
    if (hipEventCreate(&e1) != hipSuccess) {
        hipEventDestroy(e0);
        return SP_ERR_HIP;
    }
    int rc = SP_OK;
    sp_dispatch_key key{};
    int32_t winner = -1;
    for (int32_t i = 0; i < ncand && rc == SP_OK; ++i) {
        sp_plan* p = nullptr;
        rc = sp_plan_create(&p, m, n, nnz, row_ptr, col_idx, val, nullptr, nullptr, nullptr, &cand[i], stream);
        if (rc != SP_OK) break;
        size_t need = 0;
        rc = sp_plan_workspace_size(p, 1, &need);
        if (rc == SP_OK && (!work || work_bytes < need)) rc = SP_ERR_WORKSPACE;
        if (rc == SP_OK) rc = sp_plan_bind(p, work, work_bytes, 1, stream);
        if (rc == SP_OK && i == 0) rc = sp_plan_dispatch_key(p, 0, 1, version, &key);
        if (rc == SP_OK) rc = spmv(p, 1.0f, x, 0.0f, y, stream);  // warm-up
        if (rc == SP_OK) {
            if (hipEventRecord(e0, s) != hipSuccess) rc = SP_ERR_HIP;
            for (int32_t r = 0; r < reps && rc == SP_OK; ++r) rc = spmv(p, 1.0f, x, 0.0f, y, stream);
            float t = 0.0f;
            if (rc == SP_OK && (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                                hipEventElapsedTime(&t, e0, e1) != hipSuccess))
                rc = SP_ERR_HIP;
            if (rc == SP_OK) {
                ms[i] = t / (float)reps;
                if (winner < 0 || ms[i] < ms[winner]) winner = i;
            }
        }
        sp_plan_destroy(p);
    }
    hipEventDestroy(e0);
    hipEventDestroy(e1);
    if (rc != SP_OK) return rc;
    *best = winner;
    {
        std::lock_guard<std::mutex> lock(cache_mutex());
        cache()[key] = cand[winner];
    }
    return SP_OK;
}

}  // extern "C"
