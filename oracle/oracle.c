/*
 * CPU oracle for row-wise top-k selection.  TEST INFRASTRUCTURE ONLY: the
 * tests, the smoke check and the benchmark's CPU-baseline leg are the only
 * callers.  It shares no code, header or constant with the GPU library.
 *
 * What it computes is the plain definition of the operator the pages describe
 * (CSDN page "DeepSeek 一次开源三个仓库", section 三 算子层: per row, return the
 * k largest entries, values and indices, k <= 4096; the usage example there
 * is a topk(x, k) call with a sorted-index flag and an index-type option).  The pages' blocked scan / threshold / compaction algorithm
 * only prunes elements that cannot be among the k largest, so it reaches this
 * same result; the oracle therefore does not follow that algorithm -- it sorts.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - Order.  Element i precedes element j (i is "larger") iff
 *       v_i > v_j numerically, or
 *       v_i == v_j == 0 with v_i = +0 and v_j = -0 (IEEE-754 totalOrder), or
 *       v_i and v_j are the same value and i < j (lower index wins a tie).
 *     +inf ranks first and -inf last, like any other value.
 *   - The selected set of a row is the k elements of rank < k.
 *   - Output order (the `sorted_index` argument): 1 writes the selected
 *     indices in ascending order (the aiutil project card, 关键技术亮点 item
 *     2, names sorting by index); 2 writes them by value, in the order above
 *     (largest first; the same page names sorting by value as the other
 *     option); 0 leaves the order free, and the oracle then also writes the
 *     order above (any order is correct; this one is just convenient).
 *   - Values are exact bit copies of the input elements at the chosen indices.
 *   - NaN: any NaN of either sign in columns [0, n) of any row makes the call
 *     return ORACLE_NAN (the pages say NaN checking is always on; see the
 *     zh-TW page "深入 DeepSeek V4.1 全新開放推論工具包", section DeepSelect).
 *     Padding columns [n, row_stride) are never looked at.
 *
 *   - Per-row valid lengths (oracle_topk_lengths): row r holds len_r valid
 *     columns; columns [len_r, n) act as -inf, are never read and never
 *     NaN-checked, and their values are written as -inf (the lengths stand
 *     in for -inf tails: the C4 decode workload's rows are valid prefixes
 *     followed by -inf).  A length outside [0, n] is clamped to it.
 *
 * Values are widened exactly to double (bf16 -> binary32 by a 16-bit shift,
 * then binary32 -> binary64), so every comparison is exact.
 *
 * Parity pins: brute-force rank counting on tiny rows, closed forms
 * (ascending, constant, k = n, -inf tails, quantised ascending levels), a
 * lexsort cross-check and an O(n) completeness invariant; see tests/.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_BF16 = 0, ORACLE_F32 = 1 };
enum { ORACLE_OK = 0, ORACLE_BAD_ARG = 1, ORACLE_NAN = 4, ORACLE_NOMEM = 6 };

typedef struct {
    double v;    /* exact widening of the element */
    int64_t i;   /* column index */
} item;

/* The element at column `col` of a row, widened exactly. */
static double widen(const void* row, int dtype, int64_t col) {
    if (dtype == ORACLE_BF16) {
        uint16_t b = ((const uint16_t*)row)[col];
        uint32_t u = (uint32_t)b << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    } else {
        float f;
        memcpy(&f, (const char*)row + 4 * col, sizeof f);
        return (double)f;
    }
}

/* qsort comparator: negative when *a precedes *b in the order above. */
static int by_rank(const void* pa, const void* pb) {
    const item* a = (const item*)pa;
    const item* b = (const item*)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    if (a->v == 0.0) { /* both zero: +0 before -0 */
        int sa = signbit(a->v) != 0, sb = signbit(b->v) != 0;
        if (sa != sb) return sa ? 1 : -1;
    }
    if (a->i < b->i) return -1;
    if (a->i > b->i) return 1;
    return 0;
}

static int by_index(const void* pa, const void* pb) {
    const item* a = (const item*)pa;
    const item* b = (const item*)pb;
    return (a->i > b->i) - (a->i < b->i);
}

/* One row with `len` valid columns (the rest act as -inf): returns
   ORACLE_OK, ORACLE_NAN or ORACLE_NOMEM. */
static int one_row(const void* row, int dtype, int64_t n, int64_t len, int32_t k, int sorted_index,
                   int return_value, int32_t* out_idx, void* out_val) {
    item* it = (item*)malloc((size_t)n * sizeof(item));
    if (!it) return ORACLE_NOMEM;
    for (int64_t c = 0; c < n; ++c) {
        it[c].v = c < len ? widen(row, dtype, c) : -INFINITY;
        it[c].i = c;
        if (isnan(it[c].v)) {
            free(it);
            return ORACLE_NAN;
        }
    }
    qsort(it, (size_t)n, sizeof(item), by_rank);
    if (sorted_index == 1) qsort(it, (size_t)k, sizeof(item), by_index);
    const size_t es = dtype == ORACLE_BF16 ? 2 : 4;
    const uint16_t ninf16 = 0xFF80;
    const uint32_t ninf32 = 0xFF800000u;
    for (int32_t j = 0; j < k; ++j) {
        out_idx[j] = (int32_t)it[j].i;
        if (return_value) {
            const void* src = it[j].i < len ? (const void*)((const char*)row + es * it[j].i)
                              : dtype == ORACLE_BF16 ? (const void*)&ninf16 : (const void*)&ninf32;
            memcpy((char*)out_val + es * j, src, es);
        }
    }
    free(it);
    return ORACLE_OK;
}

/*
 * Top-k of every row of `in` ([batch][row_stride] elements, bf16 bits or
 * fp32).  out_idx is [batch][k] int32; out_val (same dtype as in) is written
 * when return_value is set.  nthreads <= 0 means "all available".
 * Returns ORACLE_OK, ORACLE_BAD_ARG, ORACLE_NAN (some row holds a NaN in
 * [0, n); outputs are then incomplete) or ORACLE_NOMEM.
 */
int oracle_topk_lengths(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride,
                        int32_t k, const int32_t* lengths, int sorted_index, int return_value,
                        int32_t* out_idx, void* out_val, int nthreads);

int oracle_topk(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride,
                int32_t k, int sorted_index, int return_value, int32_t* out_idx,
                void* out_val, int nthreads) {
    return oracle_topk_lengths(in, dtype, batch, n, row_stride, k, NULL, sorted_index, return_value,
                               out_idx, out_val, nthreads);
}

/*
 * As oracle_topk, with row r's valid columns [0, lengths[r]) (host array of
 * batch entries, each clamped to [0, n]; NULL: all n valid).
 */
int oracle_topk_lengths(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride,
                        int32_t k, const int32_t* lengths, int sorted_index, int return_value,
                        int32_t* out_idx, void* out_val, int nthreads) {
    if ((dtype != ORACLE_BF16 && dtype != ORACLE_F32) || sorted_index < 0 || sorted_index > 2 || batch < 0 || n < 1 || k < 1 ||
        k > n || row_stride < n || !in || !out_idx || (return_value && !out_val))
        return ORACLE_BAD_ARG;
    const size_t es = dtype == ORACLE_BF16 ? 2 : 4;
    int status = ORACLE_OK;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(max : status)
#endif
    for (int64_t r = 0; r < batch; ++r) {
        const void* row = (const char*)in + es * (size_t)(r * row_stride);
        int64_t len = lengths ? (int64_t)lengths[r] : n;
        len = len < 0 ? 0 : len > n ? n : len;
        int s = one_row(row, dtype, n, len, k, sorted_index, return_value, out_idx + r * (int64_t)k,
                        return_value ? (char*)out_val + es * (size_t)(r * (int64_t)k) : NULL);
        if (s > status) status = s;
    }
    (void)nthreads;
    return status;
}

/*
 * Sampling over the top-k candidates -- the step after the selection on the
 * sampler path.  The pages name temperature and top-p as the generation
 * parameters (CSDN page, section 二 接入层; zh-TW page, the deepseek-recipe
 * section) without a formula; this is the textbook reading:
 *   c_1 .. c_k   the row's top-k in value order (the order above);
 *   w_j          exp((x_{c_j} - x_{c_1}) / T), with w_j = 1 where
 *                x_{c_j} == x_{c_1} (equal values, +inf tops) and w_j = 0
 *                where x_{c_j} = -inf below a larger top;
 *   W_j          w_1 + ... + w_j;
 *   m            the smallest j with W_j >= top_p * W_k (top-p nucleus;
 *                at least one candidate; m = k when top_p >= 1);
 *   token        c_j for the smallest j with W_j > u * W_m, u in [0, 1)
 *                the caller's uniform draw (inverse CDF).
 * T <= 0 (or NaN) means greedy: token = c_1.  u is clamped to [0, 1).
 * Computed in double.  Returns as oracle_topk; out_token[r] per row.
 */
int oracle_sample(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k,
                  const float* temperature, const float* top_p, const float* uniform, int32_t* out_token) {
    if (!temperature || !top_p || !uniform || !out_token) return ORACLE_BAD_ARG;
    if (batch <= 0) return batch < 0 ? ORACLE_BAD_ARG : ORACLE_OK;
    int32_t* idx = (int32_t*)malloc((size_t)(batch * (int64_t)k) * sizeof(int32_t));
    if (!idx) return ORACLE_NOMEM;
    int st = oracle_topk(in, dtype, batch, n, row_stride, k, 2, 0, idx, NULL, 1);
    if (st != ORACLE_OK) {
        free(idx);
        return st;
    }
    const size_t es = dtype == ORACLE_BF16 ? 2 : 4;
    double* W = (double*)malloc((size_t)k * sizeof(double));
    if (!W) {
        free(idx);
        return ORACLE_NOMEM;
    }
    for (int64_t r = 0; r < batch; ++r) {
        const void* row = (const char*)in + es * (size_t)(r * row_stride);
        const int32_t* c = idx + r * (int64_t)k;
        const double T = temperature[r];
        if (!(T > 0.0)) {
            out_token[r] = c[0];
            continue;
        }
        const double x1 = widen(row, dtype, c[0]);
        double acc = 0.0;
        for (int32_t j = 0; j < k; ++j) {
            const double x = widen(row, dtype, c[j]);
            const double w = x == x1 ? 1.0 : isinf(x) && x < 0 ? 0.0 : exp((x - x1) / T);
            acc += w;
            W[j] = acc;
        }
        const double p = top_p[r];
        int32_t m = k;  /* 1-based nucleus size */
        for (int32_t j = 0; j < k; ++j)
            if (W[j] >= p * W[k - 1]) {
                m = j + 1;
                break;
            }
        double u = uniform[r];
        if (!(u >= 0.0)) u = 0.0;
        if (u >= 1.0) u = nextafter(1.0, 0.0);
        const double t = u * W[m - 1];
        int32_t pick = m - 1;
        for (int32_t j = 0; j < m; ++j)
            if (W[j] > t) {
                pick = j;
                break;
            }
        out_token[r] = c[pick];
    }
    free(W);
    free(idx);
    return ORACLE_OK;
}

/* Number of threads a call with nthreads <= 0 would use. */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
