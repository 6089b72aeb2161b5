/* Drives the oracle (oracle/oracle.c) through every entry point and option
 * on small rows, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py).  Besides the
 * sanitizers' own checks it verifies what holds for any correct answer:
 * indices in range and distinct per row, values copied from the input (or
 * -inf past a row's length), NaN rows reported, bad arguments refused. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_topk(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k,
                int sorted_index, int return_value, int32_t* out_idx, void* out_val, int nthreads);
int oracle_topk_lengths(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k,
                        const int32_t* lengths, int sorted_index, int return_value, int32_t* out_idx,
                        void* out_val, int nthreads);
int oracle_sample(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k,
                  const float* temperature, const float* top_p, const float* uniform, int32_t* out_token);
int oracle_max_threads(void);

static int failures = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            ++failures;                                                 \
        }                                                               \
    } while (0)

static uint32_t rng = 12345u;
static uint32_t next_u32(void) {
    rng ^= rng << 13;
    rng ^= rng >> 17;
    rng ^= rng << 5;
    return rng;
}

enum { B = 3, N = 37, S = 40 };

static void fill(int dtype, void* buf, int with_nan) {
    static const uint16_t sp16[] = {0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x8001, 0x3F80, 0x7F7F};
    static const uint32_t sp32[] = {0x00000000u, 0x80000000u, 0x7F800000u, 0xFF800000u,
                                    0x00000001u, 0x80000001u, 0x3F800000u, 0x7F7FFFFFu};
    for (int i = 0; i < B * S; ++i) {
        const uint32_t r = next_u32();
        if (dtype == 0) {
            uint16_t v = (r & 7) == 0 ? sp16[(r >> 3) & 7] : (uint16_t)(0x3000 + ((r >> 8) & 0x1FFF));
            if (r & 0x80000000u) v ^= 0x8000;
            ((uint16_t*)buf)[i] = v;
        } else {
            uint32_t v = (r & 7) == 0 ? sp32[(r >> 3) & 7] : 0x3C000000u + ((r >> 8) & 0x1FFFFFFu);
            if (r & 0x80000000u) v ^= 0x80000000u;
            memcpy((uint32_t*)buf + i, &v, 4);
        }
    }
    if (with_nan) {
        if (dtype == 0)
            ((uint16_t*)buf)[1 * S + 5] = 0x7FC1;
        else {
            const uint32_t q = 0xFFC00001u;
            memcpy((uint32_t*)buf + 1 * S + 5, &q, 4);
        }
    }
}

static void check_rows(int dtype, const void* in, int k, const int32_t* lengths, const int32_t* idx,
                       const void* val) {
    const size_t es = dtype == 0 ? 2 : 4;
    for (int r = 0; r < B; ++r) {
        int len = lengths ? lengths[r] : N;
        len = len < 0 ? 0 : len > N ? N : len;
        for (int j = 0; j < k; ++j) {
            const int32_t c = idx[r * k + j];
            CHECK(c >= 0 && c < N);
            for (int t = 0; t < j; ++t) CHECK(idx[r * k + t] != c);
            if (val && c >= 0 && c < N) {
                const unsigned char* got = (const unsigned char*)val + es * (size_t)(r * k + j);
                if (c < len) {
                    CHECK(memcmp(got, (const unsigned char*)in + es * (size_t)(r * S + c), es) == 0);
                } else {
                    const uint16_t n16 = 0xFF80;
                    const uint32_t n32 = 0xFF800000u;
                    CHECK(memcmp(got, dtype == 0 ? (const void*)&n16 : (const void*)&n32, es) == 0);
                }
            }
        }
    }
}

int main(void) {
    static unsigned char in[B * S * 4];
    static int32_t idx[B * N];
    static unsigned char val[B * N * 4];
    const int ks[] = {1, 5, N};
    for (int dtype = 0; dtype < 2; ++dtype) {
        fill(dtype, in, 0);
        for (int ki = 0; ki < 3; ++ki)
            for (int order = 0; order < 3; ++order)
                for (int rv = 0; rv < 2; ++rv) {
                    const int k = ks[ki];
                    memset(idx, 0xFF, sizeof idx);
                    CHECK(oracle_topk(in, dtype, B, N, S, k, order, rv, idx, rv ? val : NULL, 2) == 0);
                    check_rows(dtype, in, k, NULL, idx, rv ? val : NULL);
                    const int32_t lens[B] = {-5, 10, 100};
                    CHECK(oracle_topk_lengths(in, dtype, B, N, S, k, lens, order, rv, idx, rv ? val : NULL, 0) == 0);
                    check_rows(dtype, in, k, lens, idx, rv ? val : NULL);
                }
        /* a NaN in row 1 */
        fill(dtype, in, 1);
        CHECK(oracle_topk(in, dtype, B, N, S, 5, 0, 1, idx, val, 1) == 4);
        const int32_t cut[B] = {N, 5, N};  /* the NaN at column 5 is past row 1's length */
        CHECK(oracle_topk_lengths(in, dtype, B, N, S, 5, cut, 2, 1, idx, val, 1) == 0);
        fill(dtype, in, 0);
        /* sampling over the options' corners */
        const float T[] = {0.0f, NAN, 0.7f, 2.0f};
        const float P[] = {0.0f, 0.5f, 1.0f, 2.0f};
        const float U[] = {-1.0f, 0.0f, 0.5f, 1.0f, 2.0f};
        for (int a = 0; a < 4; ++a)
            for (int b = 0; b < 4; ++b)
                for (int c = 0; c < 5; ++c) {
                    float t3[B], p3[B], u3[B];
                    int32_t tok[B];
                    for (int r = 0; r < B; ++r) {
                        t3[r] = T[a];
                        p3[r] = P[b];
                        u3[r] = U[c];
                    }
                    for (int ki = 0; ki < 3; ++ki) {
                        CHECK(oracle_sample(in, dtype, B, N, S, ks[ki], t3, p3, u3, tok) == 0);
                        for (int r = 0; r < B; ++r) CHECK(tok[r] >= 0 && tok[r] < N);
                    }
                }
    }
    /* refused arguments */
    CHECK(oracle_topk(in, 7, B, N, S, 5, 0, 0, idx, NULL, 1) == 1);
    CHECK(oracle_topk(in, 0, B, N, S, 0, 0, 0, idx, NULL, 1) == 1);
    CHECK(oracle_topk(in, 0, B, N, S, N + 1, 0, 0, idx, NULL, 1) == 1);
    CHECK(oracle_topk(in, 0, B, N, N - 1, 5, 0, 0, idx, NULL, 1) == 1);
    CHECK(oracle_topk(in, 0, B, N, S, 5, 3, 0, idx, NULL, 1) == 1);
    CHECK(oracle_topk(in, 0, B, N, S, 5, 0, 1, idx, NULL, 1) == 1);
    CHECK(oracle_topk(NULL, 0, B, N, S, 5, 0, 0, idx, NULL, 1) == 1);
    CHECK(oracle_sample(in, 0, B, N, S, 5, NULL, NULL, NULL, NULL) == 1);
    CHECK(oracle_max_threads() >= 1);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle driver: all checks passed\n");
    return 0;
}
