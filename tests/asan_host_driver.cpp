// Drives the host half of libds_topk (argument checks, planning, the
// no-alloc entry point's size check, status strings, overrides) without a
// GPU, for a build of ds_topk.hip whose host code carries AddressSanitizer
// and UndefinedBehaviorSanitizer (tests/test_sanitizers.py).  Every call
// here returns before its first HIP call.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "ds_topk.h"

static int failures = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            ++failures;                                                 \
        }                                                               \
    } while (0)

int main() {
    void* fake = reinterpret_cast<void*>(uintptr_t(1) << 20);  // never dereferenced
    int32_t* fidx = static_cast<int32_t*>(fake);
    const int bf = DS_DTYPE_BF16, f32 = DS_DTYPE_F32;
    // planning over a spread of shapes, orders and forced segment counts
    const int64_t ns[] = {1, 7, 2048, 2049, 8192, 65536, 129280, 204800, 1 << 20, (int64_t(1) << 31) - 8};
    const int64_t batches[] = {0, 1, 4, 64, 257, 100000};
    const int32_t kk[] = {1, 64, 512, 1024, 1025, 4096};
    for (int forced : {0, 1, 3, 16, 300}) {
        ds_topk_set_overrides(forced, 0x1234u, DS_TOPK_FORCE_BITONIC);
        for (int dt : {bf, f32})
            for (int64_t n : ns)
                for (int64_t b : batches)
                    for (int32_t k : kk)
                        for (int order = 0; order < 3; ++order) {
                            ds_topk_plan p;
                            std::memset(&p, 0xAB, sizeof p);
                            const int64_t stride = (n + 7) / 8 * 8;
                            const int st = ds_topk_plan_for(dt, b, n, stride, k, order, 1, &p);
                            if (k > n) {
                                CHECK(st == DS_ERR_INVALID_ARGUMENT);
                                continue;
                            }
                            CHECK(st == DS_OK);
                            if (st) continue;
                            CHECK(p.threads > 0 && p.grid >= 0);
                            CHECK(p.segments >= 0 && p.segments <= 256);
                            CHECK(p.workspace_bytes >= 0);
                        }
    }
    ds_topk_set_overrides(0, 0, 0);
    // argument errors of every entry point
    CHECK(ds_topk(nullptr, bf, 4, 64, 64, 8, 0, 0, fidx, nullptr, nullptr) == DS_ERR_INVALID_ARGUMENT);
    CHECK(ds_topk(fake, bf, 4, 64, 64, 8, 0, 1, fidx, nullptr, nullptr) == DS_ERR_INVALID_ARGUMENT);
    CHECK(ds_topk(fake, 9, 4, 64, 64, 8, 0, 0, fidx, nullptr, nullptr) == DS_ERR_UNSUPPORTED);
    CHECK(ds_topk(fake, bf, 4, 64, 64, 4097, 0, 0, fidx, nullptr, nullptr) != DS_OK);
    CHECK(ds_topk(static_cast<char*>(fake) + 2, bf, 4, 64, 64, 8, 0, 0, fidx, nullptr, nullptr) == DS_ERR_MISALIGNED);
    CHECK(ds_topk(fake, bf, 4, 100, 100, 8, 0, 0, fidx, nullptr, nullptr) == DS_ERR_MISALIGNED);
    CHECK(ds_topk(fake, bf, 0, 64, 64, 8, 0, 0, fidx, nullptr, nullptr) == DS_OK);
    CHECK(ds_topk_async(fake, bf, 4, 64, 64, 8, 0, 0, fidx, nullptr, nullptr, nullptr) == DS_ERR_INVALID_ARGUMENT);
    CHECK(ds_topk_async_noalloc(fake, bf, 4, 64, 64, 8, 0, 0, fidx, nullptr, nullptr, nullptr) ==
          DS_ERR_INVALID_ARGUMENT);
    CHECK(ds_topk_async_noalloc(fake, bf, 1, int64_t(1) << 23, int64_t(1) << 23, 4096, 0, 0, fidx, nullptr,
                                fidx, nullptr) == DS_ERR_UNSUPPORTED);
    CHECK(std::strlen(ds_topk_last_error()) > 0);
    CHECK(ds_topk_lengths(fake, bf, 4, 64, 64, 8, nullptr, 0, 0, fidx, nullptr, nullptr) == DS_ERR_INVALID_ARGUMENT);
    ds_topk_options o;
    std::memset(&o, 0, sizeof o);
    o.index_bytes = 2;
    CHECK(ds_topk_ex(fake, bf, 4, 64, 64, 8, 0, 0, fidx, nullptr, &o, nullptr) == DS_ERR_INVALID_ARGUMENT);
    CHECK(ds_topk_sample(fake, bf, 4, 64, 64, 8, nullptr, nullptr, nullptr, nullptr, nullptr) ==
          DS_ERR_INVALID_ARGUMENT);
    CHECK(ds_topk_plan_for(bf, 4, 64, 64, 8, 0, 0, nullptr) == DS_ERR_INVALID_ARGUMENT);
    for (int s = -1; s < 8; ++s) CHECK(ds_topk_status_string(s) != nullptr);
    CHECK(ds_topk_version() >= 100);
    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("host driver: all checks passed\n");
    return 0;
}
