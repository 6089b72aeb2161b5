// Host side of the ds_topk C ABI: argument checks, launch planning,
// per-(device, stream) workspace, kernel launch and NaN status readback.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <utility>

#include "ds_topk.h"
#include "sample_kernels.hpp"
#include "topk_kernels.hpp"

namespace {

constexpr int kVersion = 100;       // 0.1.0
constexpr int kMaxSegs = 256;       // workgroups per row (merge keeps one LDS count each)
constexpr int kTargetWG = 256;      // one workgroup per CU on a 256-CU MI355X
constexpr int kSegPerK = 8;         // a segment holds at least 8k columns
constexpr int64_t kMinSegElems = 8192;  // and at least this many: below it the merge costs more than it saves
// Tiles per chunk (16-byte loads in flight per thread and buffer), per
// element width: a bf16 tile holds twice the elements of an fp32 one, and
// its eight slots per vector take more registers to filter.
#ifndef DS_TOPK_TILES_PER_CHUNK_F32
#define DS_TOPK_TILES_PER_CHUNK_F32 4
#endif
#ifndef DS_TOPK_TILES_PER_CHUNK_BF16
#define DS_TOPK_TILES_PER_CHUNK_BF16 2
#endif
// bf16 with k > 1024 (the larger buffer): one more tile in flight pays
// there (measured), while it slows the smaller-k shapes
#ifndef DS_TOPK_TILES_PER_CHUNK_BF16_BIGK
#define DS_TOPK_TILES_PER_CHUNK_BF16_BIGK 3
#endif
constexpr int kChunkF32 = DS_TOPK_TILES_PER_CHUNK_F32;
constexpr int kChunkBf16 = DS_TOPK_TILES_PER_CHUNK_BF16;
constexpr int kChunkBf16BigK = DS_TOPK_TILES_PER_CHUNK_BF16_BIGK;
constexpr int64_t kMaxGridWG = 1 << 22;  // workgroups per launch (grid x 512 threads < 2^32)

thread_local std::string g_err;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return status;
}

std::atomic<int32_t> g_force_segs{0};
std::atomic<uint32_t> g_tile_seed{0x2545F491u};
std::atomic<int32_t> g_flags{0};

struct Plan {
    int eb = 0;     // element bytes
    int wg = 512;   // threads per workgroup
    int vpt = 1;    // tiles per chunk (16-byte loads in flight per thread)
    int depth = 2;  // tiles in flight beyond the one being filtered
    int cap = 0;    // LDS candidate capacity
    int pub_cap = 0;  // candidates a segment may publish
    int segs = 1;
    int seg_vecs = 0;
    int n_vec = 0;
    int tiles = 0;
    int64_t rows_per_launch = 0;
    int64_t ws_bytes = 0;
};

int validate(int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k) {
    if (dtype != DS_DTYPE_BF16 && dtype != DS_DTYPE_F32)
        return fail(DS_ERR_UNSUPPORTED, "dtype %d is neither DS_DTYPE_BF16 nor DS_DTYPE_F32", dtype);
    if (batch < 0) return fail(DS_ERR_INVALID_ARGUMENT, "batch %lld < 0", (long long)batch);
    if (n < 1) return fail(DS_ERR_INVALID_ARGUMENT, "n %lld < 1", (long long)n);
    if (k < 1) return fail(DS_ERR_INVALID_ARGUMENT, "k %d < 1", k);
    if (n > 0x7FFFFFFFLL) return fail(DS_ERR_UNSUPPORTED, "n %lld exceeds the int32 index range", (long long)n);
    if (k > DS_TOPK_MAX_K) return fail(DS_ERR_UNSUPPORTED, "k %d > %d", k, DS_TOPK_MAX_K);
    if (k > n) return fail(DS_ERR_INVALID_ARGUMENT, "k %d > n %lld", k, (long long)n);
    if (row_stride < n)
        return fail(DS_ERR_INVALID_ARGUMENT, "row_stride %lld < n %lld", (long long)row_stride, (long long)n);
    const int64_t es = dtype == DS_DTYPE_BF16 ? 2 : 4;
    if ((row_stride * es) % 16 != 0)
        return fail(DS_ERR_MISALIGNED, "row pitch %lld bytes is not a multiple of 16", (long long)(row_stride * es));
    return DS_OK;
}

int make_plan(int dtype, int64_t batch, int64_t n, int32_t k, Plan* pl) {
    pl->eb = dtype == DS_DTYPE_BF16 ? 2 : 4;
    const int epv = 16 / pl->eb;
    pl->wg = 512;
    pl->depth = 0;
    pl->cap = k <= 1024 ? 8192 : 16384;
    // 16-byte loads in flight per thread (one chunk)
    pl->vpt = pl->eb == 4 ? kChunkF32 : pl->cap == 8192 ? kChunkBf16 : kChunkBf16BigK;
    pl->pub_cap = 2 * k + 1024 < pl->cap ? 2 * k + 1024 : pl->cap;
    pl->n_vec = (int)((n + epv - 1) / epv);
    int64_t s;
    const int32_t forced = g_force_segs.load();
    if (forced > 0) {
        s = forced;
    } else {
        s = batch >= kTargetWG ? 1 : (kTargetWG + batch - 1) / (batch > 0 ? batch : 1);
        const int64_t by_k = n / ((int64_t)kSegPerK * k);
        if (s > by_k) s = by_k;
        const int64_t by_size = n / kMinSegElems;
        if (s > by_size) s = by_size;
    }
    if (s > kMaxSegs) s = kMaxSegs;
    if (s > pl->n_vec) s = pl->n_vec;
    if (s < 1) s = 1;
    const int64_t by_rsrc = (pl->n_vec + dstk::kMaxSegVecs - 1) / dstk::kMaxSegVecs;
    if (s < by_rsrc) s = by_rsrc;  // each segment fits one buffer resource
    pl->seg_vecs = (int)((pl->n_vec + s - 1) / s);
    pl->segs = (pl->n_vec + pl->seg_vecs - 1) / pl->seg_vecs;
    pl->tiles = (pl->seg_vecs + pl->wg - 1) / pl->wg;
    const int64_t max_rows = kMaxGridWG / pl->segs;
    pl->rows_per_launch = batch < max_rows ? batch : max_rows;
    const int64_t r = pl->rows_per_launch;
    pl->ws_bytes = 256 + 256;  // NaN word
    if (pl->segs > 1) {
        pl->ws_bytes += ((r * 4 + 255) / 256) * 256;                          // tickets
        pl->ws_bytes += ((r * pl->segs * 32 + 255) / 256) * 256;              // segment metadata
        pl->ws_bytes += ((r * pl->segs * 4 * dstk::kBins + 255) / 256) * 256;  // digit directories
        pl->ws_bytes += ((r * pl->segs * (int64_t)pl->pub_cap * 8 + 255) / 256) * 256;  // candidates
    }
    return DS_OK;
}

// Rows this short take one wave each (dstk::topk_small_rows), unless a test
// forces a segment count; value order there holds up to kSmallValueMax.
constexpr int64_t kSmallRows = dstk::kSmallWG / dstk::kWave;  // rows per workgroup
bool use_small(int64_t n, int32_t k, int sorted_index) {
    return n <= dstk::kSmallN && g_force_segs.load() == 0 &&
           !(sorted_index == DS_ORDER_VALUE && k > dstk::kSmallValueMax);
}

// ------------------------------------------------------------------ workspace
struct Workspace {
    std::mutex mu;
    int device = -1;
    uint8_t* base = nullptr;
    int64_t rows = 0, slots = 0, cands = 0;
    int32_t* nan_word = nullptr;
    uint32_t* ticket = nullptr;
    uint64_t* meta = nullptr;
    uint32_t* dir = nullptr;
    uint64_t* cand = nullptr;
    int32_t* host_word = nullptr;  // pinned
    int32_t epoch = 0;
};

std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, std::unique_ptr<Workspace>> g_ws;

int hip_fail(hipError_t e, const char* what) {
    return fail(DS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Make sure ws can hold `rows` rows of `segs` segments of `per` entries.
int ensure(Workspace* ws, int64_t rows, int segs, int32_t per) {
    const int64_t need_rows = segs > 1 ? rows : 0;
    const int64_t need_slots = segs > 1 ? rows * segs : 0;
    const int64_t need_cands = segs > 1 ? rows * segs * (int64_t)per : 0;
    if (ws->base && need_rows <= ws->rows && need_slots <= ws->slots && need_cands <= ws->cands) return DS_OK;
    hipError_t e;
    if (!ws->host_word) {
        e = hipHostMalloc((void**)&ws->host_word, sizeof(int32_t), hipHostMallocDefault);
        if (e != hipSuccess) return hip_fail(e, "hipHostMalloc");
    }
    const int64_t rows2 = need_rows > ws->rows ? need_rows : ws->rows;
    const int64_t slots2 = need_slots > ws->slots ? need_slots : ws->slots;
    const int64_t cands2 = need_cands > ws->cands ? need_cands : ws->cands;
    auto al = [](int64_t b) { return ((b + 255) / 256) * 256; };
    const int64_t bytes = 256 + al(rows2 * 4) + al(slots2 * 32) + al(slots2 * 4 * dstk::kBins) + al(cands2 * 8);
    if (ws->base) {
        // Earlier calls may still be queued on this stream: let them finish.
        e = hipDeviceSynchronize();
        if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
        e = hipFree(ws->base);
        ws->base = nullptr;
        if (e != hipSuccess) return hip_fail(e, "hipFree");
    }
    e = hipMalloc((void**)&ws->base, (size_t)bytes);
    if (e != hipSuccess) {
        ws->base = nullptr;
        ws->rows = ws->slots = ws->cands = 0;
        return hip_fail(e, "hipMalloc(workspace)");
    }
    e = hipMemset(ws->base, 0, (size_t)bytes);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "hipMemset(workspace)");
    uint8_t* p = ws->base;
    ws->nan_word = (int32_t*)p;
    p += 256;
    ws->ticket = (uint32_t*)p;
    p += al(rows2 * 4);
    ws->meta = (uint64_t*)p;
    p += al(slots2 * 32);
    ws->dir = (uint32_t*)p;
    p += al(slots2 * 4 * dstk::kBins);
    ws->cand = (uint64_t*)p;
    ws->rows = rows2;
    ws->slots = slots2;
    ws->cands = cands2;
    ws->epoch = 0;
    return DS_OK;
}

Workspace* workspace_for(int dev, hipStream_t s) {
    std::lock_guard<std::mutex> g(g_ws_mu);
    auto& slot = g_ws[std::make_pair(dev, s)];
    if (!slot) {
        slot.reset(new Workspace());
        slot->device = dev;
    }
    return slot.get();
}

template <int EB, int WG, int NV, int CAP>
hipError_t launch_one(const dstk::Params& prm, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((dstk::topk_rows<EB, WG, NV, CAP>), dim3((uint32_t)grid), dim3(WG), 0, s, prm);
    return hipGetLastError();
}

// The instances make_plan can choose (element bytes, capacity).  (The
// fp32 instances come first in the code object: the sampler kernel's
// timing was measured in that placement.)
hipError_t launch(const Plan& pl, const dstk::Params& prm, int64_t rows, hipStream_t s) {
    const int64_t grid = rows * pl.segs;
    if (pl.eb == 4) {
        if (pl.cap == 8192) return launch_one<4, 512, kChunkF32, 8192>(prm, grid, s);
        return launch_one<4, 512, kChunkF32, 16384>(prm, grid, s);
    }
    if (pl.cap == 8192) return launch_one<2, 512, kChunkBf16, 8192>(prm, grid, s);
    return launch_one<2, 512, kChunkBf16BigK, 16384>(prm, grid, s);
}

int run(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k, int sorted_index,
        int return_value, void* out_idx, void* out_val, int32_t* status_dev, hipStream_t stream,
        const int32_t* lengths = nullptr, int index_bytes = 4) {
    g_err.clear();
    int st = validate(dtype, batch, n, row_stride, k);
    if (st) return st;
    if (sorted_index < DS_ORDER_NONE || sorted_index > DS_ORDER_VALUE)
        return fail(DS_ERR_INVALID_ARGUMENT, "sorted_index %d is not a ds_topk_order", sorted_index);
    if (index_bytes != 4 && index_bytes != 8)
        return fail(DS_ERR_INVALID_ARGUMENT, "index_bytes %d is neither 4 nor 8", index_bytes);
    if (!in) return fail(DS_ERR_INVALID_ARGUMENT, "in is NULL");
    if (!out_idx) return fail(DS_ERR_INVALID_ARGUMENT, "out_idx is NULL");
    if (return_value && !out_val) return fail(DS_ERR_INVALID_ARGUMENT, "return_value set but out_val is NULL");
    if (((uintptr_t)in) % 16 != 0) return fail(DS_ERR_MISALIGNED, "in is not 16-byte aligned");
    if (batch == 0) return DS_OK;
    Plan pl;
    make_plan(dtype, batch, n, k, &pl);
    const bool small = use_small(n, k, sorted_index);

    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    Workspace* ws = workspace_for(dev, stream);
    std::lock_guard<std::mutex> g(ws->mu);
    st = ensure(ws, pl.rows_per_launch, pl.segs, pl.pub_cap);
    if (st) return st;

    int32_t* flag = status_dev;
    int32_t flag_value = DS_ERR_NAN;
    if (!status_dev) {
        if (ws->epoch >= 0x7FFFFFF0) {
            e = hipMemsetAsync(ws->nan_word, 0, sizeof(int32_t), stream);
            if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync");
            ws->epoch = 0;
        }
        flag = ws->nan_word;
        flag_value = ++ws->epoch;
    }

    const int64_t es = dtype == DS_DTYPE_BF16 ? 2 : 4;
    for (int64_t r0 = 0; r0 < batch; r0 += pl.rows_per_launch) {
        const int64_t rows = batch - r0 < pl.rows_per_launch ? batch - r0 : pl.rows_per_launch;
        dstk::Params prm;
        prm.in = (const uint8_t*)in + r0 * row_stride * es;
        prm.row_stride_bytes = row_stride * es;
        prm.n = (int32_t)n;
        prm.k = k;
        prm.segs = pl.segs;
        prm.seg_vecs = pl.seg_vecs;
        prm.n_vec = pl.n_vec;
        prm.seed = g_tile_seed.load();
        prm.sorted = sorted_index;
        prm.retval = return_value ? 1 : 0;
        prm.out_idx = (uint8_t*)out_idx + r0 * k * index_bytes;
        prm.out_val = return_value ? (void*)((uint8_t*)out_val + r0 * k * es) : nullptr;
        prm.ws_cand = ws->cand;
        prm.ws_meta = ws->meta;
        prm.ws_dir = ws->dir;
        prm.pub_cap = pl.pub_cap;
        prm.ws_ticket = ws->ticket;
        prm.flag = flag;
        prm.flag_value = flag_value;
        prm.flags = (g_flags.load() & dstk::kFlagBitonic) | (index_bytes == 8 ? dstk::kFlagIdx64 : 0);
        prm.lengths = lengths ? lengths + r0 : nullptr;
        if (small) {
            const int64_t grid = (rows + kSmallRows - 1) / kSmallRows;
            if (dtype == DS_DTYPE_BF16)
                hipLaunchKernelGGL(dstk::topk_small_rows<2>, dim3((uint32_t)grid), dim3(dstk::kSmallWG), 0, stream,
                                   prm, rows);
            else
                hipLaunchKernelGGL(dstk::topk_small_rows<4>, dim3((uint32_t)grid), dim3(dstk::kSmallWG), 0, stream,
                                   prm, rows);
            e = hipGetLastError();
        } else {
            e = launch(pl, prm, rows, stream);
        }
        if (e != hipSuccess) return hip_fail(e, "kernel launch");
    }
    if (status_dev) return DS_OK;

    e = hipMemcpyAsync(ws->host_word, ws->nan_word, sizeof(int32_t), hipMemcpyDeviceToHost, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(status)");
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    if (*ws->host_word == flag_value) return fail(DS_ERR_NAN, "a row holds NaN in columns [0, n)");
    return DS_OK;
}

// ------------------------------------------------------------------ sampling
// Per-(device, stream) buffers of the value-ordered top-k that sampling reads.
struct SampleWs {
    std::mutex mu;
    void* buf = nullptr;  // idx [rows][k] int32, then values [rows][k]
    int64_t bytes = 0;
    int32_t* status = nullptr;
    int32_t* host_word = nullptr;  // pinned
};
std::mutex g_sws_mu;
std::map<std::pair<int, hipStream_t>, std::unique_ptr<SampleWs>> g_sws;

int sample(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k,
           const float* temperature, const float* top_p, const float* uniform, int32_t* out_token,
           hipStream_t stream) {
    g_err.clear();
    int st = validate(dtype, batch, n, row_stride, k);
    if (st) return st;
    if (!in || !temperature || !top_p || !uniform || !out_token)
        return fail(DS_ERR_INVALID_ARGUMENT, "a pointer argument is NULL");
    if (((uintptr_t)in) % 16 != 0) return fail(DS_ERR_MISALIGNED, "in is not 16-byte aligned");
    if (batch == 0) return DS_OK;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    SampleWs* sw;
    {
        std::lock_guard<std::mutex> g(g_sws_mu);
        auto& slot = g_sws[std::make_pair(dev, stream)];
        if (!slot) slot.reset(new SampleWs());
        sw = slot.get();
    }
    std::lock_guard<std::mutex> g(sw->mu);
    const int64_t es = dtype == DS_DTYPE_BF16 ? 2 : 4;
    const int64_t idx_bytes = ((batch * k * 4 + 255) / 256) * 256;
    const int64_t need = idx_bytes + batch * k * es;
    if (!sw->status) {
        e = hipMalloc((void**)&sw->status, 256);
        if (e != hipSuccess) return hip_fail(e, "hipMalloc(sample status)");
        e = hipHostMalloc((void**)&sw->host_word, sizeof(int32_t), hipHostMallocDefault);
        if (e != hipSuccess) return hip_fail(e, "hipHostMalloc");
    }
    if (need > sw->bytes) {
        if (sw->buf) {
            e = hipDeviceSynchronize();  // earlier calls on this stream may still read it
            if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
            e = hipFree(sw->buf);
            sw->buf = nullptr;
            sw->bytes = 0;
            if (e != hipSuccess) return hip_fail(e, "hipFree");
        }
        e = hipMalloc(&sw->buf, (size_t)need);
        if (e != hipSuccess) return hip_fail(e, "hipMalloc(sample buffers)");
        sw->bytes = need;
    }
    int32_t* cidx = (int32_t*)sw->buf;
    void* cval = (uint8_t*)sw->buf + idx_bytes;
    e = hipMemsetAsync(sw->status, 0, sizeof(int32_t), stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync");
    st = run(in, dtype, batch, n, row_stride, k, DS_ORDER_VALUE, 1, cidx, cval, sw->status, stream);
    if (st) return st;
    if (dtype == DS_DTYPE_BF16)
        hipLaunchKernelGGL(dssample::sample_rows<uint16_t>, dim3((uint32_t)batch), dim3(dssample::kWG), 0, stream,
                           (const uint16_t*)cval, cidx, k, temperature, top_p, uniform, out_token);
    else
        hipLaunchKernelGGL(dssample::sample_rows<float>, dim3((uint32_t)batch), dim3(dssample::kWG), 0, stream,
                           (const float*)cval, cidx, k, temperature, top_p, uniform, out_token);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "sample launch");
    e = hipMemcpyAsync(sw->host_word, sw->status, sizeof(int32_t), hipMemcpyDeviceToHost, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(status)");
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    if (*sw->host_word == DS_ERR_NAN) return fail(DS_ERR_NAN, "a row holds NaN in columns [0, n)");
    return DS_OK;
}

}  // namespace

extern "C" {

int ds_topk(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k, int sorted_index,
            int return_value, int32_t* out_idx, void* out_val, void* stream) {
    return run(in, dtype, batch, n, row_stride, k, sorted_index, return_value, out_idx, out_val, nullptr,
               (hipStream_t)stream);
}

int ds_topk_async(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k,
                  int sorted_index, int return_value, int32_t* out_idx, void* out_val, int32_t* status_dev,
                  void* stream) {
    if (!status_dev) return fail(DS_ERR_INVALID_ARGUMENT, "status_dev is NULL");
    return run(in, dtype, batch, n, row_stride, k, sorted_index, return_value, out_idx, out_val, status_dev,
               (hipStream_t)stream);
}
int ds_topk_lengths(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k,
                    const int32_t* lengths, int sorted_index, int return_value, int32_t* out_idx, void* out_val,
                    void* stream) {
    if (!lengths && batch > 0) return fail(DS_ERR_INVALID_ARGUMENT, "lengths is NULL");
    return run(in, dtype, batch, n, row_stride, k, sorted_index, return_value, out_idx, out_val, nullptr,
               (hipStream_t)stream, lengths);
}
int ds_topk_ex(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k, int sorted_index,
               int return_value, void* out_idx, void* out_val, const ds_topk_options* opt, void* stream) {
    ds_topk_options o{};
    if (opt) o = *opt;
    const int ib = o.index_bytes == 0 ? 4 : o.index_bytes;
    return run(in, dtype, batch, n, row_stride, k, sorted_index, return_value, out_idx, out_val, o.status_dev,
               (hipStream_t)stream, o.lengths, ib);
}
int ds_topk_sample(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k,
                   const float* temperature, const float* top_p, const float* uniform, int32_t* out_token,
                   void* stream) {
    return sample(in, dtype, batch, n, row_stride, k, temperature, top_p, uniform, out_token, (hipStream_t)stream);
}

const char* ds_topk_status_string(int status) {
    switch (status) {
        case DS_OK: return "DS_OK: success";
        case DS_ERR_INVALID_ARGUMENT: return "DS_ERR_INVALID_ARGUMENT: invalid argument";
        case DS_ERR_UNSUPPORTED: return "DS_ERR_UNSUPPORTED: unsupported dtype, k or n";
        case DS_ERR_MISALIGNED: return "DS_ERR_MISALIGNED: input or row pitch not 16-byte aligned";
        case DS_ERR_NAN: return "DS_ERR_NAN: input holds NaN";
        case DS_ERR_HIP: return "DS_ERR_HIP: HIP runtime error";
        default: return "unknown status";
    }
}

const char* ds_topk_last_error(void) { return g_err.c_str(); }

int ds_topk_plan_for(int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k, int sorted_index,
                     int return_value, ds_topk_plan* plan) {
    (void)return_value;
    g_err.clear();
    const int st = validate(dtype, batch, n, row_stride, k);
    if (st) return st;
    if (sorted_index < DS_ORDER_NONE || sorted_index > DS_ORDER_VALUE)
        return fail(DS_ERR_INVALID_ARGUMENT, "sorted_index %d is not a ds_topk_order", sorted_index);
    if (!plan) return fail(DS_ERR_INVALID_ARGUMENT, "plan is NULL");
    Plan pl;
    make_plan(dtype, batch, n, k, &pl);
    if (use_small(n, k, sorted_index)) {
        std::memset(plan, 0, sizeof *plan);
        plan->threads = dstk::kSmallWG;
        plan->grid = (batch + kSmallRows - 1) / kSmallRows;
        plan->workspace_bytes = 256;
        return DS_OK;
    }
    plan->segments = pl.segs;
    plan->threads = pl.wg;
    plan->tiles_per_chunk = pl.vpt;
    plan->capacity = pl.cap;
    plan->segment_vectors = pl.seg_vecs;
    plan->tiles_per_segment = pl.tiles;
    plan->grid = pl.rows_per_launch * pl.segs;
    plan->workspace_bytes = pl.ws_bytes;
    return DS_OK;
}

void ds_topk_set_overrides(int32_t segments, uint32_t tile_seed, int32_t flags) {
    g_force_segs.store(segments > 0 ? segments : 0);
    g_tile_seed.store(tile_seed ? tile_seed : 0x2545F491u);
    g_flags.store(flags & DS_TOPK_FORCE_BITONIC);
}

int ds_topk_version(void) { return kVersion; }

}  // extern "C"
