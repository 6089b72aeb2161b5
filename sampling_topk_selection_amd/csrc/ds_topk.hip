// Host side of the ds_topk C ABI: argument checks, launch planning,
// per-(device, stream) workspace, kernel launch and NaN status readback.
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "ds_topk.h"
#include "sample_kernels.hpp"
#include "topk_kernels.hpp"

namespace {

constexpr int kVersion = 100;       // 0.1.0
constexpr int kMaxSegs = 256;       // workgroups per row (merge keeps one LDS count each)
constexpr int kTargetWG = 256;      // one workgroup per CU on a 256-CU MI355X
constexpr int kSegPerK = 8;         // a segment holds at least 8k columns
constexpr int64_t kMinSegElems = 8192;  // and at least this many: below it the merge costs more than it saves
// (tiles per chunk of each instance: DS_TOPK_TILES_PER_CHUNK_*, topk_kernels.hpp)
constexpr int kChunkF32 = DS_TOPK_TILES_PER_CHUNK_F32;
constexpr int kChunkBf16 = DS_TOPK_TILES_PER_CHUNK_BF16;
constexpr int kChunkBf16BigK = DS_TOPK_TILES_PER_CHUNK_BF16_BIGK;
constexpr int64_t kMaxGridWG = 1 << 22;  // workgroups per launch (grid x 512 threads < 2^32)
// (row, segment) slots per launch of a split plan: bounds its workspace
// (at most 2048 x 9216 candidates x 8 bytes, 151 MB, at k = 4096).
constexpr int64_t kMaxSplitSlots = 2048;

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

// Test and measurement overrides (ds_topk_set_overrides), per calling thread.
constexpr uint32_t kDefaultTileSeed = 0x2545F491u;
thread_local int32_t g_force_segs = 0;
thread_local uint32_t g_tile_seed = kDefaultTileSeed;
thread_local int32_t g_flags = 0;

#ifdef DSTK_TIMING
uint64_t* g_timing = nullptr;  // measurement build: phase timestamps of the next launches
#endif

struct Plan {
    int eb = 0;     // element bytes
    int wg = 512;   // threads per workgroup
    int vpt = 1;    // tiles per chunk (16-byte loads in flight per thread)
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

int64_t al256(int64_t b) { return ((b + 255) / 256) * 256; }

// Bytes of the split-row workspace for `rows` rows of `segs` segments that
// publish at most `per` entries each: tickets, per-segment metadata (four
// u64), per-segment digit directories, lists.
int64_t split_ws_bytes(int64_t rows, int segs, int32_t per) {
    const int64_t slots = rows * segs;
    return al256(rows * 4) + al256(slots * 32) + al256(slots * 4 * dstk::kBins) + al256(slots * (int64_t)per * 8);
}

int make_plan(int dtype, int64_t batch, int64_t n, int32_t k, Plan* pl) {
    pl->eb = dtype == DS_DTYPE_BF16 ? 2 : 4;
    const int epv = 16 / pl->eb;
    pl->wg = 512;
    pl->cap = k <= 1024 ? 8192 : 16384;
    // 16-byte loads in flight per thread (one chunk)
    pl->vpt = pl->eb == 4 ? kChunkF32 : pl->cap == 8192 ? kChunkBf16 : kChunkBf16BigK;
    pl->pub_cap = 2 * k + 1024 < pl->cap ? 2 * k + 1024 : pl->cap;
    pl->n_vec = (int)((n + epv - 1) / epv);
    int64_t s;
    const int32_t forced = g_force_segs;
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
    int64_t max_rows = kMaxGridWG / pl->segs;
    if (pl->segs > 1) {
        const int64_t by_ws = kMaxSplitSlots / pl->segs;  // bounds the split workspace
        max_rows = by_ws < max_rows ? by_ws : max_rows;
        if (max_rows < 1) max_rows = 1;
    }
    pl->rows_per_launch = batch < max_rows ? batch : max_rows;
    pl->ws_bytes = pl->segs > 1 ? split_ws_bytes(pl->rows_per_launch, pl->segs, pl->pub_cap) : 0;
    return DS_OK;
}

// Rows this short take one wave each (dstk::topk_small_rows), unless a test
// forces a segment count; value order there holds up to kSmallValueMax.
constexpr int64_t kSmallRows = dstk::kSmallWG / dstk::kWave;  // rows per workgroup
bool use_small(int64_t n, int32_t k, int sorted_index) {
    return n <= dstk::kSmallN && g_force_segs == 0 &&
           !(sorted_index == DS_ORDER_VALUE && k > dstk::kSmallValueMax);
}

// ds_topk_sample draws each row's token in the selection's own launch
// (dstk::topk_sample_rows, after the row's value-ordered output) for the
// workgroup-per-row kernels with k <= 1024; else a second kernel does it
// (dssample::sample_rows) from the selection's output.
bool sampling_fused(int64_t n, int32_t k, const Plan& pl) {
    return !use_small(n, k, DS_ORDER_VALUE) && pl.cap == 8192;
}

// ------------------------------------------------------------------ workspace
// One per (device, stream).  A block that has been handed to kernels is
// never freed while the process runs (queued work, or a graph captured on
// the stream, may still use it); growth allocates a larger block, clears it
// with an ordered memset on the stream and retires the old one.
// Where the split-row kernels keep their hand-off state: per-row tickets
// (zero between calls), per-segment metadata and directories, lists.
struct WsPtrs {
    uint32_t* ticket = nullptr;
    uint64_t* meta = nullptr;
    uint32_t* dir = nullptr;
    uint64_t* cand = nullptr;
};

struct Workspace {
    std::mutex mu;
    int device = -1;
    uint8_t* base = nullptr;
    int64_t rows = 0, slots = 0, cands = 0;
    WsPtrs ptrs;
    std::vector<uint8_t*> retired;
    // synchronous calls: their kernels note a NaN in nan_word (device); a
    // signal kernel after them folds it into the pinned host word as
    // (epoch << 1) | nan and clears it, and the host spins on that word
    int32_t* host_word = nullptr;      // pinned
    int32_t* host_word_dev = nullptr;  // its device address
    int32_t* nan_word = nullptr;       // device memory, zero between calls
    int32_t epoch = 0;
};

std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, std::unique_ptr<Workspace>> g_ws;

int hip_fail(hipError_t e, const char* what) {
    return fail(DS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int capturing(hipStream_t s, bool* yes) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(s, &cs);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    *yes = cs != hipStreamCaptureStatusNone;
    return DS_OK;
}

// The words of synchronous calls (which never run under capture: they wait).
int ensure_host_word(Workspace* ws) {
    if (ws->host_word) return DS_OK;
    int32_t* h = nullptr;
    hipError_t e = hipHostMalloc((void**)&h, 256, hipHostMallocDefault);
    if (e != hipSuccess) return hip_fail(e, "hipHostMalloc");
    int32_t* d = nullptr;
    e = hipHostGetDevicePointer((void**)&d, h, 0);
    if (e != hipSuccess) {
        (void)hipHostFree(h);
        return hip_fail(e, "hipHostGetDevicePointer");
    }
    int32_t* nw = nullptr;
    e = hipMalloc((void**)&nw, 256);
    if (e == hipSuccess) e = hipMemset(nw, 0, 256);
    if (e != hipSuccess) {
        if (nw) (void)hipFree(nw);
        (void)hipHostFree(h);
        return hip_fail(e, "hipMalloc/hipMemset(NaN word)");
    }
    *h = 0;
    ws->host_word = h;
    ws->host_word_dev = d;
    ws->nan_word = nw;
    ws->epoch = 0;
    return DS_OK;
}

// Make sure ws can hold `rows` rows of `segs` segments of `per` entries.
int ensure(Workspace* ws, int64_t rows, int segs, int32_t per, hipStream_t stream) {
    if (segs <= 1) return DS_OK;
    const int64_t need_slots = rows * segs;
    const int64_t need_cands = rows * segs * (int64_t)per;
    if (ws->base && rows <= ws->rows && need_slots <= ws->slots && need_cands <= ws->cands) return DS_OK;
    bool cap_on = false;
    int st = capturing(stream, &cap_on);
    if (st) return st;
    if (cap_on)
        return fail(DS_ERR_HIP, "the workspace of this stream must grow, which cannot be captured; make one "
                                "uncaptured call of the largest shape on the stream first");
    const int64_t rows2 = rows > ws->rows ? rows : ws->rows;
    const int64_t slots2 = need_slots > ws->slots ? need_slots : ws->slots;
    const int64_t cands2 = need_cands > ws->cands ? need_cands : ws->cands;
    const int64_t bytes = al256(rows2 * 4) + al256(slots2 * 32) + al256(slots2 * 4 * dstk::kBins) + al256(cands2 * 8);
    uint8_t* nb = nullptr;
    hipError_t e = hipMalloc((void**)&nb, (size_t)bytes);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(workspace)");
    // tickets start at zero; ordered before the kernels on this stream
    e = hipMemsetAsync(nb, 0, (size_t)bytes, stream);
    if (e != hipSuccess) {
        (void)hipFree(nb);
        return hip_fail(e, "hipMemsetAsync(workspace)");
    }
    if (ws->base) ws->retired.push_back(ws->base);
    uint8_t* p = nb;
    ws->ptrs.ticket = (uint32_t*)p;
    p += al256(rows2 * 4);
    ws->ptrs.meta = (uint64_t*)p;
    p += al256(slots2 * 32);
    ws->ptrs.dir = (uint32_t*)p;
    p += al256(slots2 * 4 * dstk::kBins);
    ws->ptrs.cand = (uint64_t*)p;
    ws->base = nb;
    ws->rows = rows2;
    ws->slots = slots2;
    ws->cands = cands2;
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
}  // namespace

// The selection with its sampling step (sample_fused.hip: a translation unit
// of its own, so the selection kernels here share no out-of-line function
// with it and keep their own register allocation).
hipError_t ds_topk_launch_sample_fused(int eb, const dstk::Params& prm, int64_t grid, hipStream_t s);
// The selection with the 16384-entry buffer (bigk.hip: a unit of its own,
// built with other scheduling options).
hipError_t ds_topk_launch_bigk(int eb, const dstk::Params& prm, int64_t grid, hipStream_t s);
// The bf16 selection with the 8192-entry buffer (rows_bf16.hip, likewise).
hipError_t ds_topk_launch_bf16(const dstk::Params& prm, int64_t grid, hipStream_t s);

namespace {

// The instances make_plan can choose (element bytes, capacity).  (The
// fp32 instances come first in the code object: the sampler kernel's
// timing was measured in that placement.)
hipError_t launch(const Plan& pl, const dstk::Params& prm, int64_t rows, hipStream_t s, bool sample = false) {
    const int64_t grid = rows * pl.segs;
    if (sample) return ds_topk_launch_sample_fused(pl.eb, prm, grid, s);  // (sampling_fused: capacity 8192)
    if (pl.cap != 8192) return ds_topk_launch_bigk(pl.eb, prm, grid, s);
    if (pl.eb == 4) return launch_one<4, 512, kChunkF32, 8192>(prm, grid, s);
    return ds_topk_launch_bf16(prm, grid, s);
}

// Per-row sampling inputs and the token output, for a selection that draws
// the token in the same launch (see sampling_fused).
struct SampleIn {
    const float* temperature;
    const float* top_p;
    const float* uniform;
    int32_t* out_token;
};

// Checks the arguments and enqueues the selection on `stream`; a NaN makes
// the kernels store flag_value into *flag.  With `samp` (value order, a plan
// sampling_fused accepts) each row's workgroup also draws its token.
int enqueue(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k, int sorted_index,
            int return_value, void* out_idx, void* out_val, const WsPtrs& ws, int32_t* flag, int32_t flag_value,
            hipStream_t stream, const int32_t* lengths, int index_bytes, const Plan& pl,
            const SampleIn* samp = nullptr) {
    const bool small = use_small(n, k, sorted_index);
    const int64_t es = dtype == DS_DTYPE_BF16 ? 2 : 4;
    for (int64_t r0 = 0; r0 < batch; r0 += pl.rows_per_launch) {
        const int64_t rows = batch - r0 < pl.rows_per_launch ? batch - r0 : pl.rows_per_launch;
        dstk::Params prm{};
        prm.in = (const uint8_t*)in + r0 * row_stride * es;
        prm.row_stride_bytes = row_stride * es;
        prm.n = (int32_t)n;
        prm.k = k;
        prm.segs = pl.segs;
        prm.seg_vecs = pl.seg_vecs;
        prm.n_vec = pl.n_vec;
        prm.seed = g_tile_seed;
        prm.sorted = sorted_index;
        prm.retval = return_value ? 1 : 0;
        prm.out_idx = (uint8_t*)out_idx + r0 * k * index_bytes;
        prm.out_val = return_value ? (void*)((uint8_t*)out_val + r0 * k * es) : nullptr;
        prm.ws_cand = ws.cand;
        prm.ws_meta = ws.meta;
        prm.ws_dir = ws.dir;
        prm.ws_ticket = ws.ticket;
        prm.pub_cap = pl.pub_cap;
        prm.flag = flag;
        prm.flag_value = flag_value;
        prm.flags = (g_flags & dstk::kFlagBitonic) | (index_bytes == 8 ? dstk::kFlagIdx64 : 0);
        prm.lengths = lengths ? lengths + r0 : nullptr;
        if (samp) {
            prm.temperature = samp->temperature + r0;
            prm.top_p = samp->top_p + r0;
            prm.uniform = samp->uniform + r0;
            prm.out_token = samp->out_token + r0;
        }
#ifdef DSTK_TIMING
        prm.timing = g_timing;
#endif
        hipError_t e;
        if (small) {
            const int64_t grid = (rows + kSmallRows - 1) / kSmallRows;
            const bool tiny = n <= dstk::kTinyN;
            if (dtype == DS_DTYPE_BF16 && tiny)
                hipLaunchKernelGGL((dstk::topk_small_rows<2, 8>), dim3((uint32_t)grid), dim3(dstk::kSmallWG), 0,
                                   stream, prm, rows);
            else if (dtype == DS_DTYPE_BF16)
                hipLaunchKernelGGL((dstk::topk_small_rows<2, dstk::kHistBits>), dim3((uint32_t)grid),
                                   dim3(dstk::kSmallWG), 0, stream, prm, rows);
            else if (tiny)
                hipLaunchKernelGGL((dstk::topk_small_rows<4, 8>), dim3((uint32_t)grid), dim3(dstk::kSmallWG), 0,
                                   stream, prm, rows);
            else
                hipLaunchKernelGGL((dstk::topk_small_rows<4, dstk::kHistBits>), dim3((uint32_t)grid),
                                   dim3(dstk::kSmallWG), 0, stream, prm, rows);
            e = hipGetLastError();
        } else {
            e = launch(pl, prm, rows, stream, samp != nullptr);
        }
        if (e != hipSuccess) return hip_fail(e, "kernel launch");
    }
    return DS_OK;
}

int check_args(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k, int sorted_index,
               int return_value, const void* out_idx, const void* out_val, int index_bytes) {
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
    return DS_OK;
}

// The next epoch a synchronous call on ws waits for.  Only synchronous
// calls use the word, and each waits for its signal, so none is in flight
// here.
int32_t next_epoch(Workspace* ws) {
    if (ws->epoch >= 0x3FFFFFF0) {
        *(volatile int32_t*)ws->host_word = 0;
        ws->epoch = 0;
    }
    return ++ws->epoch;
}

// After a synchronous call's kernels on the stream: one thread reads and
// clears the NaN word (the kernels before it on the stream have completed)
// and stores (epoch << 1) | nan into the pinned host word.
__global__ void signal_done(int32_t* nan_word, int32_t* host_word, int32_t epoch) {
    if (threadIdx.x == 0) {
        const int32_t nan = *nan_word != 0 ? 1 : 0;
        *nan_word = 0;
        __hip_atomic_store(host_word, (int32_t)((uint32_t)epoch << 1) | nan, __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

// Enqueue the signal and wait for it: spin on the pinned word for up to
// 2 ms, then wait for the stream (which also reports a failed kernel).
// Spinning saves the runtime's completion path, about 10 us per call.
int signal_and_wait(Workspace* ws, int32_t epoch, hipStream_t stream) {
    hipLaunchKernelGGL(signal_done, dim3(1), dim3(64), 0, stream, ws->nan_word, ws->host_word_dev, epoch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "signal launch");
    volatile int32_t* w = ws->host_word;
    const auto t0 = std::chrono::steady_clock::now();
    int32_t v = *w;
    for (uint32_t i = 1; (v >> 1) != epoch; ++i) {
        if ((i & 1023u) == 0 && std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(2)) {
            e = hipStreamSynchronize(stream);
            if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
            v = *w;
            if ((v >> 1) != epoch) return fail(DS_ERR_HIP, "the completion word was not written");
            break;
        }
        __builtin_ia32_pause();
        v = *w;
    }
    if (v & 1) return fail(DS_ERR_NAN, "a row holds NaN in columns [0, n)");
    return DS_OK;
}

// Synchronous calls wait by spinning on their signal: refuse them while the
// stream captures (nothing would run).
int refuse_capture(hipStream_t stream) {
    bool cap_on = false;
    const int st = capturing(stream, &cap_on);
    if (st) return st;
    if (cap_on) return fail(DS_ERR_HIP, "a synchronous call cannot be captured; use ds_topk_async");
    return DS_OK;
}

int run(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k, int sorted_index,
        int return_value, void* out_idx, void* out_val, int32_t* status_dev, hipStream_t stream,
        const int32_t* lengths = nullptr, int index_bytes = 4) {
    g_err.clear();
    int st = check_args(in, dtype, batch, n, row_stride, k, sorted_index, return_value, out_idx, out_val, index_bytes);
    if (st) return st;
    if (batch == 0) return DS_OK;
    Plan pl;
    make_plan(dtype, batch, n, k, &pl);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    Workspace* ws = workspace_for(dev, stream);
    std::lock_guard<std::mutex> g(ws->mu);
    if (!status_dev) {
        st = refuse_capture(stream);
        if (st) return st;
        st = ensure_host_word(ws);
        if (st) return st;
    }
    st = ensure(ws, pl.rows_per_launch, use_small(n, k, sorted_index) ? 1 : pl.segs, pl.pub_cap, stream);
    if (st) return st;
    int32_t* flag = status_dev ? status_dev : ws->nan_word;
    st = enqueue(in, dtype, batch, n, row_stride, k, sorted_index, return_value, out_idx, out_val, ws->ptrs, flag,
                 DS_ERR_NAN, stream, lengths, index_bytes, pl);
    if (st || status_dev) return st;
    return signal_and_wait(ws, next_epoch(ws), stream);
}

// ------------------------------------------------------------------ sampling
// Per-(device, stream) buffers of the value-ordered top-k that sampling reads
// (grown like the workspace: never freed while the process runs).
struct SampleBuf {
    std::mutex mu;
    void* buf = nullptr;  // idx [rows][k] int32, then values [rows][k]
    int64_t bytes = 0;
    std::vector<void*> retired;
};
std::mutex g_sbuf_mu;
std::map<std::pair<int, hipStream_t>, std::unique_ptr<SampleBuf>> g_sbuf;

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
    st = refuse_capture(stream);
    if (st) return st;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    SampleBuf* sb;
    {
        std::lock_guard<std::mutex> g(g_sbuf_mu);
        auto& slot = g_sbuf[std::make_pair(dev, stream)];
        if (!slot) slot.reset(new SampleBuf());
        sb = slot.get();
    }
    std::lock_guard<std::mutex> g(sb->mu);
    const int64_t es = dtype == DS_DTYPE_BF16 ? 2 : 4;
    const int64_t idx_bytes = al256(batch * k * 4);
    const int64_t need = idx_bytes + batch * k * es;
    if (need > sb->bytes) {
        bool cap_on = false;
        st = capturing(stream, &cap_on);
        if (st) return st;
        if (cap_on) return fail(DS_ERR_HIP, "the sampling buffer of this stream must grow, which cannot be captured");
        void* nb = nullptr;
        e = hipMalloc(&nb, (size_t)need);
        if (e != hipSuccess) return hip_fail(e, "hipMalloc(sample buffers)");
        if (sb->buf) sb->retired.push_back(sb->buf);
        sb->buf = nb;
        sb->bytes = need;
    }
    int32_t* cidx = (int32_t*)sb->buf;
    void* cval = (uint8_t*)sb->buf + idx_bytes;
    Plan pl;
    make_plan(dtype, batch, n, k, &pl);
    Workspace* ws = workspace_for(dev, stream);
    std::lock_guard<std::mutex> g2(ws->mu);
    st = ensure_host_word(ws);
    if (st) return st;
    st = ensure(ws, pl.rows_per_launch, use_small(n, k, DS_ORDER_VALUE) ? 1 : pl.segs, pl.pub_cap, stream);
    if (st) return st;
    const SampleIn samp{temperature, top_p, uniform, out_token};
    const bool fused = sampling_fused(n, k, pl);
    st = enqueue(in, dtype, batch, n, row_stride, k, DS_ORDER_VALUE, 1, cidx, cval, ws->ptrs, ws->nan_word,
                 DS_ERR_NAN, stream, nullptr, 4, pl, fused ? &samp : nullptr);
    if (st) return st;
    if (!fused) {
        if (dtype == DS_DTYPE_BF16)
            hipLaunchKernelGGL(dssample::sample_rows<uint16_t>, dim3((uint32_t)batch), dim3(dssample::kWG), 0,
                               stream, (const uint16_t*)cval, cidx, k, temperature, top_p, uniform, out_token);
        else
            hipLaunchKernelGGL(dssample::sample_rows<float>, dim3((uint32_t)batch), dim3(dssample::kWG), 0, stream,
                               (const float*)cval, cidx, k, temperature, top_p, uniform, out_token);
        e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, "sample launch");
    }
    return signal_and_wait(ws, next_epoch(ws), stream);
}

// Releases the workspace and sampling buffers of (current device, stream)
// after waiting for the stream.
int release(hipStream_t stream) {
    g_err.clear();
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    std::unique_ptr<Workspace> w;
    std::unique_ptr<SampleBuf> b;
    {
        std::lock_guard<std::mutex> g(g_ws_mu);
        auto it = g_ws.find(std::make_pair(dev, stream));
        if (it != g_ws.end()) {
            w = std::move(it->second);
            g_ws.erase(it);
        }
    }
    {
        std::lock_guard<std::mutex> g(g_sbuf_mu);
        auto it = g_sbuf.find(std::make_pair(dev, stream));
        if (it != g_sbuf.end()) {
            b = std::move(it->second);
            g_sbuf.erase(it);
        }
    }
    hipError_t first = hipSuccess;
    auto fr = [&](void* p) {
        const hipError_t x = hipFree(p);
        if (x != hipSuccess && first == hipSuccess) first = x;
    };
    if (w) {
        std::lock_guard<std::mutex> g(w->mu);
        if (w->base) fr(w->base);
        for (uint8_t* p : w->retired) fr(p);
        if (w->host_word) {
            const hipError_t x = hipHostFree(w->host_word);
            if (x != hipSuccess && first == hipSuccess) first = x;
        }
        if (w->nan_word) fr(w->nan_word);
    }
    if (b) {
        std::lock_guard<std::mutex> g(b->mu);
        if (b->buf) fr(b->buf);
        for (void* p : b->retired) fr(p);
    }
    if (first != hipSuccess) return hip_fail(first, "hipFree");
    return DS_OK;
}

}  // namespace

// ------------------------------------------------------------------ no-alloc
// ds_topk_async_noalloc keeps the split-row hand-off state (tickets,
// metadata, directories, lists) in this array instead of a workspace.  Each
// device the library runs on holds its own copy until the process ends.
// Host code never passes this name to a kernel or a copy (on the host it is
// only a stand-in): it uses the copy's device address from
// hipGetSymbolAddress, taken once per device.
constexpr int64_t kScratchBytes = DS_TOPK_NOALLOC_SCRATCH_BYTES;
constexpr int64_t kScratchTicketBytes = 4096;  // tickets of up to 1024 rows, always at offset 0
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

static_assert(kMaxSplitSlots / 2 * 4 <= kScratchTicketBytes, "the ticket area holds the rows of any split launch");

__global__ void clear_words(uint32_t* p, int n) {
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch[kMaxDevices] = {};

// The device address of the current device's scratch copy.  The first use
// on a device takes the address and clears the ticket area with a kernel on
// `stream` (the array starts zeroed and every completed call leaves its
// tickets at zero; the clear makes that independent of what ran before).
int scratch_for(hipStream_t stream, uint8_t** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(DS_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(DS_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        const int words = (int)(kScratchTicketBytes / 4);
        hipLaunchKernelGGL(clear_words, dim3((uint32_t)((words + 255) / 256)), dim3(256), 0, stream, (uint32_t*)ptr,
                           words);
        e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, "scratch ticket clear");
        g_scratch[dev] = (uint8_t*)ptr;
    }
    *out = g_scratch[dev];
    return DS_OK;
}

// Bytes after the ticket area that `rows` split rows of the plan use.
int64_t scratch_state_bytes(const Plan& pl, int64_t rows) {
    const int64_t slots = rows * pl.segs;
    return al256(slots * 32) + al256(slots * 4 * dstk::kBins) + al256(slots * (int64_t)pl.pub_cap * 8);
}

// Rows per launch whose hand-off state fits the scratch (the plan's own, or
// fewer); an error if one row alone does not fit.
int scratch_rows(const Plan& pl, int64_t* rows_out) {
    const int64_t room = kScratchBytes - kScratchTicketBytes;
    const int64_t one = scratch_state_bytes(pl, 1);
    if (one > room)
        return fail(DS_ERR_UNSUPPORTED,
                    "ds_topk_async_noalloc: one row of %d segments publishing up to %d entries needs %lld bytes of "
                    "hand-off state; its static scratch holds %lld (use ds_topk_async)",
                    pl.segs, pl.pub_cap, (long long)one, (long long)room);
    int64_t rows = room / one < pl.rows_per_launch ? room / one : pl.rows_per_launch;
    while (rows > 1 && scratch_state_bytes(pl, rows) > room) --rows;
    *rows_out = rows;
    return DS_OK;
}

int run_noalloc(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k, int sorted_index,
                int return_value, void* out_idx, void* out_val, int32_t* status_dev, hipStream_t stream) {
    g_err.clear();
    if (!status_dev) return fail(DS_ERR_INVALID_ARGUMENT, "status_dev is NULL");
    int st = check_args(in, dtype, batch, n, row_stride, k, sorted_index, return_value, out_idx, out_val, 4);
    if (st) return st;
    if (batch == 0) return DS_OK;
    Plan pl;
    make_plan(dtype, batch, n, k, &pl);
    WsPtrs ws;
    if (!use_small(n, k, sorted_index) && pl.segs > 1) {
        int64_t rows = 0;
        st = scratch_rows(pl, &rows);  // (checked before any device call)
        if (st) return st;
        pl.rows_per_launch = rows;
        uint8_t* base = nullptr;
        st = scratch_for(stream, &base);
        if (st) return st;
        const int64_t slots = rows * pl.segs;
        ws.ticket = (uint32_t*)base;
        ws.meta = (uint64_t*)(base + kScratchTicketBytes);
        ws.dir = (uint32_t*)((uint8_t*)ws.meta + al256(slots * 32));
        ws.cand = (uint64_t*)((uint8_t*)ws.dir + al256(slots * 4 * dstk::kBins));
    }
    return enqueue(in, dtype, batch, n, row_stride, k, sorted_index, return_value, out_idx, out_val, ws, status_dev,
                   DS_ERR_NAN, stream, nullptr, 4, pl);
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
int ds_topk_async_noalloc(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k,
                          int sorted_index, int return_value, int32_t* out_idx, void* out_val, int32_t* status_dev,
                          void* stream) {
    return run_noalloc(in, dtype, batch, n, row_stride, k, sorted_index, return_value, out_idx, out_val, status_dev,
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
    std::memset(plan, 0, sizeof *plan);
    if (use_small(n, k, sorted_index)) {
        plan->threads = dstk::kSmallWG;
        plan->grid = (batch + kSmallRows - 1) / kSmallRows;
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
    plan->publish_capacity = pl.segs > 1 ? pl.pub_cap : 0;
    return DS_OK;
}

void ds_topk_set_overrides(int32_t segments, uint32_t tile_seed, int32_t flags) {
    g_force_segs = segments > 0 ? segments : 0;
    g_tile_seed = tile_seed ? tile_seed : kDefaultTileSeed;
    g_flags = flags & DS_TOPK_FORCE_BITONIC;
}

int ds_topk_release_stream(void* stream) { return release((hipStream_t)stream); }

#ifdef DSTK_TIMING
// Measurement build only: the next launches note their phase timestamps in
// buf[grid][16] (null: stop).
void ds_topk_timing_buffer(uint64_t* buf) { g_timing = buf; }
#endif

int ds_topk_version(void) { return kVersion; }

}  // extern "C"
