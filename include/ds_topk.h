/*
 * ds_topk -- row-wise small-k top-k selection on AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only.  Device buffers are HIP device
 * memory of the current device; `stream` is a hipStream_t (NULL = the null
 * stream).
 *
 * The operation (CSDN page "DeepSeek 一次开源三个仓库", section 三 算子层:
 * a top-k operator for sparse-attention indexing and for sampling, small k
 * only, at most 4096; its usage example is a topk(x, k) call with a
 * sorted-index flag and an index-type option that returns the values and
 * the indices):
 *
 *   For every row r of a [batch][row_stride] matrix, select the k largest of
 *   the elements in columns [0, n) and return their column indices (int32)
 *   and, optionally, their values.
 *
 *   "Largest" is a strict total order: element i comes before element j iff
 *   its value is larger, or both are zeros and i is +0 while j is -0, or the
 *   two values are the same and i < j (the lower index wins a tie).  +inf is
 *   largest and -inf smallest; they are ordinary values.  The answer is
 *   therefore unique for every input without NaN.
 *
 * Scenarios (aiutil project card "deepseek-ai/DeepSelect", 关键技术亮点
 * item 1): bf16 scores with any batch and length (the sparse-attention
 * "Lightning Indexer"), fp32 logits with a vocabulary of about 128K (the
 * sampler); k <= 4096 for both.  One library call serves both; the plan
 * (one workgroup per row, or several per row plus a merge) is chosen from
 * dtype, batch, n and k.
 */
#ifndef DS_TOPK_H
#define DS_TOPK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types (aiutil card, 关键技术亮点 item 1; no other dtype). */
enum ds_topk_dtype {
    DS_DTYPE_BF16 = 0, /* bfloat16: the upper 16 bits of an IEEE binary32 */
    DS_DTYPE_F32 = 1   /* IEEE binary32 */
};

/* Output order within a row (the `sorted_index` argument). */
enum ds_topk_order {
    DS_ORDER_NONE = 0,  /* any order; it may differ between calls */
    DS_ORDER_INDEX = 1, /* ascending column index */
    DS_ORDER_VALUE = 2  /* by value, largest first, in the selection's own
                           order (see the top of this file): equal values
                           by lower index, +0 before -0 */
};

/* Status codes returned by every entry point. */
enum ds_topk_status {
    DS_OK = 0,
    /* A null `in` or `out_idx`; `return_value` set with a null `out_val`;
       batch < 0; n < 1; k < 1; k > n; row_stride < n; sorted_index not a
       ds_topk_order. */
    DS_ERR_INVALID_ARGUMENT = 1,
    /* k > 4096 (CSDN page, section 三: small top-k only, at most 4096);
       an unknown dtype; n > 2^31 - 1 (indices are int32). */
    DS_ERR_UNSUPPORTED = 2,
    /* `in` not 16-byte aligned, or row_stride * element size not a multiple
       of 16 bytes.  The pages say input rows need a specific alignment and
       callers may need to pad them (zh-TW page "深入 DeepSeek V4.1
       全新開放推論工具包", section DeepSelect); here: pad each row to a
       multiple of 8 bf16 / 4 fp32 elements. */
    DS_ERR_MISALIGNED = 3,
    /* Some row holds a NaN (either sign, any payload) in columns [0, n).
       The pages: NaN checking is always on, and their default traps and
       aborts (same zh-TW page and section); this library reports it
       instead.  Outputs are unspecified.  Padding columns are never
       examined. */
    DS_ERR_NAN = 4,
    /* A HIP runtime call failed; ds_topk_last_error() has the detail. */
    DS_ERR_HIP = 5
};

#define DS_TOPK_MAX_K 4096

/*
 * ds_topk: top-k of every row, synchronous.
 *
 *   in           device pointer to batch * row_stride elements of `dtype`,
 *                row r at element offset r * row_stride, 16-byte aligned.
 *                Columns [n, row_stride) are padding: never used for results
 *                or NaN checks (they may be read, up to the next 16-byte
 *                boundary after column n - 1).
 *   dtype        DS_DTYPE_BF16 or DS_DTYPE_F32.
 *   batch        number of rows, >= 0 (0 is a no-op returning DS_OK).
 *   n            valid columns per row, 1 <= n <= 2^31 - 1.
 *   row_stride   elements between row starts, >= n; row_stride * element
 *                size must be a multiple of 16 bytes.
 *   k            1 <= k <= min(n, 4096).
 *   sorted_index a ds_topk_order.  DS_ORDER_INDEX: each row's k indices
 *                are written in ascending order (aiutil card, 关键技术亮点
 *                item 2, which names sorting by index or by value and notes
 *                that sorted output costs speed, so leave it off unless
 *                needed).  DS_ORDER_VALUE: largest value first, ties by
 *                lower index.  DS_ORDER_NONE: the order within a row is
 *                unspecified and may differ between calls; the set is
 *                always the same.
 *   return_value nonzero: write the selected values to out_val.  Zero: skip
 *                that output (zh-TW page, section DeepSelect:
 *                return_value=False skips the values and is faster).
 *   out_idx      device pointer, [batch][k] int32, contiguous: column
 *                indices in [0, n).
 *   out_val      device pointer, [batch][k] elements of `dtype`, contiguous;
 *                out_val[r][j] is a bit-exact copy of in[r][out_idx[r][j]]
 *                (-0, -inf and every bf16 bit pattern are kept).  May be
 *                NULL when return_value is zero.
 *   stream       hipStream_t the work is enqueued on.
 *
 * Ownership: the caller owns in, out_idx, out_val and the stream.  The
 * library owns a per-(device, stream) workspace (split-row lists, their
 * metadata and digit directories, tickets; a pinned host word for the NaN
 * status of synchronous calls).  It is allocated on first use and grows when a larger call needs
 * it: growth allocates a new block, clears it with a memset ordered on
 * `stream` and keeps the old block until the process exits or
 * ds_topk_release_stream, so work already queued, or a graph captured
 * earlier, never sees freed memory.  Growth never synchronises.
 *
 * Synchronisation: the call enqueues the kernel(s) on `stream`, then one
 * single-thread kernel that stores the call's completion tag and NaN status
 * into a pinned host word, and spins on that word (up to 2 ms, then it
 * waits for the stream, which also reports a failed kernel); when it
 * returns, the outputs are complete.  A synchronous call on a capturing
 * stream returns DS_ERR_HIP before enqueuing anything.
 * Argument errors are returned before any HIP call, and nothing is
 * written.  Calls on different streams may run concurrently; they use
 * different workspaces.  Calls on one stream share its workspace, so they
 * must run in stream order: a graph captured from ds_topk_async on a stream
 * must be replayed on that stream (or in order with its other calls), never
 * concurrently with them.  A call whose workspace would have to grow while
 * `stream` is capturing returns DS_ERR_HIP (make one uncaptured call of the
 * largest shape on the stream first).
 */
int ds_topk(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k,
            int sorted_index, int return_value, int32_t* out_idx, void* out_val, void* stream);

/*
 * ds_topk_async: the same selection, enqueued without waiting.
 *
 * Arguments are those of ds_topk, plus `status_dev`: a device pointer to one
 * int32 that the caller has set to 0 (DS_OK).  If any row holds a NaN, the
 * kernels store DS_ERR_NAN there; they never store anything else, so one
 * status word can collect several calls.  The return value reports argument
 * and launch errors only.  Work on `stream` is ordered as usual; the
 * workspace rules of ds_topk apply (calls on one stream may be queued back to
 * back).
 */
int ds_topk_async(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride,
                  int32_t k, int sorted_index, int return_value, int32_t* out_idx, void* out_val,
                  int32_t* status_dev, void* stream);

/*
 * ds_topk_async_noalloc: ds_topk_async for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc).  It calls no hipMalloc, hipFree or other
 * allocating routine.
 *
 * Arguments, outputs, status and errors are those of ds_topk_async; the
 * result is the same.  Split rows keep their hand-off state in a static
 * device array of 16 MiB (DS_TOPK_NOALLOC_SCRATCH_BYTES), one copy per
 * device, held until the process ends, instead of a workspace; a batch whose
 * state exceeds it runs as several launches of fewer rows.  A shape of
 * which one row alone needs more (at most k = 4096 with more than about 190
 * segments, i.e. rows of several million columns) returns
 * DS_ERR_UNSUPPORTED before any device call.  The first call on a device
 * also enqueues one small kernel on `stream` that clears the array's ticket
 * area.
 *
 * Every call on a device shares that device's array, and the array keeps
 * what the last call left in it: calls that overlap in time on one device
 * (other streams, other threads, replays of captured graphs running
 * concurrently with them) race and give wrong results.  Order them, e.g.
 * on one stream.
 */
#define DS_TOPK_NOALLOC_SCRATCH_BYTES (16ll << 20)
int ds_topk_async_noalloc(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride,
                          int32_t k, int sorted_index, int return_value, int32_t* out_idx, void* out_val,
                          int32_t* status_dev, void* stream);

/*
 * ds_topk_lengths: ds_topk with a valid length per row, in place of -inf
 * tails (a decode-time indexer row covers a context of its own length; the
 * aiutil card, 关键技术亮点 item 1, gives the indexer's vocab range as
 * 1~+∞).
 *
 * Arguments are those of ds_topk, plus `lengths`: a device pointer to batch
 * int32 values; row r's valid columns are [0, lengths[r]), a length outside
 * [0, n] being clamped to it.  Columns past a row's length act as -inf: they
 * are not read (beyond the 16-byte vector holding the row's last valid
 * column), never NaN-checked, and rank after every valid column; when
 * a row is shorter than k its output ends with those columns, lowest index
 * first, with -inf values (bit pattern 0xFF80 / 0xFF800000).  The result
 * equals ds_topk on the same rows with their tails set to -inf.  A null
 * `lengths` (with batch > 0) is DS_ERR_INVALID_ARGUMENT; the lengths
 * themselves are not validated on the host.  Synchronous, like ds_topk.
 */
int ds_topk_lengths(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k,
                    const int32_t* lengths, int sorted_index, int return_value, int32_t* out_idx,
                    void* out_val, void* stream);

/*
 * ds_topk_ex: every option in one call.  Arguments as ds_topk, except that
 * out_idx is untyped (its element type is set by the options) and `opt`
 * (may be NULL: all defaults) adds:
 *   index_bytes  4 (int32 indices; also 0) or 8 (int64: the usage example on
 *                the CSDN page, section 三, passes indices_type=torch.int32,
 *                one choice of an index type); other values are
 *                DS_ERR_INVALID_ARGUMENT.
 *   lengths      NULL, or per-row valid lengths as in ds_topk_lengths.
 *   status_dev   NULL: synchronous, as ds_topk.  Else: enqueue only, NaN
 *                reported into *status_dev, as ds_topk_async.
 * The caller owns the options struct; it is read during the call only.
 */
typedef struct ds_topk_options {
    int32_t index_bytes;
    const int32_t* lengths;
    int32_t* status_dev;
} ds_topk_options;

int ds_topk_ex(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k,
               int sorted_index, int return_value, void* out_idx, void* out_val, const ds_topk_options* opt,
               void* stream);

/*
 * ds_topk_sample: one token per row drawn from the row's top-k -- the step
 * after the selection on the sampler path.  The pages list temperature and
 * top-p among the generation parameters (CSDN page, section 二 接入层;
 * zh-TW page, the deepseek-recipe section) without a formula; this is the
 * textbook one.  With c_1 .. c_k the row's top-k in value order (as
 * DS_ORDER_VALUE) and x_j their values:
 *   w_j = exp((x_j - x_1) / T), taken as 1 where x_j == x_1 and as 0 for
 *         x_j = -inf below a larger x_1;
 *   W_j = w_1 + ... + w_j;
 *   m   = the smallest j with W_j >= top_p * W_k (the nucleus; k if none);
 *   the token is c_j for the smallest j <= m with W_j > u * W_m.
 * T <= 0 (or NaN) draws greedily: c_1.  u is clamped to [0, 1).
 *
 *   temperature, top_p, uniform  device pointers, batch floats each (u: the
 *                caller's uniform random numbers, one per row).
 *   out_token    device pointer, batch int32 column indices.
 * Other arguments, errors (NaN included) and synchronisation as ds_topk.
 * The weights and sums are fp32: a draw within a few fp32 ulps of a
 * boundary may land on the neighbouring candidate of the exact (real
 * number) draw.  The library keeps the k candidates of each row in a
 * per-(device, stream) buffer of its own.  For rows of more than 2048
 * columns with k <= 1024 the workgroup that writes a row's value-ordered
 * top-k also draws its token, in the same launch; otherwise a second kernel
 * draws from the candidates.  Both follow the definition above in fp32.
 */
int ds_topk_sample(const void* in, int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k,
                   const float* temperature, const float* top_p, const float* uniform, int32_t* out_token,
                   void* stream);

/* Static text for a status code ("unknown status" for other values). */
const char* ds_topk_status_string(int status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* ds_topk_last_error(void);

/*
 * The launch plan ds_topk would use for these arguments, without touching
 * the GPU.  Validates exactly like ds_topk (same status codes, except that
 * the pointer checks are skipped).
 */
typedef struct ds_topk_plan {
    int32_t segments;        /* workgroups per row; > 1 means split rows + merge;
                                0: rows of at most 2048 columns, one 64-lane
                                wave each, threads / 64 rows per workgroup */
    int32_t threads;         /* threads per workgroup */
    int32_t tiles_per_chunk; /* tiles whose loads are in flight together; a tile is
                                one 16-byte vector per thread */
    int32_t capacity;        /* candidate-buffer entries per workgroup (LDS) */
    int32_t segment_vectors; /* 16-byte vectors per segment (last may be shorter) */
    int32_t tiles_per_segment;
    int64_t grid;            /* workgroups launched */
    int64_t workspace_bytes; /* device workspace this call needs */
    int32_t publish_capacity;/* split rows: most entries one segment publishes */
} ds_topk_plan;

int ds_topk_plan_for(int dtype, int64_t batch, int64_t n, int64_t row_stride, int32_t k,
                     int sorted_index, int return_value, ds_topk_plan* plan);

/*
 * Tuning overrides for tests and measurements.  They apply to the calls the
 * calling thread makes (thread-local state; other threads keep their own).
 * segments > 0 forces that many workgroups per row (clamped to what the row
 * length allows); 0 restores the automatic choice.  tile_seed changes the
 * pseudo-random tile visiting order (the result never depends on it); 0
 * restores the default.  flags: DS_TOPK_FORCE_BITONIC makes index-ordered
 * output always use the bitonic sort instead of the bitmap ranking.
 */
#define DS_TOPK_FORCE_BITONIC 1
void ds_topk_set_overrides(int32_t segments, uint32_t tile_seed, int32_t flags);

/*
 * Waits for `stream`, then frees the workspace and sampling buffers the
 * library holds for (current device, stream), retired blocks included.  For
 * servers that create and destroy streams.  No graph captured on the stream
 * may be replayed afterwards.  Returns DS_OK, or DS_ERR_HIP.
 */
int ds_topk_release_stream(void* stream);

/* Library version, major * 10000 + minor * 100 + patch. */
int ds_topk_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DS_TOPK_H */
