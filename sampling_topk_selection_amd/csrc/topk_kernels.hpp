// Device code for row-wise small-k top-k on gfx950 (CDNA4, wave64).
//
// Method (CSDN page "DeepSeek 一次开源三个仓库", section 三 算子层, its three
// steps): scan the input block by block in a random order and admit into a
// candidate buffer only elements above the current threshold; when the
// buffer grows large, or the scan ends, reduce the candidates to k in shared
// memory and raise the threshold to the least of the k kept; a higher
// threshold then rejects more of what follows.  The random order makes the
// threshold approach the true k-th value early.
//
// MI355X design:
//   * one workgroup streams one row segment with 16-byte buffer loads, in
//     chunks of tiles, the next chunk in flight while the current one is
//     filtered;
//   * every element is mapped to a 64-bit composite key
//         (order-preserving value key << ...) | (~column << ...)
//     so that the operator's total order (value, then +0 over -0, then the
//     lower column) is plain unsigned order and all keys are distinct;
//   * the first chunk is counted in an 11-bit histogram of composites and
//     the bin of its k-th entry seeds the admission bound;
//   * a float compare against the bound's value rejects most elements in one
//     VALU op (it also lets NaN through, to be caught exactly); survivors go
//     to the wave's own region of an LDS buffer behind a scalar write
//     pointer, with no atomics and no barrier;
//   * a full region, and a few scheduled points, move the regions together
//     (counting them), reduce the buffer if needed and raise the bound;
//   * short batches split each row over several workgroups; each publishes
//     its entries from the bin of its k-th up, by top digit, with a
//     directory of per-bin counts, and the last one to finish (agent-scope
//     ticket) merges them: row histogram from the directories, the share of
//     each segment at or above the row's k-th bin, exact selection;
//   * the exact k-th composite comes from radix levels inside its bin (or a
//     one-wave ranking when few entries remain); index-ordered output ranks
//     columns through a bitmap of the selected columns, value order sorts;
//   * rows of at most 2048 columns take one wave each (topk_small_rows).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

namespace dstk {

using u32 = uint32_t;
using u64 = uint64_t;
// A pointer to global memory in the compiler's address space 1: accesses
// are plain global_* instructions.  (A generic pointer whose origin the
// compiler cannot see becomes flat_* accesses, which also count against
// the LDS wait counter, so every LDS wait would wait for them too.)
template <class T>
using gptr = __attribute__((address_space(1))) T*;
// One 16-byte vector as the hardware loads it: kept whole in registers (a
// four-register tuple), so a load's destination is the register the scan
// reads, also across loop iterations.
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
// The first vector index of each tile of a chunk, passed by value.
template <int NV>
struct VecBases {
    int b[NV];
};

constexpr int kWave = 64;
// Word 3 of a raw buffer resource on CDNA (32-bit data format, no swizzle,
// no index stride): byte-addressed loads with a range check.
constexpr int kBufferWord3 = 0x00020000;
// Cache policy of the scan's loads: non-temporal (each input line is read
// once; measured on a plain 33 MB read over 256 workgroups: 6.9 -> 6.3 us).
constexpr int kScanAux = 2;
// A segment is addressed by one buffer resource: at most 2^27 vectors (2 GiB).
constexpr int kMaxSegVecs = 1 << 27;

// ------------------------------------------------------------------ elements
// Order-preserving keys: positive values get the sign bit set, negative
// values are bit-inverted, so unsigned key order is the IEEE totalOrder on
// non-NaN values (and +0 > -0).
template <int EB>
struct Elem;

template <>
struct Elem<2> {  // bfloat16
    static constexpr int kKeyBits = 16;
    static constexpr int kPerVec = 8;     // elements per 16-byte vector
    static constexpr int kIdxShift = 16;  // ~column occupies composite bits [16, 48)
    __device__ static u32 key(u32 b) { return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u); }
    __device__ static u32 bits(u32 key) { return (key & 0x8000u) ? (key & 0x7FFFu) : (~key & 0xFFFFu); }
    __device__ static bool is_nan(u32 b) { return (b & 0x7FFFu) > 0x7F80u; }
};

template <>
struct Elem<4> {  // fp32
    static constexpr int kKeyBits = 32;
    static constexpr int kPerVec = 4;
    static constexpr int kIdxShift = 0;  // ~column occupies composite bits [0, 32)
    __device__ static u32 key(u32 b) { return (b & 0x80000000u) ? ~b : (b | 0x80000000u); }
    __device__ static u32 bits(u32 key) { return (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key; }
    __device__ static bool is_nan(u32 b) { return (b & 0x7FFFFFFFu) > 0x7F800000u; }
};

template <class E>
__device__ __forceinline__ u64 compose(u32 key, u32 col) {
    return ((u64)key << (64 - E::kKeyBits)) | ((u64)(~col) << E::kIdxShift);
}
template <class E>
__device__ __forceinline__ u32 comp_key(u64 c) {
    return (u32)(c >> (64 - E::kKeyBits));
}
template <class E>
__device__ __forceinline__ u32 comp_col(u64 c) {
    return ~(u32)(c >> E::kIdxShift);
}

// Float thresholds for the one-op pre-filter "!(v < t)".  For an admission
// bound L (admit iff composite >= L) every admitted element has value >= the
// value of L's key, so the float test only lets through a superset.  A bound
// of 0 maps to a NaN threshold, which lets everything through.
template <class E>
struct PreFilter;

// Next value above the finite nonzero value of bits b (sign-magnitude, one
// step in the last place, toward +inf).
__device__ __forceinline__ u32 next_up(u32 b, u32 sign) { return (b & sign) ? b - 1u : b + 1u; }

template <>
struct PreFilter<Elem<2>> {
    float t;   // the threshold value, exact (bf16 << 16)
    float ts;  // the next bf16 value above it: "!(x < ts)" is "x > t" (strict_ok)
    bool strict_ok;  // t is finite or -inf, and not a zero
    __device__ void set(u64 L) {
        const u32 b = Elem<2>::bits(comp_key<Elem<2>>(L));
        t = __uint_as_float(b << 16);
        strict_ok = (b & 0x7FFFu) != 0u && b != 0x7F80u;
        ts = __uint_as_float(next_up(b, 0x8000u) << 16);
    }
    // Each half is compared alone (the other zeroed): read with its
    // neighbour, a -inf half would look like a NaN and always pass.
    __device__ u32 any(u32 d) const {
        return (u32)!(__uint_as_float(d & 0xFFFF0000u) < t) | (u32)!(__uint_as_float(d << 16) < t);
    }
};

template <>
struct PreFilter<Elem<4>> {
    float t;
    __device__ void set(u64 L) { t = __uint_as_float(Elem<4>::bits(comp_key<Elem<4>>(L))); }
    __device__ u32 any(u32 d) const { return (u32)!(__uint_as_float(d) < t); }
};

// Element s of a thread's 16-byte vector, given as its four words; s is a
// compile-time constant at every use, so this selects registers.  Slot order
// is element order (bf16: low half of a word first).
template <int s>
__device__ __forceinline__ u32 slot_bits(Elem<4>, const u32 (&dw)[4]) {
    return dw[s];
}
template <int s>
__device__ __forceinline__ u32 slot_bits(Elem<2>, const u32 (&dw)[4]) {
    return (s & 1) ? (dw[s >> 1] >> 16) : (dw[s >> 1] & 0xFFFFu);
}
// Pre-filter of element s: may it be at or above the bound (NaN passes)?
template <int s>
__device__ __forceinline__ bool pass_slot(const PreFilter<Elem<4>>& pf, const u32 (&dw)[4]) {
    return !(__uint_as_float(dw[s]) < pf.t);
}
template <int s>
__device__ __forceinline__ bool pass_slot(const PreFilter<Elem<2>>& pf, const u32 (&dw)[4]) {
    return (s & 1) ? !(__uint_as_float(dw[s >> 1] & 0xFFFF0000u) < pf.t) : !(__uint_as_float(dw[s >> 1] << 16) < pf.t);
}
// Is element s a NaN?  (Its value widened to fp32: a NaN stays a NaN.)
template <int s>
__device__ __forceinline__ bool nan_slot(Elem<4>, const u32 (&dw)[4]) {
    return __builtin_isnan(__uint_as_float(dw[s]));
}
template <int s>
__device__ __forceinline__ bool nan_slot(Elem<2>, const u32 (&dw)[4]) {
    return __builtin_isnan(__uint_as_float((s & 1) ? (dw[s >> 1] & 0xFFFF0000u) : (dw[s >> 1] << 16)));
}

// ------------------------------------------------------------------ shared
constexpr int kHistBits = 11;  // radix-select digit width
constexpr int kBins = 1 << kHistBits;
constexpr int kFlagBitonic = 1;  // Params::flags: always use the bitonic index sort
constexpr int kFlagIdx64 = 2;    // Params::flags: the output indices are int64
constexpr int kOrderIndex = 1;   // Params::sorted: ascending column index
constexpr int kOrderValue = 2;   // Params::sorted: largest composite first

// Where a row's column indices go: int32 or int64 elements.
struct IdxOut {
    gptr<void> p;
    int i64;
    __device__ __forceinline__ void put(u32 pos, u32 col) const {
        if (i64)
            ((gptr<int64_t>)p)[pos] = (int64_t)col;
        else
            ((gptr<int32_t>)p)[pos] = (int32_t)col;
    }
    __device__ __forceinline__ IdxOut at(u64 pos) const {
        return IdxOut{(gptr<void>)((gptr<uint8_t>)p + pos * (i64 ? 8u : 4u)), i64};
    }
};

// Histogram storage is transposed with a padded row: bin d lives at
// ((d mod 32) * 65 + d / 32), so atomics on consecutive bins (the hot bins
// next to the bound) and reads of runs of bins by consecutive lanes hit
// distinct banks.
constexpr int kHistRow = 65;
constexpr int kHistWords = 32 * kHistRow;
__device__ __forceinline__ u32 hidx(u32 d) { return (d & 31u) * (u32)kHistRow + (d >> 5); }

template <int CAP>
struct Smem {
    u64 buf[CAP];      // candidate composites
    u32 hist[kHistWords];  // radix-select histogram (bin d at hidx(d))
    u64 red[16][3];    // per-wave OR / AND / MIN
    u64 L;             // admission bound: admit iff composite >= L
    u64 kth;           // k-th composite after the last compaction
    u32 side_count;    // refine: entries gathered for it (in trash[])
    u32 count;         // entries in buf
    u32 sel_digit, sel_r, sel_c, sel_above, sel_total;
    u32 d_hi;
    u32 wsum[16];      // per-wave partial sums
    u32 nan;
    u32 last;
    u32 newtotal;
    u32 seg_count[256];  // merge: offset of each segment's list
    // wave_locate results, for up to two ranks
    u32 loc_digit[2], loc_r[2], loc_c[2], loc_above[2];
    u32 loc_total, loc_dhi;
    u32 outcount;        // emit: output slots handed out
    u32 pflag[2];        // scan: "some wave has a tile left over", two slots
    u32 wfill[16];       // scan: raw entries each wave has appended since the last sync
    u32 tie_min, tie_max;  // seed: least and greatest key in the crowded bin
    u32 tie_col;           // seed: column of the tied k-th entry
    u32 tie_cnt[8];        // seed: the crowded bin's entries per bound tile
    u32 pubseed;           // split row: the histogram holds the seed's publishing offsets
    u64 chain_t;           // refine: the k-th composite found by a chain walk
    u32 smp_m, smp_pick;   // sampling: nucleus end and the drawn slot
    float smp_w;           // sampling: the nucleus weight
    u32 lwsum[16];       // block_locate: per-wave bin totals
    u32 lwfirst[16];     // block_locate: per-wave highest non-empty bin (waves with any)
    u64 trash[64];       // scan: written by the lanes that append nothing
    u32 tbase[512];      // emit: per-thread base rank in the column bitmap
#ifdef DSTK_TIMING
    u64 ts[16];          // phase timestamps (measurement build only)
#endif
};

// Phase timestamps, compiled in only by the measurement build (DSTK_TIMING):
// thread 0 notes the constant 100 MHz clock at the points below, and a
// workgroup copies its notes to Params::timing[blockIdx.x][kTimingSlots]
// where it ends.  Unvisited points stay 0.
enum Phase : int {
    kPhStart = 0,     // kernel entry
    kPhSeed,          // seed bound located
    kPhScan,          // last chunk appended
    kPhSync,          // candidates converted and counted
    kPhLocate,        // bin of the segment's k-th entry located (split rows: and the directory written)
    kPhExchange,      // (unused)
    kPhPublish,       // candidates stored (split rows)
    kPhTicket,        // ticket taken (split rows)
    kPhHeaders,       // merger: metadata and directory heads read
    kPhLoad,          // merger: row histogram, row bin and shares worked out
    kPhMergeLocate,   // merger: the lists' needed prefixes loaded
    kPhRefine,        // exact k-th composite found
    kPhEmit,          // outputs written
    kTimingSlots = 16
};
#ifdef DSTK_TIMING
// Slots kClkStart / kClkEnd hold the shader clock counter (s_memtime) at
// entry and at the flush, for the workgroup's mean shader clock rate.
constexpr int kClkStart = 13, kClkEnd = 14;
#define DSTK_T(sm, id)                                                  \
    do {                                                                \
        if (threadIdx.x == 0) {                                         \
            (sm).ts[id] = wall_clock64();                               \
            if ((id) == kPhStart) (sm).ts[kClkStart] = clock64();       \
        }                                                               \
    } while (0)
#define DSTK_T_FLUSH(sm, timing)                                                      \
    do {                                                                              \
        if (threadIdx.x == 0 && (timing)) {                                           \
            (sm).ts[kClkEnd] = clock64();                                             \
            for (int i_ = 0; i_ < kTimingSlots; ++i_)                                 \
                (timing)[(uint64_t)blockIdx.x * kTimingSlots + i_] = (sm).ts[i_];     \
        }                                                                             \
    } while (0)
#else
#define DSTK_T(sm, id) ((void)0)
#define DSTK_T_FLUSH(sm, timing) ((void)0)
#endif

// Ends the wave where the last output of a workgroup is written (nothing
// follows it on any path; a return from an out-of-line caller would first
// reload the registers that caller saved).
#ifndef DSTK_EXIT
#define DSTK_EXIT() __builtin_amdgcn_endpgm()
#endif

// ------------------------------------------------------------------ wave helpers
// Cross-lane steps use DPP (row_shr, quad_perm, row mirrors, row_bcast15/31),
// which stay in the VALU; __shfl_* would be an LDS round trip per step.
__device__ __forceinline__ u32 lane_id() { return __lane_id(); }

__device__ __forceinline__ u32 mbcnt(u64 m) {
    return __builtin_amdgcn_mbcnt_hi((u32)(m >> 32), __builtin_amdgcn_mbcnt_lo((u32)m, 0u));
}
// base + number of lanes below this one whose bit is set in m
__device__ __forceinline__ u32 mbcnt_from(u64 m, u32 base) {
    return __builtin_amdgcn_mbcnt_hi((u32)(m >> 32), __builtin_amdgcn_mbcnt_lo((u32)m, base));
}

// A copy of x in a register of its own (one v_mov).  A 64-bit store of x
// and another value needs them in an aligned register pair; without the
// copy the compiler may place x there, and then keeps loaded vectors in
// split registers, copying them out of each load's destination (which
// waits for the load).
__device__ __forceinline__ u32 fresh_copy(u32 x) {
    u32 y;
    asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
    return y;
}

// Count bin d of each lane with `valid` in hist.  The lanes in the first
// active lane's bin are added by one atomic (all of them, for runs of equal
// values: the padding of short rows, quantized scores; often the most
// crowded bin otherwise), the others one by one: atomics that several lanes
// aim at one address are serialized.
__device__ __forceinline__ void hist_add(u32* hist, u32 d, bool valid) {
    const u64 act = __ballot(valid);
    if (act == 0) return;
    const u32 lead = (u32)__builtin_ctzll(act);
    const u32 first = __builtin_amdgcn_readlane(d, lead);
    const u64 same = __ballot(valid && d == first);
    if (__lane_id() == lead) atomicAdd(&hist[hidx(first)], (u32)__popcll(same));
    if (valid && d != first) atomicAdd(&hist[hidx(d)], 1u);
}

// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

// Inclusive prefix sum across the 64 lanes (all lanes active).
__device__ __forceinline__ u32 wave_incl_scan(u32 x) {
    x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// Reductions across the 64 lanes; the result is wave-uniform.
#define DSTK_WAVE_REDUCE(NAME, OPEXPR, IDENT)                                         \
    __device__ __forceinline__ u32 NAME(u32 v) {                                      \
        u32 t;                                                                        \
        t = __builtin_amdgcn_update_dpp(IDENT, v, 0xB1, 0xF, 0xF, false); v = OPEXPR;  \
        t = __builtin_amdgcn_update_dpp(IDENT, v, 0x4E, 0xF, 0xF, false); v = OPEXPR;  \
        t = __builtin_amdgcn_update_dpp(IDENT, v, 0x141, 0xF, 0xF, false); v = OPEXPR; \
        t = __builtin_amdgcn_update_dpp(IDENT, v, 0x140, 0xF, 0xF, false); v = OPEXPR; \
        t = __builtin_amdgcn_update_dpp(IDENT, v, 0x142, 0xA, 0xF, false); v = OPEXPR; \
        t = __builtin_amdgcn_update_dpp(IDENT, v, 0x143, 0xC, 0xF, false); v = OPEXPR; \
        return __builtin_amdgcn_readlane(v, 63);                                      \
    }
DSTK_WAVE_REDUCE(wave_min, (t < v ? t : v), 0xFFFFFFFFu)
DSTK_WAVE_REDUCE(wave_max, (t > v ? t : v), 0u)
DSTK_WAVE_REDUCE(wave_or, (t | v), 0u)
DSTK_WAVE_REDUCE(wave_and, (t & v), 0xFFFFFFFFu)
#undef DSTK_WAVE_REDUCE

__device__ __forceinline__ u64 wave_min64(u64 v) {
    const u32 hi = wave_min((u32)(v >> 32));
    const u32 lo = wave_min((u32)(v >> 32) == hi ? (u32)v : 0xFFFFFFFFu);
    return ((u64)hi << 32) | lo;
}
__device__ __forceinline__ u64 wave_max64(u64 v) {
    const u32 hi = wave_max((u32)(v >> 32));
    const u32 lo = wave_max((u32)(v >> 32) == hi ? (u32)v : 0u);
    return ((u64)hi << 32) | lo;
}

// Device-coherent (agent scope) stores and loads.  On gfx950 these are plain
// vector memory ops with the device-scope cache policy: stores go through to
// the device-coherent level, loads do not hit a stale L2 line.  Data handed
// from one workgroup to another goes through these, so the hand-off needs no
// release fence (which would write back the whole L2).
template <class P, class T>
__device__ __forceinline__ void st_agent(P p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class P>
__device__ __forceinline__ auto ld_agent(P p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A uniform value as an opaque register value.  Values loaded from the
// kernel-argument segment count as free to reload for the register
// allocator; under SGPR pressure it reloads them inside loops (a scalar
// load and a wait per use).  After this empty asm the value is an ordinary
// one that it keeps, or spills to a VGPR lane (one v_readlane).
template <class T>
__device__ __forceinline__ T keep(T x) {
    asm volatile("" : "+s"(x));
    return x;
}
// The same for a pointer to global memory, kept as one.
template <class T>
__device__ __forceinline__ gptr<T> keep_g(T* x) {
    uint64_t v = (uint64_t)(uintptr_t)x;
    asm volatile("" : "+s"(v));
    return (gptr<T>)(uintptr_t)v;
}
template <class T>
__device__ __forceinline__ gptr<T> keep_g(gptr<T> x) {
    uint64_t v = (uint64_t)(uintptr_t)x;
    asm volatile("" : "+s"(v));
    return (gptr<T>)(uintptr_t)v;
}

// Reserve `c` consecutive slots per lane behind *counter (one LDS atomic per
// wave); returns this lane's first slot, or ~0u if the wave has nothing.
__device__ __forceinline__ u32 wave_reserve(u32* counter, u32 c) {
    const u32 incl = wave_incl_scan(c);
    const u32 tot = __builtin_amdgcn_readlane(incl, 63);
    if (tot == 0) return ~0u;
    u32 base = 0;
    if (lane_id() == 0) base = atomicAdd(counter, tot);
    base = __builtin_amdgcn_readfirstlane(base);
    return base + incl - c;
}

// Reserve `tot` consecutive slots for the wave behind *counter, never past
// `cap`.  Returns the first slot, or kFull (reserving nothing) when they do
// not fit.  The result is wave-uniform (read from lane 0), so branches on it
// stay uniform.  Lock-free CAS by one lane.
constexpr u32 kFull = 0xFFFFFFFEu;
__device__ __forceinline__ u32 wave_reserve_base(u32* counter, u32 tot, u32 cap) {
    u32 base = 0;
    if (lane_id() == 0) {
        u32 old = __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        for (;;) {
            if (old + tot > cap) {
                base = kFull;
                break;
            }
            const u32 seen = atomicCAS(counter, old, old + tot);
            if (seen == old) {
                base = old;
                break;
            }
            old = seen;
        }
    }
    return __builtin_amdgcn_readfirstlane(base);
}

// ------------------------------------------------------------------ block helpers
// Exclusive prefix sum of one value per thread, in thread order; *total gets
// the block sum.  Separate consecutive calls by a barrier.
template <int WG, int CAP>
__device__ __forceinline__ u32 block_excl_scan(Smem<CAP>& sm, u32 v, u32* total) {
    const u32 wave = threadIdx.x / kWave;
    const u32 incl = wave_incl_scan(v);
    if (lane_id() == kWave - 1) sm.wsum[wave] = incl;
    __syncthreads();
    u32 off = 0, tot = 0;
#pragma unroll
    for (u32 w = 0; w < WG / kWave; ++w) {
        const u32 s = sm.wsum[w];
        off += w < wave ? s : 0u;
        tot += s;
    }
    *total = tot;
    return off + incl - v;
}

constexpr int kBatch = 8;  // LDS loads kept in flight per thread in buffer passes
// A seed bin this crowded is checked for a single value (the tied seed bound).
constexpr u32 kTiedBin = 512;

// MIN and MAX over the entries of buf[lo, hi) whose bits under `mask` equal
// `prefix` (MIN = ~0, MAX = 0 when none do).  Also zeroes the histogram for
// the block_hist_find that follows.  Separate consecutive calls by a barrier.
template <int WG, int CAP>
__device__ __forceinline__ void block_minmax(Smem<CAP>& sm, u32 lo, u32 hi, u64 prefix, u64 mask, u64& mn, u64& mx) {
    const u32 tid = threadIdx.x;
    for (u32 i = tid; i < (u32)kHistWords; i += WG) sm.hist[i] = 0;
    u64 vmn = ~0ull, vmx = 0;
    for (u32 base = lo; base < hi; base += WG * kBatch) {
        u64 v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const u32 i = base + u * WG + tid;
            v[u] = i < hi ? sm.buf[i] : 0ull;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const u32 i = base + u * WG + tid;
            if (i < hi && (v[u] & mask) == prefix) {
                vmn = v[u] < vmn ? v[u] : vmn;
                vmx = v[u] > vmx ? v[u] : vmx;
            }
        }
    }
    vmn = wave_min64(vmn);
    vmx = wave_max64(vmx);
    const u32 wave = tid / kWave;
    if (lane_id() == 0) {
        sm.red[wave][0] = vmn;
        sm.red[wave][1] = vmx;
    }
    __syncthreads();
    mn = ~0ull;
    mx = 0;
#pragma unroll
    for (u32 w = 0; w < WG / kWave; ++w) {
        mn = sm.red[w][0] < mn ? sm.red[w][0] : mn;
        mx = sm.red[w][1] > mx ? sm.red[w][1] : mx;
    }
}

// In the filled histogram, the bin holding the r-th largest counted entry
// (r >= 1), scanning from the highest bin.  Leaves sel_digit, sel_r (rank
// inside the bin), sel_c (bin size) and sel_above (entries in higher bins) in
// shared memory; sel_c = 0 when fewer than r entries are counted.
template <int WG, int CAP>
__device__ __forceinline__ void hist_locate(Smem<CAP>& sm, u32 r) {
    const u32 tid = threadIdx.x;
    if (tid == 0) {  // overwritten below unless fewer than r are counted
        sm.sel_digit = 0;
        sm.sel_r = 0;
        sm.sel_c = 0;
        sm.sel_above = 0;
    }
    constexpr int kPer = kBins / WG;  // bins per thread, highest bins first
    u32 h[kPer];
    u32 s = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        h[j] = sm.hist[hidx(kBins - 1 - tid * kPer - j)];
        s += h[j];
    }
    u32 tot;
    const u32 excl = block_excl_scan<WG, CAP>(sm, s, &tot);
    if (tid == 0) sm.sel_total = tot;
    if (excl < r && r <= excl + s) {
        u32 acc = excl;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            if (acc < r && r <= acc + h[j]) {
                sm.sel_digit = kBins - 1 - tid * kPer - j;
                sm.sel_r = r - acc;
                sm.sel_c = h[j];
                sm.sel_above = acc;
            }
            acc += h[j];
        }
    }
    __syncthreads();
}

// Histogram of the digit (e >> shift) & (kBins-1) over the entries of
// buf[lo, hi) matching (prefix, mask) -- the histogram must have been zeroed
// by block_minmax -- then hist_locate(r).
template <int WG, int CAP>
__device__ __forceinline__ void block_hist_find(Smem<CAP>& sm, u32 lo, u32 hi, u64 prefix, u64 mask, int shift, u32 r) {
    const u32 tid = threadIdx.x;
    for (u32 base = lo; base < hi; base += WG * kBatch) {
        u64 v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const u32 i = base + u * WG + tid;
            v[u] = i < hi ? sm.buf[i] : 0ull;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const u32 i = base + u * WG + tid;
            if (i < hi && (v[u] & mask) == prefix) atomicAdd(&sm.hist[hidx((u32)(v[u] >> shift) & (kBins - 1))], 1u);
        }
    }
    __syncthreads();
    hist_locate<WG, CAP>(sm, r);
}

// Window of kHistBits bits whose top bit is the highest bit set in diff.
__device__ __forceinline__ int window_shift(u64 diff) {
    const int msb = 63 - __clzll((long long)diff);
    return msb >= kHistBits - 1 ? msb - (kHistBits - 1) : 0;
}
__device__ __forceinline__ u64 bits_above(int shift) {
    return shift + kHistBits >= 64 ? 0ull : (~0ull << (shift + kHistBits));
}

// ------------------------------------------------------------------ compaction
// Keep the entries of buf[lo, hi) that are >= T, packed from position lo in a
// deterministic order (block prefix sum).  Returns the kept count.
template <int WG, int CAP>
__device__ __forceinline__ u32 keep_at_least(Smem<CAP>& sm, u32 lo, u32 hi, u64 T) {
    const u32 tid = threadIdx.x;
    constexpr int kItems = CAP / WG;
    u64 mine[kItems];
    u32 nk = 0;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const u32 i = lo + tid + j * WG;
        mine[j] = i < hi ? sm.buf[i] : 0ull;
        nk += (i < hi && mine[j] >= T) ? 1u : 0u;
    }
    u32 tot;
    u32 pk = lo + block_excl_scan<WG, CAP>(sm, nk, &tot);  // its barrier orders reads before writes
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const u32 i = lo + tid + j * WG;
        if (i < hi && mine[j] >= T) sm.buf[pk++] = mine[j];
    }
    __syncthreads();
    return tot;
}

// The r-th largest entry of the undecided set (entries of buf[lo, hi)
// matching prefix/mask).  Radix select with 11-bit digits whose window
// starts at the highest bit where the undecided entries differ.
template <int WG, int CAP>
__device__ __forceinline__ u64 select_in(Smem<CAP>& sm, u32 lo, u32 hi, u64 prefix, u64 mask, u32 r) {
    u64 mn, mx;
    // Each level fixes at least one more bit; the bound only guards the loop.
    for (int level = 0; level < 64 / kHistBits + 2; ++level) {
        block_minmax<WG, CAP>(sm, lo, hi, prefix, mask, mn, mx);
        if (mn == mx) return mn;  // a single entry left
        const int shift = window_shift(mn ^ mx);
        // keep the bits fixed so far: a window clamped at bit 0 can overlap them
        mask |= bits_above(shift);
        prefix = mn & mask;
        block_hist_find<WG, CAP>(sm, lo, hi, prefix, mask, shift, r);
        const u32 d = sm.sel_digit, c = sm.sel_c, rr = sm.sel_r;
        prefix |= (u64)d << shift;
        mask |= (u64)(kBins - 1) << shift;
        if (rr == c) break;  // the whole bin is kept: the answer is its least entry
        r = rr;
    }
    block_minmax<WG, CAP>(sm, lo, hi, prefix, mask, mn, mx);
    return mn;
}

// Reduce buf[0, cnt) (distinct composites, cnt > k) to its k largest, in
// buf[0, k); sets kth and the bound L to the least kept entry.
//
// First level over the whole buffer; then the buffer is partitioned once
// (entries in higher bins kept outright, the boundary bin moved next to
// them) and only the boundary list is refined.
template <class E, int WG, int CAP>
__device__ __forceinline__ void compact_to_k(Smem<CAP>& sm, u32 cnt, u32 k) {
    const u32 tid = threadIdx.x;
    constexpr int kItems = CAP / WG;
    u64 mn, mx;
    block_minmax<WG, CAP>(sm, 0, cnt, 0ull, 0ull, mn, mx);
    const int shift = window_shift(mn ^ mx);
    u64 mask = bits_above(shift);
    u64 prefix = mn & mask;
    block_hist_find<WG, CAP>(sm, 0, cnt, prefix, mask, shift, k);
    const u32 b = sm.sel_digit, above = sm.sel_above, c = sm.sel_c, r = sm.sel_r;

    // Partition: higher bins to [0, above), bin b to [above, above + c).
    u64 mine[kItems];
    u32 nd = 0, nm = 0;
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const u32 i = tid + j * WG;
        mine[j] = i < cnt ? sm.buf[i] : 0ull;
        const u32 d = (u32)(mine[j] >> shift) & (kBins - 1);
        nd += (i < cnt && d > b) ? 1u : 0u;
        nm += (i < cnt && d == b) ? 1u : 0u;
    }
    u32 tot;
    const u32 ex = block_excl_scan<WG, CAP>(sm, nd | (nm << 16), &tot);  // counts < 2^16
    u32 pd = ex & 0xFFFFu, pm = above + (ex >> 16);
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const u32 i = tid + j * WG;
        const u32 d = (u32)(mine[j] >> shift) & (kBins - 1);
        if (i < cnt && d > b) sm.buf[pd++] = mine[j];
        if (i < cnt && d == b) sm.buf[pm++] = mine[j];
    }
    __syncthreads();
    prefix |= (u64)b << shift;
    mask |= (u64)(kBins - 1) << shift;

    const u32 lo = above, hi = above + c;
    const u64 T = select_in<WG, CAP>(sm, lo, hi, prefix, mask, r);
    if (r != c) {
        __syncthreads();
        keep_at_least<WG, CAP>(sm, lo, hi, T);
    }
    if (tid == 0) {
        sm.count = k;
        sm.kth = T;
        // inclusive bound: k entries are >= T, and any later element is
        // admitted only if it is > T (composites are distinct)
        sm.L = T;
    }
    __syncthreads();
}

// ------------------------------------------------------------------ histogram-tracked bound
// The workgroup keeps a histogram of the top kHistBits bits of the value key
// of every entry it has appended to the buffer (and, for the first tile, of
// every element of that tile).  The lower edge of the bin holding the k-th
// counted entry is a valid admission bound: at least k counted elements lie
// at or above it.  Invariant: for every bin at or above the current bound's
// bin, the histogram count equals the number of buffer entries in that bin.
__device__ __forceinline__ u32 top_digit(u64 c) { return (u32)(c >> (64 - kHistBits)); }
__device__ __forceinline__ u64 digit_floor(u32 d) { return (u64)d << (64 - kHistBits); }

// Recount the buffer into a zeroed histogram (after an exact reduction).
template <int WG, int CAP>
__device__ __forceinline__ void rebuild_hist(Smem<CAP>& sm, u32 cnt) {
    const u32 tid = threadIdx.x;
    for (u32 i = tid; i < (u32)kHistWords; i += WG) sm.hist[i] = 0;
    __syncthreads();
    for (u32 base = 0; base < cnt; base += WG) {
        const u32 i = base + tid;
        hist_add(sm.hist, i < cnt ? top_digit(sm.buf[i]) : 0u, i < cnt);
    }
    __syncthreads();
}

// Free room for `room` more entries: drop entries below the histogram
// bound's bin edge, or, if that is not enough, reduce exactly to k.
template <class E, int WG, int CAP>
__device__ __noinline__ void make_room(Smem<CAP>& sm, u32 cnt, u32 k, u32 room) {
    const u32 tid = threadIdx.x;
    hist_locate<WG, CAP>(sm, k);
    const u32 d = sm.sel_digit, keep = sm.sel_above + sm.sel_c;
    if (sm.sel_c > 0 && keep + room <= (u32)CAP) {
        // (at least 1: the empty composite 0 left by an overflow never stays)
        const u32 kept = keep_at_least<WG, CAP>(sm, 0, cnt, d > 0 ? digit_floor(d) : 1ull);
        if (tid == 0) {
            sm.count = kept;
            sm.L = digit_floor(d) > sm.L ? digit_floor(d) : sm.L;
        }
        __syncthreads();
        return;
    }
    compact_to_k<E, WG, CAP>(sm, cnt, k);
    rebuild_hist<WG, CAP>(sm, k);
}

// Reduce the buffer (cnt >= k entries, histogram consistent) to exactly the
// k largest, in buf[0, k).  The histogram gives the first radix level.
template <class E, int WG, int CAP>
__device__ __noinline__ void final_select(Smem<CAP>& sm, u32 cnt, u32 k) {
    const u32 tid = threadIdx.x;
    constexpr int kItems = CAP / WG;
    if (cnt > k) {
        hist_locate<WG, CAP>(sm, k);
        const u32 b = sm.sel_digit, above = sm.sel_above, c = sm.sel_c, r = sm.sel_r;
        // Partition: higher bins to [0, above), bin b to [above, above + c).
        u64 mine[kItems];
        u32 nd = 0, nm = 0;
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            const u32 i = tid + j * WG;
            mine[j] = i < cnt ? sm.buf[i] : 0ull;
            const u32 d = top_digit(mine[j]);
            nd += (i < cnt && d > b) ? 1u : 0u;
            nm += (i < cnt && d == b) ? 1u : 0u;
        }
        u32 tot;
        const u32 ex = block_excl_scan<WG, CAP>(sm, nd | (nm << 16), &tot);  // counts < 2^16
        u32 pd = ex & 0xFFFFu, pm = above + (ex >> 16);
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            const u32 i = tid + j * WG;
            const u32 d = top_digit(mine[j]);
            if (i < cnt && d > b) sm.buf[pd++] = mine[j];
            if (i < cnt && d == b) sm.buf[pm++] = mine[j];
        }
        __syncthreads();
        if (r != c) {
            const u64 mask = ~0ull << (64 - kHistBits);
            const u64 T = select_in<WG, CAP>(sm, above, above + c, digit_floor(b), mask, r);
            __syncthreads();
            keep_at_least<WG, CAP>(sm, above, above + c, T);
        }
    }
    if (tid == 0) sm.count = k;
    __syncthreads();
}

// ------------------------------------------------------------------ output
// Ranks of the selected columns in index order, from a bitmap of them.
// Thread t owns the 2^lp consecutive bitmap words [t 2^lp, (t + 1) 2^lp),
// kept as one row of an LDS table with an odd pitch (2^lp + 1 words when
// 2^lp > 1), so the lanes of a wave reading word j of their own rows hit
// distinct banks.  A block scan of the rows' popcounts gives each row's
// first rank.  A column's rank adds the popcounts before its word in the
// row (with 4 or more words per row, from a table of them, 16-bit, written
// by the row's owner) and the bits below it in its word.
template <int WG>
struct ColRanks {
    static_assert(WG <= 512, "one first rank per thread in Smem::tbase");
    u32* bm;        // the bitmap table: WG rows of `pitch` words
    uint16_t* pre;  // popcount of the row's words before each word (lp >= 2)
    u32 lp;         // log2 of the words per row
    u32 pitch;      // row pitch in words
    // The words of LDS needed for n columns.
    __device__ static __forceinline__ u32 plan(u32 n, u32& lp, u32& pitch) {
        const u32 words = (n + 31) / 32;
        lp = 0;
        while (((u32)WG << lp) < words) ++lp;
        pitch = lp ? (1u << lp) + 1u : 1u;
        const u32 tw = (u32)WG * pitch;
        return lp >= 2 ? tw + tw / 2 : tw;
    }
    __device__ ColRanks(u32* mem, u32 lp_, u32 pitch_)
        : bm(mem), pre(lp_ >= 2 ? (uint16_t*)(mem + (u32)WG * pitch_) : nullptr), lp(lp_), pitch(pitch_) {}
    __device__ u32 table_words() const { return (u32)WG * pitch; }
    __device__ void mark(u32 c) const {
        const u32 w = c >> 5;
        atomicOr(&bm[(w >> lp) * pitch + (w & ((1u << lp) - 1u))], 1u << (c & 31));
    }
    // Popcount of this thread's row (and, with 4 or more words, its prefix table).
    __device__ u32 row_count() const {
        const u32 r0 = threadIdx.x * pitch;
        if (lp == 0) return __popc(bm[r0]);
        if (lp == 1) return __popc(bm[r0]) + __popc(bm[r0 + 1]);
        const u32 per = 1u << lp;
        u32 s = 0;
        for (u32 j0 = 0; j0 < per; j0 += 4) {
            u32 x[4];
#pragma unroll
            for (u32 u = 0; u < 4; ++u) x[u] = bm[r0 + j0 + u];
#pragma unroll
            for (u32 u = 0; u < 4; ++u) {
                pre[r0 + j0 + u] = (uint16_t)s;
                s += __popc(x[u]);
            }
        }
        return s;
    }
    // Rank of selected column c, given each row's first rank in `base`.
    // Call after a barrier that follows row_count.
    __device__ u32 rank(u32 c, const u32* base) const {
        const u32 w = c >> 5, t = w >> lp, wj = w & ((1u << lp) - 1u), sl = t * pitch + wj;
        const u32 below = __popc(bm[sl] & ((1u << (c & 31)) - 1u));
        if (lp == 0) return base[t] + below;
        if (lp == 1) return base[t] + below + (wj ? __popc(bm[sl - 1]) : 0u);
        return base[t] + (u32)pre[sl] + below;
    }
};

// Writes the k entries of buf[0, k) in the order `sorted` asks for
// (0, kOrderIndex or kOrderValue).  Index order comes from a bitmap of the
// selected columns and a prefix popcount over it (when the row's bitmap
// fits in the free LDS), else from a bitonic sort; value order from ranks
// (sorted runs of one wave each and binary searches) when k fits one entry
// per thread, else from a bitonic sort of the composites in LDS.
template <class E, int WG, int CAP>
__device__ __noinline__ void emit(Smem<CAP>& sm, u32 k, u32 n, int sorted, int retval, int flags, gptr<void> out_idx_p,
                     gptr<void> out_val) {
    const IdxOut out_idx{out_idx_p, flags & kFlagIdx64};
    const u32 tid = threadIdx.x;
    using VT = typename std::conditional<E::kKeyBits == 16, uint16_t, uint32_t>::type;
    const gptr<VT> ov = (gptr<VT>)out_val;
    if (!sorted) {
        for (u32 i = tid; i < k; i += WG) {
            const u64 e = sm.buf[i];
            out_idx.put(i, comp_col<E>(e));
            if (retval) ov[i] = (VT)E::bits(comp_key<E>(e));
        }
        return;
    }
    u32 lp, pitch;
    const u32 need = ColRanks<WG>::plan(n, lp, pitch);
    if (sorted == kOrderIndex && !(flags & kFlagBitonic) && (u64)k * 2 + need <= (u64)CAP * 2) {
        const ColRanks<WG> cr((u32*)(sm.buf + k), lp, pitch);
        for (u32 w = tid; w < cr.table_words(); w += WG) cr.bm[w] = 0;
        __syncthreads();
        for (u32 i = tid; i < k; i += WG) cr.mark(comp_col<E>(sm.buf[i]));
        __syncthreads();
        u32 tot;
        sm.tbase[tid] = block_excl_scan<WG, CAP>(sm, cr.row_count(), &tot);
        __syncthreads();
        for (u32 i = tid; i < k; i += WG) {
            const u64 e = sm.buf[i];
            const u32 c = comp_col<E>(e);
            const u32 pos = cr.rank(c, sm.tbase);
            out_idx.put(pos, c);
            if (retval) ov[pos] = (VT)E::bits(comp_key<E>(e));
        }
        return;
    }
    if (sorted == kOrderValue && k <= (u32)WG) {
        // value order, one entry per thread.  The composites are distinct,
        // so an entry's output slot is the number of selected composites
        // above it.  Each wave first ranks its 64 entries among themselves
        // (lane broadcasts) and stores them in that order, as a descending
        // run; the count above an entry in every run (its own included) is
        // then a binary search of that run.  Threads past k hold 0, which
        // no composite equals and which sorts below all of them.
        const u32 wave = tid / kWave, l = lane_id();
        const u64 e = tid < k ? sm.buf[tid] : 0ull;
        const u32 elo = (u32)e, ehi = (u32)(e >> 32);
        u32 local = 0;
#pragma unroll
        for (int j = 0; j < kWave; ++j) {
            const u64 o = ((u64)(u32)__builtin_amdgcn_readlane((int)ehi, j) << 32) |
                          (u32)__builtin_amdgcn_readlane((int)elo, j);
            local += o > e ? 1u : 0u;
        }
        if (tid >= k) local = l;  // the zeros keep distinct slots behind the entries
        __syncthreads();          // every entry is read before the runs overwrite buf
        sm.buf[wave * kWave + local] = e;
        __syncthreads();
        u32 rank = 0;
#pragma unroll
        for (u32 w = 0; w < (u32)(WG / kWave); ++w) {
            const u64* run = sm.buf + w * kWave;
            u32 c = 0;
#pragma unroll
            for (u32 st = kWave / 2; st > 0; st >>= 1) c += run[c + st - 1] > e ? st : 0u;
            rank += c + (run[c] > e ? 1u : 0u);
        }
        __syncthreads();  // the runs are read; reorder through buf for coalesced stores
        if (tid < k) sm.buf[rank] = e;
        __syncthreads();
        if (tid < k) {
            const u64 s = sm.buf[tid];
            out_idx.put(tid, comp_col<E>(s));
            if (retval) ov[tid] = (VT)E::bits(comp_key<E>(s));
        }
        return;
    }
    // Bitonic sort, ascending, of (column, key) for index order, or of the
    // complemented composites for value order (largest composite first);
    // padding ~0 sorts last either way.
    u32 P = 1;
    while (P < k) P <<= 1;
    for (u32 i = tid; i < P; i += WG) {
        const u64 e = i < k ? sm.buf[i] : 0ull;
        sm.buf[i] = i >= k ? ~0ull : sorted == kOrderValue ? ~e : (((u64)comp_col<E>(e) << 32) | comp_key<E>(e));
    }
    __syncthreads();
    // Pair t of a stage is (i, i + stride) with i = 2t - (t mod stride); for
    // strides up to 64 the pairs of one wave's 64 t's lie in one block of
    // 128 entries, the same block at every such stage, and a wave's LDS
    // accesses take effect in order: only stages with a longer stride, and
    // their neighbours, need the workgroup barrier.
    for (u32 size = 2; size <= P; size <<= 1) {
        for (u32 stride = size >> 1; stride > 0; stride >>= 1) {
            for (u32 t = tid; t < P / 2; t += WG) {
                const u32 i = 2 * t - (t & (stride - 1));
                const u32 j = i + stride;
                const bool up = (i & size) == 0;
                const u64 x = sm.buf[i], y = sm.buf[j];
                if ((x > y) == up) {
                    sm.buf[i] = y;
                    sm.buf[j] = x;
                }
            }
            const u32 next = stride > 1 ? stride >> 1 : size;  // the next stage's stride
            if (stride > kWave || next > kWave) __syncthreads();
        }
    }
    __syncthreads();
    for (u32 i = tid; i < k; i += WG) {
        const u64 s = sm.buf[i];
        if (sorted == kOrderValue) {
            out_idx.put(i, comp_col<E>(~s));
            if (retval) ov[i] = (VT)E::bits(comp_key<E>(~s));
        } else {
            out_idx.put(i, (u32)(s >> 32));
            if (retval) ov[i] = (VT)E::bits((u32)s);
        }
    }
}

// ------------------------------------------------------------------ selection by threshold
__device__ __forceinline__ u64 low_mask(int b) { return b >= 64 ? ~0ull : ((1ull << b) - 1ull); }

// For ranks r0 and r1 (r >= 1; 0 = not wanted): the bin holding the r-th
// largest counted entry, as loc_digit, loc_r (rank inside the bin), loc_c
// (bin count; 0 when fewer than r are counted) and loc_above (entries in
// higher bins); also loc_total and loc_dhi (highest non-empty bin, 0 if
// none).  The whole workgroup takes part: thread t owns the kBins / WG bins
// just below kBins - t kBins / WG (descending bin order is thread order), a
// wave scan and one exchange of wave totals give every thread the entries in
// higher bins, and the thread whose bins hold rank r writes the result.
// Call from every thread; returns after a barrier, with the results visible
// to all.  With `zero` the histogram is cleared on the way.
template <int WG, int CAP, bool kPub = false>
__device__ __forceinline__ void block_locate(Smem<CAP>& sm, u32 r0, u32 r1, bool zero, gptr<u32> dir = nullptr) {
    constexpr u32 kPer = kBins / WG;
    constexpr u32 kW = WG / kWave;
    static_assert(kPer * WG == kBins && kW <= 16, "bins per thread");
    const u32 tid = threadIdx.x, wave = tid / kWave, l = lane_id();
    u32 c[kPer];
    u32 s = 0;
#pragma unroll
    for (u32 j = 0; j < kPer; ++j) {
        u32* h = &sm.hist[hidx(kBins - 1u - (tid * kPer + j))];
        c[j] = *h;
        s += c[j];
        if (zero) *h = 0;
    }
    const u32 incl = wave_incl_scan(s);
    const u64 nz = __ballot(s != 0);
    if (l == kWave - 1) sm.lwsum[wave] = incl;
    if (nz && l == (u32)__builtin_ctzll(nz)) {
        // this wave's highest non-empty bin
        u32 d = 0;
#pragma unroll
        for (int j = (int)kPer - 1; j >= 0; --j)
            if (c[j]) d = kBins - 1u - (tid * kPer + (u32)j);
        sm.lwfirst[wave] = d;
    }
    __syncthreads();
    u32 off = 0, tot = 0, fw = kW;
#pragma unroll
    for (u32 w = 0; w < kW; ++w) {
        const u32 v = sm.lwsum[w];
        off += w < wave ? v : 0u;
        tot += v;
        fw = (fw == kW && v != 0) ? w : fw;
    }
    const u32 dh = fw == kW ? 0u : sm.lwfirst[fw];
    const u32 excl = off + incl - s;  // entries in bins above this thread's
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const u32 r = q == 0 ? r0 : r1;
        if (r == 0) continue;
        if (r > tot) {
            if (tid == 0) {
                sm.loc_digit[q] = 0;
                sm.loc_r[q] = 0;
                sm.loc_c[q] = 0;
                sm.loc_above[q] = 0;
            }
        } else if (excl < r && r <= excl + s) {
            u32 above = excl;
#pragma unroll
            for (u32 j = 0; j < kPer; ++j) {
                if (above < r && r <= above + c[j]) {
                    sm.loc_digit[q] = kBins - 1u - (tid * kPer + j);
                    sm.loc_r[q] = r - above;
                    sm.loc_c[q] = c[j];
                    sm.loc_above[q] = above;
                }
                above += c[j];
            }
        }
    }
    if (tid == 0) {
        sm.loc_total = tot;
        sm.loc_dhi = dh;
    }
    if constexpr (kPub) {
        // Publishing: for every bin from the highest non-empty one down to
        // the bin of the r0-th entry, the directory entry (entries at or
        // above the bin) and, over the histogram, the bin's first slot in
        // the descending list.
        u32 above = excl;
#pragma unroll
        for (u32 j = 0; j < kPer; ++j) {
            const u32 d = kBins - 1u - (tid * kPer + j);
            if (d <= dh && above < r0) {
                sm.hist[hidx(d)] = above;
                st_agent(&dir[dh - d], above + c[j]);
            }
            above += c[j];
        }
    }
    __syncthreads();
}

// The rr-th largest of the (at most 64) entries of buf[0, cnt) whose bits
// under `mask` equal `prefix`.  Each wave counts its matches, reserves that
// many slots of sm.trash with one atomic and writes them there; then wave w
// compares every gathered entry with entries 8w .. 8w + 7 and adds the
// number of larger ones to the entry's rank.  side_count must be zero on
// entry; sm.seg_count[0, 64) is used for the ranks.
template <int WG, int CAP>
__device__ __forceinline__ u64 side_select(Smem<CAP>& sm, u32 cnt, u64 mask, u64 prefix, u32 rr) {
    static_assert(WG / kWave * 8 >= kWave, "eight entries compared per wave");
    const u32 tid = threadIdx.x, l = lane_id(), wave = tid / kWave;
    u32* const rank = sm.seg_count;
    // one pass, four loads in flight: a bit per matching entry of this thread
    // (entry tid + it WG for bit it; cnt <= CAP, so it < CAP / WG <= 32)
    static_assert(CAP / WG <= 32, "one flag bit per entry of a thread");
    u32 bits = 0, mine = 0;
    for (u32 b0 = 0; b0 < cnt; b0 += 4 * WG) {
        u64 e[4];
#pragma unroll
        for (u32 u = 0; u < 4; ++u) {
            const u32 i = b0 + u * WG + tid;
            e[u] = i < cnt ? sm.buf[i] : 0ull;
        }
#pragma unroll
        for (u32 u = 0; u < 4; ++u) {
            const u32 i = b0 + u * WG + tid;
            const bool in = i < cnt && (e[u] & mask) == prefix;
            bits |= (in ? 1u : 0u) << (b0 / WG + u);
            mine += (u32)__popcll(__ballot(in));
        }
    }
    if (tid < kWave) rank[tid] = 0;
    if (mine) {
        u32 base = 0;
        if (l == 0) base = atomicAdd(&sm.side_count, mine);
        base = __builtin_amdgcn_readfirstlane(base);
        for (u32 it = 0; it * WG < cnt; ++it) {
            const bool in = (bits >> it) & 1u;
            const u64 m = __ballot(in);
            if (!m) continue;
            const u32 slot = base + mbcnt(m);
            if (in && slot < (u32)kWave) sm.trash[slot] = sm.buf[it * WG + tid];  // (at most 64 match)
            base += (u32)__popcll(m);
        }
    }
    __syncthreads();
    const u32 c = min(__builtin_amdgcn_readfirstlane(sm.side_count), (u32)kWave);
    const u64 x = l < c ? sm.trash[l] : 0ull;
    u32 above = 0;  // gathered entries larger than this lane's, among this wave's eight
#pragma unroll
    for (u32 q = 0; q < 8; ++q) {
        const u32 j = wave * 8 + q;
        above += (j < c && sm.trash[j] > x) ? 1u : 0u;
    }
    if (l < c && above) atomicAdd(&rank[l], above);
    __syncthreads();
    const u64 hit = __ballot(l < c && rank[l] == rr - 1);  // one lane: the entries are distinct
    const u32 hl = hit ? (u32)__builtin_ctzll(hit) : 0u;
    return ((u64)(u32)__builtin_amdgcn_readlane((u32)(x >> 32), hl) << 32) |
           (u32)__builtin_amdgcn_readlane((u32)x, hl);
}

// The rr-th largest of the c entries of a first-level sub-bin, found by
// walking the sub-bin's chain: head[d] is the last of its entries to be
// counted, next[i] the one counted before entry i (the first one's link is
// never followed).  One lane walks it into sm.trash, the wave ranks the c
// entries (a wave's LDS accesses take effect in order); the result is
// shared through LDS.  Call from every thread.
template <int WG, int CAP>
__device__ __forceinline__ u64 chain_select(Smem<CAP>& sm, const u32* head, const u32* next, u32 d, u32 c, u32 rr) {
    const u32 l = lane_id();
    if (threadIdx.x < (u32)kWave) {
        if (l == 0) {
            u32 i = head[d];
            for (u32 j = 0; j < c; ++j) {
                sm.trash[j] = sm.buf[i];
                if (j + 1 < c) i = next[i];
            }
        }
        const u64 x = l < c ? sm.trash[l] : 0ull;
        u32 above = 0;
        for (u32 q = 0; q < c; ++q) above += sm.trash[q] > x ? 1u : 0u;
        const u64 hit = __ballot(l < c && above == rr - 1);  // one lane: the entries are distinct
        if (hit && l == (u32)__builtin_ctzll(hit)) sm.chain_t = x;
    }
    __syncthreads();
    return sm.chain_t;
}

// A sub-bin this small is settled by side_select rather than another radix
// level (measured: with more entries, the gather and the ranking cost more
// than a level).
constexpr u32 kSideMax = 16;

// The threshold T with exactly k entries of buf[0, cnt) at or above it,
// given the top-digit bin b1 that holds the k-th largest entry, the rank r1
// inside it and its size c1.  Radix refinement inside the bin with 11-bit
// digits made only of bits where the bin's entries still differ (taken
// from their OR and AND): the highest run of such bits and, when it is
// shorter than 11, the next such bits below it, so runs of bits shared by
// all of them (equal values, the high bits of small column numbers) cost
// no level.  With a fixed first level the digit's bits are known in advance
// and it is counted in the same pass that gathers the OR and AND (for the
// levels that may follow): kFirst 1, 32-bit keys, whose 11 bits below the
// top digit seldom tie: those bits; kFirst 2, 16-bit keys (composite = key
// << 48 | ~column << 16, columns below 2^cb): the key's 5 bits below the top
// digit and the column's highest min(6, cb) bits, the bits between them
// being ones for every such column.  A sub-bin of at most kSideMax entries
// that still holds the k-th is settled directly by side_select (with
// 16-bit keys the first digit already takes high column bits below the
// value's, so a tied value's entries spread over many sub-bins).  The
// histogram must be zero on entry and is zero again on return.
// The fixed first refine level (kFirst 1: 32-bit keys, kFirst 2: 16-bit
// keys; see refine) for buf[0, cnt): an entry of the k-th entry's bin is
// counted by its digit, gathered into the OR / AND of the bin, and chained
// into its sub-bin.  With a fixed first level, the entries of each sub-bin
// are chained (heads and links in the free buffer behind the entries, when
// they fit), so a small sub-bin holding the k-th is ranked by one wave
// without another pass (chain_select).  Not in the k > 1024 kernels: there
// the k-th entry's bin can hold thousands of tied entries, whose returning
// atomics cost more than the pass they save (256 x 32768, k = 4096, 16
// levels: +1.4 us).
template <int kFirst, int CAP>
struct FirstLevel {
    static constexpr int kSh1 = 64 - 2 * kHistBits;
    u32 len2;  // kFirst 2: the column part's length and position
    int csh;
    bool chain;
    u32* head;
    u32* next;
    __device__ __forceinline__ FirstLevel(Smem<CAP>& sm, u32 cnt, u32 cb)
        : len2(cb < 6u ? cb : 6u), csh(16 + (int)cb - (int)(cb < 6u ? cb : 6u)),
          chain(kFirst != 0 && CAP == 8192 && (u64)cnt * 12u + (u64)kBins * 4u <= (u64)CAP * 8u),
          head((u32*)(sm.buf + cnt)), next((u32*)(sm.buf + cnt) + kBins) {}
    __device__ __forceinline__ u32 digit(u64 e) const {
        if constexpr (kFirst == 1) return (u32)(e >> kSh1) & (kBins - 1);
        return (((u32)(e >> 48) & 31u) << len2) | ((u32)(e >> csh) & ((1u << len2) - 1u));
    }
    // entry i (= e) of the bin
    __device__ __forceinline__ void add(Smem<CAP>& sm, u64 e, u32 i, u64& o, u64& a) const {
        o |= e;
        a &= e;
        if constexpr (kFirst != 0) {
            const u32 d = digit(e);
            atomicAdd(&sm.hist[hidx(d)], 1u);
            if (chain) next[i] = atomicExch(&head[d], i);
        }
    }
};

// kCounted: the caller has already passed every entry of bin b1 through
// FirstLevel::add (the merge does it while loading), and o, a are its
// thread's OR and AND.
template <int WG, int CAP, int kFirst = 0, bool kCounted = false>
__device__ __forceinline__ u64 refine(Smem<CAP>& sm, u32 cnt, u32 b1, u32 r1, u32 c1, u32 cb = 0, u64 o0 = 0,
                                      u64 a0 = ~0ull) {
    const u32 tid = threadIdx.x, wave = tid / kWave;
    if (r1 >= c1) {  // the whole bin is kept
        if constexpr (kCounted) {
            __syncthreads();
            for (u32 i = tid; i < (u32)kHistWords; i += WG) sm.hist[i] = 0;
            __syncthreads();
        }
        return digit_floor(b1);
    }
    constexpr int kTop = 64 - kHistBits;
    constexpr int kSh1 = kTop - kHistBits;
    if (tid == 0) sm.side_count = 0;  // (read after the barriers below)
    u64 P = digit_floor(b1);  // bits of T fixed so far: those at or above `fixed`
    int fixed = kTop;
    u32 r = r1;
    u64 o = o0, a = a0;
    const FirstLevel<kFirst, CAP> fl(sm, cnt, cb);
    const u32 len2 = fl.len2;
    const int csh = fl.csh;
    const bool chain = fl.chain;
    u32* const head = fl.head;
    u32* const next = fl.next;
    if constexpr (!kCounted) {
        for (u32 i = tid; i < cnt; i += WG) {
            const u64 e = sm.buf[i];
            if (top_digit(e) == b1) fl.add(sm, e, i, o, a);
        }
    }
    if constexpr (kFirst == 1) {
        __syncthreads();
        block_locate<WG, CAP>(sm, r1, 0u, true);
        P |= (u64)sm.loc_digit[0] << kSh1;
        fixed = kSh1;
        r = sm.loc_r[0];
        if (r >= sm.loc_c[0]) return P;  // the whole sub-bin is kept: T is its least possible key
        if (sm.loc_c[0] <= kSideMax) {
            if (chain) return chain_select<WG, CAP>(sm, head, next, sm.loc_digit[0], sm.loc_c[0], r);
            return side_select<WG, CAP>(sm, cnt, ~low_mask(kSh1), P, r);
        }
    }
    if constexpr (kFirst == 2) {
        __syncthreads();
        block_locate<WG, CAP>(sm, r1, 0u, true);
        const u32 d = sm.loc_digit[0];
        P |= ((u64)(d >> len2) << 48) | ((u64)(d & ((1u << len2) - 1u)) << csh) |
             (low_mask(48) & ~low_mask(16 + (int)cb));
        fixed = csh;
        r = sm.loc_r[0];
        if (r >= sm.loc_c[0]) return P;  // the whole sub-bin is kept: T is its least possible key
        if (sm.loc_c[0] <= kSideMax) {
            if (chain) return chain_select<WG, CAP>(sm, head, next, d, sm.loc_c[0], r);
            return side_select<WG, CAP>(sm, cnt, ~low_mask(csh), P, r);
        }
    }
    {
        const u32 ohi = wave_or((u32)(o >> 32)), olo = wave_or((u32)o);
        const u32 ahi = wave_and((u32)(a >> 32)), alo = wave_and((u32)a);
        if (lane_id() == 0) {
            sm.red[wave][0] = ((u64)ohi << 32) | olo;
            sm.red[wave][1] = ((u64)ahi << 32) | alo;
        }
    }
    __syncthreads();
    u64 O = 0, A = ~0ull;
#pragma unroll
    for (u32 w = 0; w < WG / kWave; ++w) {
        O |= sm.red[w][0];
        A &= sm.red[w][1];
    }
    u64 D = (O ^ A) & low_mask(fixed);  // bits below those fixed where entries of the bin differ
    for (int level = 0; level < 64 / kHistBits + 2; ++level) {
        // D != 0 here: the remaining set has at least two (distinct) entries
        const int hb = 63 - __clzll((long long)D);
        P |= A & (low_mask(fixed) & ~low_mask(hb + 1));  // bits shared by the whole set
        const u64 pm = ~low_mask(hb + 1);
        // The digit: D's run of set bits from hb down (at most 11 bits,
        // [lo1, hb]) and, when that is shorter, the highest bits of D below
        // it ([sh2, hb2]); the bits between are shared by the whole set, so
        // the digit orders the set like the composites do.
        const u64 z = ~D & low_mask(hb + 1);
        int lo1 = z ? 64 - __clzll((long long)z) : 0;
        lo1 = lo1 > hb - (kHistBits - 1) ? lo1 : hb - (kHistBits - 1);
        const int len1 = hb - lo1 + 1;
        const u64 D2 = D & low_mask(lo1);
        int len2 = 0, hb2 = lo1 - 1;
        if (len1 < kHistBits && D2) {
            hb2 = 63 - __clzll((long long)D2);
            len2 = kHistBits - len1 < hb2 + 1 ? kHistBits - len1 : hb2 + 1;
        }
        if (len2 == 0) {  // one part: 11 bits from hb down
            lo1 = hb >= kHistBits - 1 ? hb - (kHistBits - 1) : 0;
            hb2 = lo1 - 1;
        }
        const int sh2 = hb2 - len2 + 1;  // (= lo1 with one part)
        if (len2 == 0) {
            for (u32 i = tid; i < cnt; i += WG) {
                const u64 e = sm.buf[i];
                if ((e & pm) == P) atomicAdd(&sm.hist[hidx((u32)(e >> lo1) & (kBins - 1))], 1u);
            }
        } else {
            const u64 m1 = low_mask(len1), m2 = low_mask(len2);
            for (u32 i = tid; i < cnt; i += WG) {
                const u64 e = sm.buf[i];
                if ((e & pm) == P) atomicAdd(&sm.hist[hidx((u32)((((e >> lo1) & m1) << len2) | ((e >> sh2) & m2)))], 1u);
            }
        }
        __syncthreads();
        block_locate<WG, CAP>(sm, r, 0u, true);
        const u32 d = sm.loc_digit[0], rr = sm.loc_r[0], c = sm.loc_c[0];
        P |= ((u64)(d >> len2) << lo1) | ((u64)(d & (u32)low_mask(len2)) << sh2);
        P |= A & (low_mask(lo1) & ~low_mask(hb2 + 1));  // the shared bits between the two parts
        fixed = sh2;
        if (rr >= c) return P;  // the whole sub-bin is kept: T is its least possible key
        if (c <= kSideMax && (kFirst != 0 || cnt <= 4096u))
            return side_select<WG, CAP>(sm, cnt, ~low_mask(sh2), P, rr);
        r = rr;
        D &= low_mask(sh2);
    }
    return P;
}

// Compact the entries >= T to buf[0, k) and write them with emit() (index
// order by a bitmap behind them, or a bitonic sort).
template <class E, int WG, int CAP>
__device__ __noinline__ void emit_compacted(Smem<CAP>& sm, u32 cnt, u64 T, u32 k, u32 n, int sorted, int retval,
                                            int flags, gptr<void> out_idx_p, gptr<void> out_val) {
    const IdxOut out_idx{out_idx_p, flags & kFlagIdx64};
    __syncthreads();
    keep_at_least<WG, CAP>(sm, 0, cnt, T);
    emit<E, WG, CAP>(sm, k, n, sorted, retval, flags, out_idx.p, out_val);
}

// Reduce buf[0, cnt) exactly to its k largest (b1/r1/c1 locate the k-th in
// the histogram), rebuild the histogram and locate ranks k and q again.
// Returns the new count; sm.kth gets the k-th entry.
template <int WG, int CAP, bool kPub = false>
__device__ __noinline__ u32 reduce_to_k(Smem<CAP>& sm, u32 cnt, u32 k, u32 q, u32 b1, u32 r1, u32 c1,
                                        gptr<u32> dir = nullptr) {
    const u32 tid = threadIdx.x;
    __syncthreads();
    for (u32 i = tid; i < (u32)kHistWords; i += WG) sm.hist[i] = 0;
    __syncthreads();
    const u64 T = refine<WG, CAP>(sm, cnt, b1, r1, c1);
    __syncthreads();
    cnt = keep_at_least<WG, CAP>(sm, 0, cnt, T);
    if (tid == 0) sm.kth = T;
    rebuild_hist<WG, CAP>(sm, cnt);
    block_locate<WG, CAP, kPub>(sm, k, q, false, dir);
    return cnt;
}

// Write the k entries of buf[0, cnt) that are >= T.  Unordered: one slot
// reservation per wave.  Index order: a bitmap of the selected columns (in
// the free histogram, or behind the entries) and a prefix popcount over it;
// when no bitmap fits, compact and fall back to emit().
template <class E, int WG, int CAP>
__device__ __forceinline__ void emit_threshold(Smem<CAP>& sm, u32 cnt, u64 T, u32 k, u32 n, int sorted, int retval,
                                               int flags, IdxOut out_idx, gptr<void> out_val) {
    const u32 tid = threadIdx.x;
    using VT = typename std::conditional<E::kKeyBits == 16, uint16_t, uint32_t>::type;
    const gptr<VT> ov = (gptr<VT>)out_val;
    if (!sorted) {
        u32 mine = 0;
        for (u32 i = tid; i < cnt; i += WG) mine += sm.buf[i] >= T ? 1u : 0u;
        u32 pos = wave_reserve(&sm.outcount, mine);
        if (mine == 0) return;
        for (u32 i = tid; i < cnt; i += WG) {
            const u64 e = sm.buf[i];
            if (e >= T) {
                if (pos < k) {
                    out_idx.put(pos, comp_col<E>(e));
                    if (retval) ov[pos] = (VT)E::bits(comp_key<E>(e));
                }
                ++pos;
            }
        }
        return;
    }
    u32 lp, pitch;
    const u32 need = ColRanks<WG>::plan(n, lp, pitch);
    u32* bm = nullptr;
    if (sorted == kOrderIndex && !(flags & kFlagBitonic)) {
        if (need <= (u32)kHistWords) bm = sm.hist;
        else if ((u64)cnt * 2 + need <= (u64)CAP * 2) bm = (u32*)(sm.buf + cnt);
    }
    if (!bm) {
        emit_compacted<E, WG, CAP>(sm, cnt, T, k, n, sorted, retval, flags, out_idx.p, out_val);
        return;
    }
    const ColRanks<WG> cr(bm, lp, pitch);
    if (bm == sm.hist) __syncthreads();  // the histogram may still be read by the last locate
    for (u32 w = tid; w < cr.table_words(); w += WG) bm[w] = 0;
    __syncthreads();
    for (u32 i = tid; i < cnt; i += WG) {
        const u64 e = sm.buf[i];
        if (e >= T) cr.mark(comp_col<E>(e));
    }
    __syncthreads();
    u32 tot;
    sm.tbase[tid] = block_excl_scan<WG, CAP>(sm, cr.row_count(), &tot);
    __syncthreads();
    for (u32 i = tid; i < cnt; i += WG) {
        const u64 e = sm.buf[i];
        if (e >= T) {
            const u32 c = comp_col<E>(e);
            const u32 pos = cr.rank(c, sm.tbase);
            if (pos < k) {
                out_idx.put(pos, c);
                if (retval) ov[pos] = (VT)E::bits(comp_key<E>(e));
            }
        }
    }
}

// ------------------------------------------------------------------ scan helpers
// While scanning, buf[0, cbase) holds composites, counted in the histogram,
// and the rest is split into one region of R entries per wave, where each
// wave appends raw entries (element bits << 32 | column); wfill[w] counts
// wave w's.  sync_regions moves them behind the composites, converting and
// counting them with every lane busy, and returns the new count.  Entry j of
// the regions' concatenation goes to cbase + j, at or below where it is,
// and each batch is read before it is written, so nothing is overwritten
// before it has been read.  A NaN sets sm.nan.  Call after a barrier that
// follows every wave's last append and wfill store.
template <class E, int WG, int CAP>
__device__ __forceinline__ u32 sync_regions(Smem<CAP>& sm, u32 cbase, u32 R) {
    constexpr u32 kWaves = WG / kWave;
    const u32 tid = threadIdx.x;
    // Entry j of the concatenation lies at cbase + j plus the unused tails
    // of the regions before its own: gap[q] = R - fill[q - 1] is added for
    // every region start off[q] at or below j.
    u32 off[kWaves], gap[kWaves], N = 0;
#pragma unroll
    for (u32 w = 0; w < kWaves; ++w) {
        const u32 f = __builtin_amdgcn_readfirstlane(sm.wfill[w]);
        off[w] = N;
        gap[w] = w ? R - __builtin_amdgcn_readfirstlane(sm.wfill[w - 1]) : 0u;
        N += f;
    }
    bool nan = false;
    constexpr u32 kB = 8;  // entries per thread and batch: one batch for most syncs
    for (u32 base = 0; base < N; base += WG * kB) {
        u64 e[kB];
        u32 src[kB];
#pragma unroll
        for (u32 i = 0; i < kB; ++i) {
            const u32 j = min(base + i * WG + tid, N - 1u);
            u32 a = cbase + j;
#pragma unroll
            for (u32 q = 1; q < kWaves; ++q) a += j >= off[q] ? gap[q] : 0u;
            src[i] = a;
        }
#pragma unroll
        for (u32 i = 0; i < kB; ++i) e[i] = sm.buf[src[i]];
#pragma unroll
        for (u32 i = 0; i < kB; ++i) {
            const u32 bits = (u32)(e[i] >> 32);
            nan |= base + i * WG + tid < N && E::is_nan(bits);
            e[i] = compose<E>(E::key(bits), (u32)e[i]);
        }
        __syncthreads();
#pragma unroll
        for (u32 i = 0; i < kB; ++i) {
            const u32 j = base + i * WG + tid;
            if (j < N) sm.buf[cbase + j] = e[i];
            hist_add(sm.hist, top_digit(e[i]), j < N);
        }
        __syncthreads();
    }
    if (nan) sm.nan = 1;  // benign race: every writer stores 1
    return cbase + N;
}

// Where entry j of the scan's buffer lies when the regions have not been
// moved together: below cbase at j, past it behind the unused tails of the
// regions before its own (see sync_regions).
template <int WG>
struct RegionMap {
    static constexpr u32 kWaves = WG / kWave;
    u32 cbase, total;
    u32 off[kWaves], gap[kWaves];
    template <int CAP>
    __device__ __forceinline__ RegionMap(const Smem<CAP>& sm, u32 cb, u32 R) : cbase(cb) {
        u32 N = 0;
#pragma unroll
        for (u32 w = 0; w < kWaves; ++w) {
            off[w] = N;
            gap[w] = w ? R - __builtin_amdgcn_readfirstlane(sm.wfill[w - 1]) : 0u;
            N += __builtin_amdgcn_readfirstlane(sm.wfill[w]);
        }
        total = cb + N;
    }
    __device__ __forceinline__ u32 addr(u32 j) const {
        if (j < cbase) return j;
        const u32 r = j - cbase;
        u32 a = j;
#pragma unroll
        for (u32 q = 1; q < kWaves; ++q) a += r >= off[q] ? gap[q] : 0u;
        return a;
    }
};

// Moves the (converted, counted) entries of the regions together behind
// cbase, in batches each read before it is written (see sync_regions);
// returns the count.  Returns after a barrier.
template <int WG, int CAP>
__device__ __forceinline__ u32 move_regions(Smem<CAP>& sm, const RegionMap<WG>& map) {
    const u32 tid = threadIdx.x;
    constexpr u32 kB = 8;
    for (u32 base = map.cbase; base < map.total; base += WG * kB) {
        u64 e[kB];
#pragma unroll
        for (u32 i = 0; i < kB; ++i) {
            const u32 j = base + i * WG + tid;
            e[i] = j < map.total ? sm.buf[map.addr(j)] : 0ull;
        }
        __syncthreads();
#pragma unroll
        for (u32 i = 0; i < kB; ++i) {
            const u32 j = base + i * WG + tid;
            if (j < map.total) sm.buf[j] = e[i];
        }
        __syncthreads();
    }
    return map.total;
}

// Converts the regions' raw entries to composites where they lie and counts
// them (the split-row end of scan, which publishes from there; the regions
// are not moved together).  Each wave converts its own region.  A NaN sets
// sm.nan.  Call after a barrier that follows every wave's last append and
// wfill store; returns after a barrier.
template <class E, int WG, int CAP>
__device__ __forceinline__ void convert_regions(Smem<CAP>& sm, u32 cbase, u32 R) {
    const u32 wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const u32 fill = __builtin_amdgcn_readfirstlane(sm.wfill[wave]);
    const u32 rb = cbase + wave * R;
    bool nan = false;
    constexpr u32 kU = 4;  // entries in flight per lane
    for (u32 i0 = 0; i0 < fill; i0 += kU * kWave) {
        u64 e[kU];
#pragma unroll
        for (u32 u = 0; u < kU; ++u) {
            const u32 i = i0 + u * kWave + lane_id();
            e[u] = i < fill ? sm.buf[rb + i] : 0ull;
        }
#pragma unroll
        for (u32 u = 0; u < kU; ++u) {
            const u32 i = i0 + u * kWave + lane_id();
            const u32 bits = (u32)(e[u] >> 32);
            nan |= i < fill && E::is_nan(bits);
            e[u] = compose<E>(E::key(bits), (u32)e[u]);
            if (i < fill) sm.buf[rb + i] = e[u];
            hist_add(sm.hist, top_digit(e[u]), i < fill);
        }
    }
    if (nan) sm.nan = 1;  // benign race: every writer stores 1
    __syncthreads();
}

// After a sync of cnt composites: make room when the buffer is short of
// `room` entries (room 0: when it is more than half full), then locate the
// k-th counted entry and return the bound raised to its bin edge (and to
// sm.L, which make_room may have raised); sm.count holds the new count.
// Returns after a barrier.
template <class E, int WG, int CAP>
__device__ __forceinline__ u64 raise_bound(Smem<CAP>& sm, u32 cnt, u32 room, u32 k, u64 L) {
    if (room ? cnt > (u32)CAP - room : (cnt > (u32)CAP / 2 && cnt > k)) {
        make_room<E, WG, CAP>(sm, cnt, k, room);
    } else {
        if (threadIdx.x == 0) sm.count = cnt;
    }
    block_locate<WG, CAP>(sm, k, 0u, false);
    if (sm.loc_c[0] > 0 && digit_floor(sm.loc_digit[0]) > L) L = digit_floor(sm.loc_digit[0]);
    if (sm.L > L) L = sm.L;
    return L;
}

// ------------------------------------------------------------------ scan: admission
// One segment's scan, per workgroup.  The state a wave carries from chunk to
// chunk (all wave-uniform but `nan`).
struct ScanState {
    u64 L;      // admission bound: admit iff composite >= L
    u32 cbase;  // buf[0, cbase) holds counted composites
    u32 R;      // entries per wave region behind them
    u32 wp;     // this wave's write pointer ...
    u32 re;     // ... and region end
    u32 par;    // slot of sm.pflag used by the next check
    u32 exact;  // also test survivors against the composite bound
    u32 nan;    // per lane: a NaN met by the exact test
};
// What a scan reads but never changes.
struct ScanCtx {
    __amdgpu_buffer_rsrc_t rsrc;  // the segment; offset (vi - v0) * 16
    int v0, v1;                   // vectors [v0, v1) of the row
    u32 n, k;
};

template <int WG, int CAP>
__device__ __forceinline__ void assign_regions(ScanState& st, u32 cnt) {
    constexpr u32 kWaves = WG / kWave;
    st.cbase = cnt;
    st.R = ((u32)CAP - cnt) / kWaves;
    st.wp = cnt + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave) * st.R;
    st.re = st.wp + st.R;
}

// Appends the survivors of one tile (vector vb + thread of the row) to the
// wave's region: one ballot per element slot gives them as scalar masks,
// so every branch is on a scalar, and every lane writes, with no branch or
// exec mask per slot: a survivor to its place behind the write pointer, any
// other lane to its own word of a scratch row.  In exact mode the survivors
// are also tested against the composite bound, so long runs of values equal
// to the bound's value cannot refill the buffer.  Returns false (nothing
// appended) when they do not fit.
template <class E, int WG, int CAP>
__device__ __forceinline__ bool append_tile(Smem<CAP>& sm, const ScanCtx& cx, ScanState& st, const PreFilter<E>& pf,
                                            const u32x4& x, int vb) {
    constexpr int P = E::kPerVec;
    constexpr int kTileVecs = WG;
    const u32 dw[4] = {x[0], x[1], x[2], x[3]};
    const u32 vi = (u32)(vb + (int)threadIdx.x);
    // With an exact bound, a tile whose columns all lie above the bound's
    // can only add values strictly above the bound's value (a tie there has
    // the smaller composite): filter on the next value up, and skip the
    // composite test.  (Not for a zero or +inf bound value: -0 and +0 are
    // equal as floats but not here, and nothing lies above +inf.)
    // (bf16 only, with the tied seed bound; see kTiedSeed)
    bool strict = false;
    PreFilter<E> q = pf;
    if constexpr (E::kKeyBits == 16) {
        strict = st.exact && pf.strict_ok && (u32)vb * (u32)P > comp_col<E>(st.L);
        if (strict) q.t = pf.ts;
    }
    u64 m[P];
    u64 any = 0;
    static_for<P>([&](auto S_) {
        constexpr int s = decltype(S_)::value;
        m[s] = __ballot(pass_slot<s>(q, dw));
        any |= m[s];
    });
    if (any == 0) return true;
    if (!(vb + kTileVecs <= cx.v1 && (u32)(vb + kTileVecs) * P <= cx.n)) {
        // the tile runs past the valid columns
        static_for<P>([&](auto S_) {
            constexpr int s = decltype(S_)::value;
            m[s] &= __ballot((int)vi < cx.v1 && vi * P + s < cx.n);
        });
    }
    if (st.exact && !strict) {
        static_for<P>([&](auto S_) {
            constexpr int s = decltype(S_)::value;
            if (m[s]) {
                // (a NaN passes the pre-filter; note it before the exact test)
                st.nan |= (((m[s] >> lane_id()) & 1u) && nan_slot<s>(E{}, dw)) ? 1u : 0u;
                m[s] &= __ballot(compose<E>(E::key(slot_bits<s>(E{}, dw)), vi * P + s) >= st.L);
            }
        });
    }
    u32 tot = 0;
    static_for<P>([&](auto S_) { tot += (u32)__popcll(m[decltype(S_)::value]); });
    if (st.wp + tot > st.re) return false;
    // (the element bits go into the store's register pair as a fresh copy,
    // so the loaded vectors stay where the loads put them)
    u64* const trash = &sm.trash[lane_id()];
    static_for<P>([&](auto S_) {
        constexpr int s = decltype(S_)::value;
        u64* const dst = __builtin_amdgcn_inverse_ballot_w64(m[s]) ? &sm.buf[mbcnt_from(m[s], st.wp)] : trash;
        *dst = ((u64)fresh_copy(slot_bits<s>(E{}, dw)) << 32) | (vi * P + s);
        st.wp += (u32)__popcll(m[s]);
    });
    return true;
}

// Appends tiles from..NV-1 of a chunk (constant register indices); returns
// the first tile that did not fit, or NV.
template <class E, int WG, int NV, int CAP>
__device__ __forceinline__ u32 append_chunk(Smem<CAP>& sm, const ScanCtx& cx, ScanState& st, const PreFilter<E>& pf,
                                            const u32x4 (&v)[NV], const int (&vb)[NV], u32 from) {
    u32 stop = (u32)NV;
    static_for<NV>([&](auto I_) {
        constexpr int i = decltype(I_)::value;
        if (stop == (u32)NV && (u32)i >= from && !append_tile<E, WG, CAP>(sm, cx, st, pf, v[i], vb[i]))
            stop = (u32)i;
    });
    return stop;
}

// "Is any wave left with tiles?" in one barrier: slot par collects the
// answer; the other slot, last read before an earlier barrier, is cleared
// for the next check.  The barrier also follows every wave's last append
// and fill note, as a sync needs.
template <int WG, int CAP>
__device__ __forceinline__ bool check_pending(Smem<CAP>& sm, ScanState& st, bool pending) {
    constexpr u32 kWaves = WG / kWave;
    const u32 wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (lane_id() == 0) {
        if (pending) atomicOr(&sm.pflag[st.par], 1u);
        sm.wfill[wave] = st.wp - (st.cbase + wave * st.R);
    }
    if (threadIdx.x == 0) sm.pflag[st.par ^ 1u] = 0;
    __syncthreads();
    const bool again = sm.pflag[st.par] != 0;
    st.par ^= 1u;
    (void)kWaves;
    return again;
}

// The rare step after a chunk: a region filled up (again), or a scheduled
// raise.  Sync; make room if the buffer is short of a whole tile of the
// workgroup, raise the bound; with tiles left, reload them (from the cache)
// and append them, and repeat.  With that much room every region holds one
// wave's tile, so each round appends at least one tile of every waiting
// wave, and at most NV + 1 rounds are taken.
template <class E, int WG, int NV, int CAP>
__device__ __forceinline__ ScanState rare_rounds(Smem<CAP>& sm, ScanCtx cx, ScanState st, VecBases<NV> vb, u32 rtile,
                                              bool again) {
    constexpr u32 kTileElems = WG * E::kPerVec;
    for (u32 round = 0;; ++round) {
        if (round > (u32)NV) {  // unreachable: the room argument above
            st.nan = 1;  // reported as an invalid result, never silently
            break;
        }
        const u32 cnt = sync_regions<E, WG, CAP>(sm, st.cbase, st.R);
        st.L = raise_bound<E, WG, CAP>(sm, cnt, again ? kTileElems : 0u, cx.k, st.L);
        st.exact |= again ? 1u : 0u;
        assign_regions<WG, CAP>(st, __builtin_amdgcn_readfirstlane(sm.count));
        if (!again) break;
        PreFilter<E> pf;
        pf.set(st.L);
        u32x4 w[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i)
            w[i] = __builtin_amdgcn_raw_buffer_load_b128(cx.rsrc, (u32)(vb.b[i] + (int)threadIdx.x - cx.v0) * 16u, 0, 0);
        rtile = append_chunk<E, WG, NV, CAP>(sm, cx, st, pf, w, vb.b, rtile);
        again = check_pending<WG, CAP>(sm, st, rtile < (u32)NV);
        if (!again) break;
    }
    return st;
}

// ------------------------------------------------------------------ kernel
struct Params {
    const uint8_t* in;
    int64_t row_stride_bytes;
    int32_t n;
    int32_t k;
    int32_t segs;      // workgroups per row
    int32_t seg_vecs;  // 16-byte vectors per segment
    int32_t n_vec;     // 16-byte vectors per row holding valid columns
    uint32_t seed;
    int32_t sorted;    // output order: 0, kOrderIndex or kOrderValue
    int32_t retval;
    void* out_idx;     // [batch][k] int32, or int64 with kFlagIdx64
    void* out_val;
    u64* ws_cand;      // [batch][segs][pub_cap]: a segment's live candidates, by top digit
    u64* ws_meta;      // [batch][segs][4]: count | low digit, high digit, bound, q-bound
    u32* ws_dir;       // [batch][segs][kBins]: entries with top digit >= d, from the low digit
    u32* ws_ticket;    // [batch], zero between calls
    int32_t pub_cap;   // most candidates a segment publishes
    int32_t* flag;     // set to flag_value when a NaN is seen
    int32_t flag_value;
    int32_t flags;     // kFlag* bits
    const int32_t* lengths;  // [batch] valid columns per row (clamped to [0, n]), or null: all n
    u64* timing;       // measurement build: [grid][kTimingSlots] phase timestamps; else unused
    // the sampling instance (topk_sample_rows) only: per row temperature,
    // top-p and a uniform, and the token drawn
    const float* temperature;
    const float* top_p;
    const float* uniform;
    int32_t* out_token;
};

// Output slots [k, kout) of a row with only k = len < kout valid columns:
// the columns len .. kout - 1, which act as -inf (they come after every
// valid entry in each order), with -inf values.
template <class E, int WG>
__device__ __forceinline__ void write_tail(IdxOut row_idx, gptr<void> row_val, u32 k, u32 kout) {
    using VT = typename std::conditional<E::kKeyBits == 16, uint16_t, uint32_t>::type;
    constexpr VT kNegInf = E::kKeyBits == 16 ? (VT)0xFF80u : (VT)0xFF800000u;
    for (u32 j = k + threadIdx.x; j < kout; j += WG) {
        row_idx.put(j, j);
        if (row_val) ((gptr<VT>)row_val)[j] = kNegInf;
    }
}

__device__ __forceinline__ u32 hash32(u32 x) {
    x ^= x >> 16;
    x *= 0x7FEB352Du;
    x ^= x >> 15;
    x *= 0x846CA68Bu;
    x ^= x >> 16;
    return x;
}

__device__ __forceinline__ u32 gcd_u32(u32 a, u32 b) {
    while (b) {
        const u32 t = a % b;
        a = b;
        b = t;
    }
    return a;
}

// Element slot s of a thread's tile registers: (raw bits, column, valid).
template <class E, int VPT, int WG>
struct Slot {
    static constexpr int kSlots = VPT * E::kPerVec;
    static constexpr int kPerDword = E::kKeyBits == 16 ? 2 : 1;
    __device__ static __forceinline__ void get(const u32x4 (&v)[VPT], int s, int vb, u32 tid, int v1, u32 n,
                                               u32& bits, u32& col, bool& valid) {
        const int j = s / E::kPerVec;
        const int w = (s % E::kPerVec) / kPerDword;
        const int hh = s % kPerDword;
        const u32 d = v[j][w];
        bits = kPerDword == 2 ? ((d >> (16 * hh)) & 0xFFFFu) : d;
        const int vi = vb + j * WG + (int)tid;
        col = (u32)vi * E::kPerVec + (u32)(w * kPerDword + hh);
        valid = vi < v1 && col < n;
    }
};

// ------------------------------------------------------------------ crowded seed
struct SeedBound {
    u64 L;
    u32 exact;
};

// The seed bound when the bin of the seed's k-th entry is crowded: heavy
// ties (runs of one value such as -inf padding, quantized or monotone rows)
// look like this.  The seed tiles are read again (from the cache) with the
// segment's first and last tiles -- the largest values of a monotone row lie
// at one end, the tied entries with the lowest columns at the first -- and
// counted together; the end tiles only tighten the bound and are appended
// in their turn.  If the bin of the k-th counted entry holds one value, its
// entries differ only in their columns, and the k-th composite is that value
// at the r-th lowest of those columns (a lower column is a larger
// composite): that exact bound is returned, with survivors to be tested
// against it; otherwise the bin's floor.  The histogram is zero on entry and
// on return.  Out of line, so the common path keeps its registers.
template <class E, int WG, int CAP, int KS>
__device__ __noinline__ SeedBound crowded_seed_bound(Smem<CAP>& sm, const uint8_t* seg, VecBases<KS> sb,
                                                     int v0, int v1, u32 n, u32 k, u32 ntiles) {
    using SL = Slot<E, 1, WG>;
    // the segment as a buffer resource again, from wave-uniform values (the
    // arguments of a call arrive in vector registers, and loads through a
    // descriptor held there are issued lane group by lane group)
    // (the builtin returns int: each half goes through u32, so the low half
    // is not sign-extended into the high one)
    const u64 sa = (u64)seg;
    const u64 hi = (u32)__builtin_amdgcn_readfirstlane((int)(u32)(sa >> 32));
    const u64 lo = (u32)__builtin_amdgcn_readfirstlane((int)(u32)sa);
    const uint8_t* seg_u = (const uint8_t*)((hi << 32) | lo);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)seg_u, (short)0, (int)((u32)(__builtin_amdgcn_readfirstlane(v1 - v0)) * 16u), kBufferWord3);
    constexpr int kB = KS + 2;
    constexpr int kTileVecs = WG;
    const u32 tid = threadIdx.x;
    int bvb[kB];
#pragma unroll
    for (int i = 0; i < KS; ++i) bvb[i] = sb.b[i];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        int tv = v0 + (j == 0 ? 0 : (int)(ntiles - 1u) * kTileVecs);
#pragma unroll
        for (int i = 0; i < KS; ++i) tv = bvb[i] == tv ? v1 : tv;  // already a seed tile
        if (j == 1 && tv == bvb[KS]) tv = v1;                     // one tile only
        bvb[KS + j] = tv;
    }
    u32x4 bt[kB];
#pragma unroll
    for (int i = 0; i < kB; ++i) bt[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (u32)(bvb[i] + (int)tid - v0) * 16u, 0, 0);
    // -inf padding is the common run: its bin holds -inf only (and NaN,
    // reported anyway), so its entries per tile are counted on the way, in
    // registers, and added to the histogram once per wave (atomics that
    // every wave aims at one word are serialized)
    const u32 kNegInf = E::key(E::kKeyBits == 16 ? 0xFF80u : 0xFF800000u);
    const u32 dNegInf = top_digit(compose<E>(kNegInf, 0u));
    u32 tc[kB];
#pragma unroll
    for (int i = 0; i < kB; ++i) {
        tc[i] = 0;
        // the wave's part of the tile past the segment, or -inf throughout
        // with every column valid: counted at once
        const int vi = bvb[i] + (int)tid;
        if (__ballot(vi < v1) == 0) continue;
        const u32 pat = E::kKeyBits == 16 ? 0xFF80FF80u : 0xFF800000u;
        const bool ninf_all = vi < v1 && (u32)vi * E::kPerVec + (E::kPerVec - 1) < n && bt[i][0] == pat &&
                              bt[i][1] == pat && bt[i][2] == pat && bt[i][3] == pat;
        if (__ballot(ninf_all) == ~0ull) {
            tc[i] = E::kPerVec;
            continue;
        }
        const u32x4 xs[1] = {bt[i]};
#pragma unroll
        for (int s_ = 0; s_ < SL::kSlots; ++s_) {
            u32 bits, col;
            bool valid;
            SL::get(xs, s_, bvb[i], tid, v1, n, bits, col, valid);
            const u32 d = top_digit(compose<E>(E::key(bits), col));
            const bool ninf = valid && d == dNegInf;
            hist_add(sm.hist, d, valid && !ninf);
            tc[i] += ninf ? 1u : 0u;
        }
    }
    u32 wc[kB];  // the wave's -inf entries per tile
    u32 wn = 0;
#pragma unroll
    for (int i = 0; i < kB; ++i) {
        wc[i] = __builtin_amdgcn_readlane(wave_incl_scan(tc[i]), kWave - 1);
        wn += wc[i];
    }
    if (lane_id() == 0 && wn) atomicAdd(&sm.hist[hidx(dNegInf)], wn);
    __syncthreads();
    block_locate<WG, CAP>(sm, k, 0u, true);
    SeedBound r{sm.loc_c[0] > 0 ? digit_floor(sm.loc_digit[0]) : 0ull, 0u};
    if (sm.loc_c[0] < kTiedBin) return r;
    // one value in bin b1?  (least and greatest key; the bin's entries per
    // tile, tc[i] this thread's)
    const u32 b1 = sm.loc_digit[0], r1 = sm.loc_r[0];
    u32 key = kNegInf;
    if (b1 != dNegInf) {
        u32 kmin = ~0u, kmax = 0u;
#pragma unroll
        for (int i = 0; i < kB; ++i) {
            tc[i] = 0;
            const u32x4 xs[1] = {bt[i]};
#pragma unroll
            for (int s_ = 0; s_ < SL::kSlots; ++s_) {
                u32 bits, col;
                bool valid;
                SL::get(xs, s_, bvb[i], tid, v1, n, bits, col, valid);
                const u32 kk = E::key(bits);
                if (valid && top_digit(compose<E>(kk, col)) == b1) {
                    kmin = kk < kmin ? kk : kmin;
                    kmax = kk > kmax ? kk : kmax;
                    ++tc[i];
                }
            }
        }
        kmin = wave_min(kmin);
        kmax = wave_max(kmax);
        if (lane_id() == 0) {
            atomicMin(&sm.tie_min, kmin);
            atomicMax(&sm.tie_max, kmax);
        }
#pragma unroll
        for (int i = 0; i < kB; ++i) wc[i] = __builtin_amdgcn_readlane(wave_incl_scan(tc[i]), kWave - 1);
    }
    if (lane_id() == 0) {
#pragma unroll
        for (int i = 0; i < kB; ++i)
            if (wc[i]) atomicAdd(&sm.tie_cnt[i], wc[i]);
    }
    __syncthreads();
    if (b1 != dNegInf) {
        key = sm.tie_min;
        if (key != sm.tie_max) return r;
    }
    // the tile holding the r1-th lowest column of the bin: tiles are whole
    // column ranges, so order them by start
    u32 mine = 0, rr = 0;
    int which = -1;
#pragma unroll
    for (int i = 0; i < kB; ++i) {
        u32 below = 0;
#pragma unroll
        for (int j = 0; j < kB; ++j) below += bvb[j] < bvb[i] ? sm.tie_cnt[j] : 0u;
        if (below < r1 && r1 <= below + sm.tie_cnt[i]) {
            mine = tc[i];
            rr = r1 - below;
            which = i;
        }
    }
    // a tile of the bin's entries only: the r-th lowest column is the tile's
    // r-th (the common case for a run of one value), with no scan
    constexpr u32 kTileElems = (u32)kTileVecs * E::kPerVec;
    int whole = -1;
#pragma unroll
    for (int i = 0; i < kB; ++i)
        if (i == which && sm.tie_cnt[i] == kTileElems) whole = i;
    if (whole >= 0) {
        int vbw = 0;
#pragma unroll
        for (int i = 0; i < kB; ++i) vbw = i == whole ? bvb[i] : vbw;
        r.L = compose<E>(key, (u32)vbw * E::kPerVec + rr - 1u);
        r.exact = 1u;
        return r;
    }
    // inside it, column order is thread order, then slot order
    u32 tot;
    const u32 excl = block_excl_scan<WG, CAP>(sm, mine, &tot);
    if (excl < rr && rr <= excl + mine) {
#pragma unroll
        for (int i = 0; i < kB; ++i) {
            if (i != which) continue;
            const u32x4 xs[1] = {bt[i]};
            u32 seen = excl;
#pragma unroll
            for (int s_ = 0; s_ < SL::kSlots; ++s_) {
                u32 bits, col;
                bool valid;
                SL::get(xs, s_, bvb[i], tid, v1, n, bits, col, valid);
                if (valid && top_digit(compose<E>(E::key(bits), col)) == b1 && ++seen == rr) sm.tie_col = col;
            }
        }
    }
    __syncthreads();
    r.L = compose<E>(key, sm.tie_col);
    r.exact = 1u;
    return r;
}

// Exact selection of the k largest of buf[0, cnt) (bin b1 holds the k-th,
// rank r1 of c1 inside it) and output, the −inf tail up to kout, then the
// NaN report; the workgroup ends here.
// ------------------------------------------------------------------ sampling
// A row's sampling inputs and token output (the sampling instance).
struct SampleIO {
    const float* temperature;
    const float* top_p;
    const float* uniform;
    int32_t* out_token;
    u32 row;
};

// Inclusive prefix sum of floats across the 64 lanes (all lanes active).
__device__ __forceinline__ float wave_incl_scan_f(float x) {
    auto step = [&](auto ctrl, auto rmask) __attribute__((always_inline)) {
        const int y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value,
                                                  decltype(rmask)::value, 0xF, decltype(rmask)::value == 0xF);
        x += __int_as_float(y);
    };
    step(std::integral_constant<int, 0x111>{}, std::integral_constant<int, 0xF>{});  // row_shr:1
    step(std::integral_constant<int, 0x112>{}, std::integral_constant<int, 0xF>{});  // row_shr:2
    step(std::integral_constant<int, 0x114>{}, std::integral_constant<int, 0xF>{});  // row_shr:4
    step(std::integral_constant<int, 0x118>{}, std::integral_constant<int, 0xF>{});  // row_shr:8
    step(std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xA>{});  // row_bcast:15
    step(std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xC>{});  // row_bcast:31
    return x;
}

// One token from the row's top-k, by the definition the sampling kernel
// follows (sample_kernels.hpp): softmax weights at temperature T relative to
// the largest value, the top-p nucleus as the shortest prefix reaching top_p
// of the total weight, and the inverse CDF at the caller's uniform; T <= 0 is
// greedy.  buf[0, k) holds the top-k in value order, the composites or,
// when `cpl`, their complements (as the output step left them).  Call from
// every thread after a barrier that follows the output.
template <class E, int WG, int CAP>
__device__ __forceinline__ void sample_sorted(Smem<CAP>& sm, u32 k, bool cpl, const SampleIO& io) {
    constexpr u32 kMaxPer = 4096 / WG;  // candidates per thread (k <= 4096)
    const u32 tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    auto comp_at = [&](u32 j) -> u64 { return cpl ? ~sm.buf[j] : sm.buf[j]; };
    auto value = [&](u64 c) -> float {
        const u32 b = E::bits(comp_key<E>(c));
        return __uint_as_float(E::kKeyBits == 16 ? b << 16 : b);
    };
    const float T = io.temperature[io.row];
    if (!(T > 0.0f)) {  // greedy (also for NaN)
        if (tid == 0) io.out_token[io.row] = (int32_t)comp_col<E>(comp_at(0));
        return;
    }
    const float invT = 1.0f / T;
    const float x1 = value(comp_at(0));
    const u32 per = (k + WG - 1) / WG;
    const u32 j0 = tid * per;
    float W[kMaxPer];
    float run = 0.0f;
#pragma unroll
    for (u32 i = 0; i < kMaxPer; ++i) {
        float w = 0.0f;
        if (i < per && j0 + i < k) {
            const float x = value(comp_at(j0 + i));
            w = x == x1 ? 1.0f : (x == -__builtin_huge_valf() ? 0.0f : expf((x - x1) * invT));
        }
        run += w;
        W[i] = run;
    }
    const float incl = wave_incl_scan_f(run);
    float* const wsum = (float*)sm.wsum;
    if (lane == kWave - 1) wsum[wave] = incl;
    if (tid == 0) {
        sm.smp_m = k - 1u;
        sm.smp_pick = ~0u;
    }
    __syncthreads();
    float base = incl - run, total = 0.0f;
#pragma unroll
    for (u32 q = 0; q < (u32)(WG / kWave); ++q) {
        base += q < wave ? wsum[q] : 0.0f;
        total += wsum[q];
    }
    const float thresh = io.top_p[io.row] * total;  // the nucleus: first j with W_j >= top_p W_k
#pragma unroll
    for (u32 i = 0; i < kMaxPer; ++i)
        if (i < per && j0 + i < k && base + W[i] >= thresh) {
            atomicMin(&sm.smp_m, j0 + i);
            break;
        }
    __syncthreads();
    const u32 m = sm.smp_m;
    if (m >= j0 && m < j0 + per) sm.smp_w = base + W[m - j0];
    __syncthreads();
    float u = io.uniform[io.row];
    if (!(u >= 0.0f)) u = 0.0f;
    if (u >= 1.0f) u = 0x1.fffffep-1f;  // the largest float below 1
    const float t = u * sm.smp_w;
#pragma unroll
    for (u32 i = 0; i < kMaxPer; ++i)
        if (i < per && j0 + i <= m && base + W[i] > t) {
            atomicMin(&sm.smp_pick, j0 + i);
            break;
        }
    __syncthreads();
    if (tid == 0) {
        const u32 pk = sm.smp_pick <= m ? sm.smp_pick : m;
        io.out_token[io.row] = (int32_t)comp_col<E>(comp_at(pk));
    }
}

// The column bits of a row of n columns, and the fixed first refine level
// of an element type.
__device__ __forceinline__ u32 col_bits(u32 n) { return n > 1u ? 32u - (u32)__clz((int)(n - 1u)) : 0u; }
template <class E>
constexpr int kFirstOf = E::kKeyBits == 32 ? 1 : 2;

template <class E, int WG, int CAP, bool kSample = false, bool kCounted = false>
__device__ __forceinline__ void select_and_emit(Smem<CAP>& sm, u32 cnt, u32 b1, u32 r1, u32 c1, u32 k, u32 kout, u32 n,
                                             int sorted, int retval, int flags, gptr<void> row_idx_p, gptr<void> row_val,
                                             gptr<int32_t> flag, int32_t flag_value, u64* timing,
                                             const SampleIO& sio = SampleIO{}, u64 o = 0, u64 a = ~0ull) {
    const IdxOut row_idx{row_idx_p, flags & kFlagIdx64};
    const u32 cb = col_bits(n);
    const u64 T = refine<WG, CAP, kFirstOf<E>, kCounted>(sm, cnt, b1, r1, c1, cb, o, a);
    DSTK_T(sm, kPhRefine);
    emit_threshold<E, WG, CAP>(sm, cnt, T, k, n, sorted, retval, flags, row_idx, row_val);
    if (k < kout) write_tail<E, WG>(row_idx, row_val, k, kout);
    __syncthreads();
    if constexpr (kSample) sample_sorted<E, WG, CAP>(sm, k, k > (u32)WG, sio);
    if (threadIdx.x == 0 && sm.nan) *flag = flag_value;
    DSTK_T(sm, kPhEmit);
    DSTK_T_FLUSH(sm, timing);
    (void)timing;
    DSTK_EXIT();
}

// Merge when the boundary bin is too large for the buffer (heavy ties
// across segments): stream the published entries at or above the row
// bound through the buffer, reducing to k whenever it fills.
template <class E, int WG, int CAP>
__device__ __noinline__ void merge_fallback(Smem<CAP>& sm, gptr<const u64> rmeta, gptr<const u32> rdir, gptr<const u64> rc, u32 S,
                                            u32 cap, u64 Lrow, u32 k, u32 n, int sorted, int retval, int flags,
                                            gptr<void> row_idx_p, gptr<void> row_val, gptr<int32_t> flag, int32_t flag_value) {
    const IdxOut row_idx{row_idx_p, flags & kFlagIdx64};
    const u32 tid = threadIdx.x;
    const u32 dL = top_digit(Lrow);
    constexpr int kMI = E::kPerVec;  // entries per thread per step (one tile's worth)
    u32 mm = 0;
    if (tid < S) {
        const u64 m0 = ld_agent(&rmeta[(u64)tid * 4]);
        const u32 lv = (u32)m0, dl = (u32)(m0 >> 32);
        const u32 dh = (u32)ld_agent(&rmeta[(u64)tid * 4 + 1]);
        if (lv == 0 || dL > dh) mm = 0;
        else if (dL <= dl) mm = lv;
        else mm = ld_agent(&rdir[(u64)tid * kBins + (dh - dL)]);
    }
    __syncthreads();
    for (u32 i = tid; i < (u32)kHistWords; i += WG) sm.hist[i] = 0;
    u32 tot2;
    const u32 off2 = block_excl_scan<WG, CAP>(sm, mm, &tot2);
    if (tid < S) sm.seg_count[tid] = off2;
    if (tid == 0) sm.count = 0;
    __syncthreads();
    for (u32 base = 0; base < tot2; base += WG * kMI) {
        u64 e[kMI];
        u32 pmk = 0, c = 0;
#pragma unroll
        for (int j = 0; j < kMI; ++j) {
            const u32 f = base + j * WG + tid;
            e[j] = 0;
            if (f < tot2) {
                u32 lo = 0, hi = S;
                while (hi - lo > 1) {
                    const u32 mid = (lo + hi) >> 1;
                    if (sm.seg_count[mid] <= f) lo = mid; else hi = mid;
                }
                e[j] = ld_agent(&rc[(u64)lo * cap + (f - sm.seg_count[lo])]);
            }
            const bool ok = f < tot2 && e[j] >= Lrow;
            pmk |= (u32)ok << j;
            c += ok;
        }
        u32 pos = wave_reserve(&sm.count, c);
        if (pos != ~0u) {
#pragma unroll
            for (int j = 0; j < kMI; ++j)
                if ((pmk >> j) & 1u) {
                    sm.buf[pos++] = e[j];
                    atomicAdd(&sm.hist[hidx(top_digit(e[j]))], 1u);
                }
        }
        __syncthreads();
        const u32 c2 = sm.count;
        if (c2 > (u32)(CAP - WG * kMI)) make_room<E, WG, CAP>(sm, c2, k, WG * kMI);
    }
    final_select<E, WG, CAP>(sm, sm.count, k);
    emit<E, WG, CAP>(sm, k, n, sorted, retval, flags, row_idx.p, row_val);
    __syncthreads();
    if (tid == 0 && sm.nan) *flag = flag_value;
}

// One workgroup per (row, segment).  EB: element bytes; WG: threads; NV:
// tiles per chunk (16-byte loads each thread has in flight); CAP:
// candidate-buffer entries.
// A "tile" is one vector per thread, WG * 16 bytes; tiles are visited in a
// pseudo-random order, a chunk at a time.
// The sampling inputs of a row (only the sampling instance reads them).
template <bool kSample>
__device__ __forceinline__ SampleIO sample_io(const Params& p, u32 row) {
    if constexpr (kSample) return SampleIO{p.temperature, p.top_p, p.uniform, p.out_token, row};
    return SampleIO{};
}

template <int EB, int WG, int NV, int CAP, bool kSample>
__device__ __forceinline__ void topk_rows_body(const Params& p) {
    using E = Elem<EB>;
    using SL = Slot<E, 1, WG>;
    constexpr int kTileVecs = WG;
    constexpr int kTileElems = kTileVecs * E::kPerVec;
    static_assert(CAP % WG == 0, "capacity must be a multiple of the workgroup size");
    static_assert(CAP >= 2 * NV * kTileElems || NV * kTileElems >= 8192, "capacity must hold two chunks");
    static_assert(NV <= WG / kWave, "one wave's chunk must fit in a tile of the workgroup");
    __shared__ Smem<CAP> sm;

    const u32 tid = threadIdx.x;
    const u32 row = blockIdx.x / (u32)p.segs;
    const u32 seg = blockIdx.x % (u32)p.segs;
    // n: the row's valid columns; k: entries selected from them (k < kout
    // only for a row shorter than the output, whose other slots are the -inf
    // columns past its end)
    const u32 kout = (u32)p.k;
    u32 n = (u32)p.n;
    if (p.lengths) {
        const int32_t len = p.lengths[row];
        n = len < 0 ? 0u : (u32)len < n ? (u32)len : n;
    }
    const u32 k = kout < n ? kout : n;
    const uint8_t* row_in = p.in + (int64_t)row * p.row_stride_bytes;
    const IdxOut row_idx = IdxOut{(gptr<void>)p.out_idx, p.flags & kFlagIdx64}.at((u64)row * kout);
    const gptr<void> row_val = p.retval ? (gptr<void>)((gptr<uint8_t>)p.out_val + (int64_t)row * kout * EB) : nullptr;
    if (k == 0) {  // no valid column: the whole output is the -inf columns
        if (seg == 0) write_tail<E, WG>(row_idx, row_val, 0u, kout);
        return;
    }

    const int v0 = (int)seg * p.seg_vecs;
    int v1 = min(p.n_vec, v0 + p.seg_vecs);
    v1 = min(v1, (int)((n + E::kPerVec - 1) / E::kPerVec));  // vectors with valid columns
    v1 = max(v1, v0);
    // The segment as a raw buffer resource: loads take one 32-bit offset
    // (vector index relative to v0, times 16) and the hardware range check
    // returns zeros past the segment's end instead of faulting.
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(row_in + (int64_t)v0 * 16), (short)0, (int)((u32)(v1 - v0) * 16u), kBufferWord3);
    auto load_vec = [&](int vi) -> u32x4 {  // vi: absolute vector index in the row
        return __builtin_amdgcn_raw_buffer_load_b128(rsrc, (u32)(vi - v0) * 16u, 0, kScanAux);
    };
    const u32 ntiles = (u32)((v1 - v0 + kTileVecs - 1) / kTileVecs);

    // Tile visiting order: t -> (a t + b) mod ntiles with gcd(a, ntiles) = 1.
    // The bf16 kernel for k > 1024 first visits the segment's last and
    // first tiles, then tiles 1 .. ntiles - 2 in that permuted order: with k
    // an eighth of a row or more, a seed drawn from the middle of a sorted
    // or padded row (ascending scores, a -inf tail) admits most of the row,
    // and the sync, refine and emit then work on up to the buffer's size.
    // (Elsewhere the fixed positions cost more than they save: every
    // workgroup's first loads then fall at one offset of its segment.)
    constexpr bool kEndsFirst = EB == 2 && CAP > 8192;
    const bool ends = kEndsFirst && ntiles > 2;
    const u32 m = ends ? ntiles - 2 : ntiles;  // tiles in the permuted part
    const u32 h = hash32(blockIdx.x * 0x9E3779B9u ^ p.seed);
    u32 a = 1, b = 0;
    if (m > 1) {
        a = (u32)(((u64)m * 0x9E3779B9ull) >> 32) | 1u;
        if (a >= m) a = 1;
        while (gcd_u32(a, m) != 1) ++a;
        b = h % m;
    }

    for (u32 i = tid; i < (u32)kHistWords; i += WG) sm.hist[i] = 0;
    if (tid == 0) {
        sm.count = 0;
        sm.L = 0;
        sm.nan = 0;
        sm.last = 0;
        sm.outcount = 0;
        sm.pflag[0] = 0;
        sm.pflag[1] = 0;
        sm.tie_min = ~0u;
        sm.tie_max = 0;
        sm.tie_col = ~0u;  // (not found: the tied value's lowest composite, still a valid bound)
        sm.pubseed = 0;
        for (int i = 0; i < 8; ++i) sm.tie_cnt[i] = 0;
#ifdef DSTK_TIMING
        for (int i = 0; i < kTimingSlots; ++i) sm.ts[i] = 0;
#endif
    }
    DSTK_T(sm, kPhStart);

    PreFilter<E> pf;
    pf.set(0ull);
    __syncthreads();

    u32 pr = b;  // permuted index of the next tile to request (of the permuted part)
    // Tiles counted to seed the bound: the whole first chunk, as far as an
    // empty buffer holds it.  A tighter seed pays for itself: every later
    // tile is filtered against it, and a raise costs a sync and a locate.
    constexpr int kSeed = NV < CAP / kTileElems ? NV : CAP / kTileElems;
    static_assert(kSeed >= 1, "the seed tiles must fit an empty buffer");
    static_assert(kSeed + 2 <= 8, "tie_cnt holds the seed tiles and two end tiles");
    // The tied seed bound (crowded_seed_bound) is built into the bf16
    // kernel for k <= 1024 only: runs of one value are common there (-inf
    // padding, few distinct values), while elsewhere its mere presence costs
    // the common path more than it saves (register allocation: about a
    // microsecond on the fp32 sampler shape; in the bf16 k > 1024 kernel,
    // already at 256 VGPRs, thirty more spills, +3 us on 256 x 32768 with
    // k = 4096).  Tied rows there are selected correctly all the same,
    // through the overflow path.
    constexpr bool kTiedSeed = EB == 2 && CAP == 8192;

    // ---- buffer layout while scanning: buf[0, cbase) holds composites,
    // counted in the histogram; the free part is split into one region of R
    // entries per wave.  A wave appends raw entries (element bits << 32 |
    // column) to its own region behind a scalar write pointer, with no
    // atomics and no barrier; a sync moves the regions' entries behind the
    // composites, converting and counting them with every lane busy.
    const ScanCtx cx{rsrc, v0, v1, n, k};
    ScanState st{};
    assign_regions<WG, CAP>(st, 0u);

    auto issue = [&](u32 t0, u32x4 (&v)[NV], int (&vb)[NV]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const u32 t = t0 + (u32)i;  // visiting position
            u32 tile = pr;
            bool step = true;
            if constexpr (kEndsFirst) {
                step = !ends || t >= 2u;
                tile = step ? pr + (ends ? 1u : 0u) : (t == 0u ? ntiles - 1u : 0u);
            }
            vb[i] = t < ntiles ? v0 + (int)tile * kTileVecs : v1;
            v[i] = load_vec(vb[i] + (int)tid);
            __builtin_amdgcn_sched_barrier(0);  // keep requests in slot order
            if (step) {
                pr += a;
                if (pr >= m) pr -= m;
            }
        }
    };
    // Seed: count every element of the first kSeed tiles and take the bin
    // edge of the k-th counted as the bound; those tiles are then appended
    // like the others.
    auto seed = [&](const u32x4 (&v)[NV], const int (&vb)[NV]) __attribute__((always_inline)) {
        // Runs of equal values (padding, quantized scores) put whole waves
        // in one bin: then the wave counts the entries of each tile that
        // fall in the bin of the tile's first element in a register, adds
        // them once per tile (atomics that every wave aims at one word are
        // serialized) and only the others one by one.  The wave's first
        // elements decide, for its whole seed; in the bf16 kernels a wave's
        // part of a tile that holds one value throughout is counted at once
        // either way.
        u32 b0, c0;
        bool ok0;
        {
            const u32x4 xs[1] = {v[0]};
            SL::get(xs, 0, vb[0], tid, v1, n, b0, c0, ok0);
        }
        const u32 d0 = top_digit(compose<E>(E::key(b0), c0));
        auto count = [&](auto agg_tag) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < kSeed; ++i) {
                const u32x4 xs[1] = {v[i]};
                u32 run = 0, nrun = 0;
                if constexpr (EB == 2) {
                    // the wave's part of the tile one value throughout, every
                    // column valid (a run of padding): counted at once
                    const int vi = vb[i] + (int)tid;
                    const u32 first = __builtin_amdgcn_readfirstlane(v[i][0] & 0xFFFFu);
                    const u32 pat = first | (first << 16);
                    const bool one = vi < v1 && (u32)vi * E::kPerVec + (E::kPerVec - 1) < n && v[i][0] == pat &&
                                     v[i][1] == pat && v[i][2] == pat && v[i][3] == pat;
                    if (__ballot(one) == ~0ull) {
                        if (lane_id() == 0)
                            atomicAdd(&sm.hist[hidx(top_digit(compose<E>(E::key(first), 0u)))],
                                      (u32)(kWave * E::kPerVec));
                        continue;
                    }
                }
#pragma unroll
                for (int s = 0; s < SL::kSlots; ++s) {
                    u32 bits, col;
                    bool valid;
                    SL::get(xs, s, vb[i], tid, v1, n, bits, col, valid);
                    const u32 d = top_digit(compose<E>(E::key(bits), col));
                    if constexpr (decltype(agg_tag)::value) {
                        if (s == 0) run = __builtin_amdgcn_readfirstlane(d);
                        nrun += (u32)__popcll(__ballot(valid && d == run));
                        if (valid && d != run) atomicAdd(&sm.hist[hidx(d)], 1u);
                    } else if (valid) {
                        atomicAdd(&sm.hist[hidx(d)], 1u);
                    }
                }
                if constexpr (decltype(agg_tag)::value)
                    if (lane_id() == 0 && nrun) atomicAdd(&sm.hist[hidx(run)], nrun);
            }
        };
        if (__ballot(ok0) == ~0ull && __ballot(d0 != __builtin_amdgcn_readfirstlane(d0)) == 0)
            count(std::true_type{});
        else
            count(std::false_type{});
        __syncthreads();
        // the locate also clears the histogram: from here on it counts
        // exactly the synced entries
        // A split row's segment that the seed covers whole (all its tiles are
        // seed tiles) has its final histogram now: this locate also writes
        // the publishing directory and bin offsets, and the tail publishes
        // the appended entries straight from the regions (unless a rare
        // round or the crowded path below needs the histogram back).
        const u32 S_ = (u32)p.segs;
        const bool pub_seed = S_ > 1 && ntiles <= (u32)kSeed;
        if (pub_seed) {
            const gptr<u32> dir = keep_g(p.ws_dir) + (u64)(row * S_ + seg) * kBins;
            block_locate<WG, CAP, true>(sm, k, (k + S_ - 1) / S_, false, dir);
            if (tid == 0) sm.pubseed = 1;
        } else {
            block_locate<WG, CAP>(sm, k, 0u, true);
        }
        if (sm.loc_c[0] > 0) st.L = digit_floor(sm.loc_digit[0]);
        if (kTiedSeed && sm.loc_c[0] >= kTiedBin) {
            if (pub_seed) {  // (the crowded path starts from an empty histogram)
                for (u32 i = tid; i < (u32)kHistWords; i += WG) sm.hist[i] = 0;
                __syncthreads();
                if (tid == 0) sm.pubseed = 0;
            }
            VecBases<kSeed> sb;
#pragma unroll
            for (int i = 0; i < kSeed; ++i) sb.b[i] = vb[i];
            const SeedBound r =
                crowded_seed_bound<E, WG, CAP, kSeed>(sm, row_in + (int64_t)v0 * 16, sb, v0, v1, n, k, ntiles);
            st.L = r.L;
            st.exact = r.exact;
        }
        pf.set(st.L);
        DSTK_T(sm, kPhSeed);
    };
    // Append a chunk, then check.  After chunks 7, 15, 31, ... (a fixed
    // schedule, so every wave takes the same barriers; on long segments the
    // bound then tightens as the number of elements seen doubles) the rare
    // step syncs and raises the bound.  Shorter segments keep the seed's
    // bound: a raise there costs more than the appends it saves, and a full
    // region raises the bound anyway.
    // (first: the call for chunk 0, the only one a segment the seed covers
    // whole makes; the loop's calls carry no code for that case)
    auto process = [&](auto first, u32 t0, const u32x4 (&v)[NV], const int (&vb)[NV]) __attribute__((always_inline)) {
        const u32 c = t0 / NV;
        const bool raise = t0 + NV < ntiles && c >= 7 && ((c + 1) & c) == 0;
        const u32 rtile = append_chunk<E, WG, NV, CAP>(sm, cx, st, pf, v, vb, 0u);
        const bool again = check_pending<WG, CAP>(sm, st, rtile < (u32)NV);
        if (again || raise) {
            if constexpr (decltype(first)::value) {
                if (sm.pubseed) {  // (the sync counts into an empty histogram)
                    for (u32 i = tid; i < (u32)kHistWords; i += WG) sm.hist[i] = 0;
                    __syncthreads();
                    if (tid == 0) sm.pubseed = 0;
                }
            }
            VecBases<NV> bases;
#pragma unroll
            for (int i = 0; i < NV; ++i) bases.b[i] = vb[i];
            st = rare_rounds<E, WG, NV, CAP>(sm, cx, st, bases, rtile, again);
            pf.set(st.L);
        }
    };
    {
        // Double buffering: chunk c + 1 is in flight while chunk c is
        // appended.  The next chunk is always requested, also past the
        // segment's end (such tiles are range-checked buffer loads that
        // return zeros and touch no memory), so every path has the same loads
        // in flight and each tile waits only for its own load.
        // The loop is entered, and re-entered, with only vc's loads in
        // flight, so the wait before each tile covers exactly that tile's
        // load.
        u32x4 va[NV], vc[NV];
        int vba[NV], vbc[NV];
        issue(0, va, vba);
        issue(NV, vc, vbc);
        seed(va, vba);
        process(std::true_type{}, 0, va, vba);
        if ((u32)NV < ntiles) {
            for (u32 t0 = NV;; t0 += 2 * NV) {
                issue(t0 + NV, va, vba);
                process(std::false_type{}, t0, vc, vbc);
                if (t0 + NV >= ntiles) break;
                issue(t0 + 2 * NV, vc, vbc);
                process(std::false_type{}, t0 + NV, va, vba);
                if (t0 + 2 * NV >= ntiles) break;
            }
        }
    }
    // (the last check's barrier follows every wave's last append)
    DSTK_T(sm, kPhScan);
    // the arguments the tail uses, as kept values (see keep())
    const gptr<int32_t> flag = keep_g(p.flag);
    const int32_t flag_value = keep(p.flag_value);
    u64* const timing = keep(p.timing);
    (void)timing;
    const int sorted = keep(p.sorted), retval = keep(p.retval), flags = keep(p.flags);
    const u32 S = keep((u32)p.segs);
    const u32 cap = keep((u32)p.pub_cap);
    // Published from the seed's bins?  (Not if more than the list holds.)
    bool fast = false;
    if (S > 1 && sm.pubseed) {
        const u32 live0 = sm.loc_c[0] ? sm.loc_above[0] + sm.loc_c[0] : sm.loc_total;
        fast = live0 <= cap;
        if (!fast) {  // (convert_regions counts into an empty histogram)
            for (u32 i = tid; i < (u32)kHistWords; i += WG) sm.hist[i] = 0;
            __syncthreads();
        }
    }
    if (S == 1) {
        const u32 c = sync_regions<E, WG, CAP>(sm, st.cbase, st.R);
        if (tid == 0) sm.count = c;
    } else if (!fast) {
        // a split row publishes from where the entries lie
        convert_regions<E, WG, CAP>(sm, st.cbase, st.R);
    }
    if (st.nan) sm.nan = 1;  // benign race: every writer stores 1
    u64 L = st.L;
    if (tid == 0) sm.L = L;
    __syncthreads();
    DSTK_T(sm, kPhSync);
    u32 cnt = sm.count;
    const u32 wave = tid / kWave;

    if (S == 1) {
        block_locate<WG, CAP>(sm, k, 0u, true);
        DSTK_T(sm, kPhLocate);
        select_and_emit<E, WG, CAP, kSample>(sm, cnt, sm.loc_digit[0], sm.loc_r[0], sm.loc_c[0], k, kout, n, sorted,
                                             retval, flags, row_idx.p, row_val, flag, flag_value, timing,
                                             sample_io<kSample>(p, row));
        return;
    }

    // ---- split row: publish this segment's live candidates (entries in the
    // bin of its k-th counted entry or above) in descending top-digit order,
    // with a directory dir[j] = number of entries with top digit >= d_hi - j.
    const u32 slot = row * S + seg;
    const gptr<u64> ws_cand = keep_g(p.ws_cand);
    const gptr<u64> ws_meta = keep_g(p.ws_meta);
    const gptr<u32> ws_dir = keep_g(p.ws_dir);
    const gptr<u32> ws_ticket = keep_g(p.ws_ticket);
    {
        // q = ceil(k / S): with every segment holding q entries at or above
        // its q-bound, the smallest q-bound over the row is a valid bound too
        const u32 q = (k + S - 1) / S;
        const gptr<u32> dir = ws_dir + (u64)slot * kBins;
        // locate, directory and placement offsets in one pass over the bins
        // (done by the seed on the fast path)
        if (!fast) block_locate<WG, CAP, true>(sm, k, q, false, dir);
        DSTK_T(sm, kPhLocate);
        u32 dl = sm.loc_c[0] ? sm.loc_digit[0] : 0u;
        u32 live = sm.loc_c[0] ? sm.loc_above[0] + sm.loc_c[0] : sm.loc_total;
        u64 bq = sm.loc_c[1] ? digit_floor(sm.loc_digit[1]) : 0ull;
        const RegionMap<WG> map(sm, st.cbase, st.R);
        bool moved = false;  // the regions have been moved together
        if (live > cap) {
            // too many to publish: move the entries together (already
            // counted: the move alone), then reduce exactly to k
            __syncthreads();  // everyone has built the map from wfill
            cnt = move_regions<WG, CAP>(sm, map);
            moved = true;
            // (the histogram is counted again; the directory is rewritten)
            cnt = reduce_to_k<WG, CAP, true>(sm, cnt, k, q, sm.loc_digit[0], sm.loc_r[0], sm.loc_c[0], dir);
            if (sm.kth > L) L = sm.kth;
            dl = sm.loc_digit[0];
            live = sm.loc_above[0] + sm.loc_c[0];
            bq = sm.loc_c[1] ? digit_floor(sm.loc_digit[1]) : 0ull;
        }
        const u32 dh = sm.loc_dhi;
        if (tid == 0) {
            const gptr<u64> meta = ws_meta + (u64)slot * 4;
            st_agent(&meta[0], (u64)live | ((u64)dl << 32));
            st_agent(&meta[1], (u64)(live ? dh : 0u));
            st_agent(&meta[2], L);
            st_agent(&meta[3], bq);
        }
        const gptr<u64> cand = ws_cand + (u64)slot * cap;
        const u32 total = moved ? cnt : map.total;
        if (fast) {
            // the regions hold raw entries (bits << 32 | column): convert here
            bool nan = false;
            for (u32 i = tid; i < total; i += WG) {
                const u64 raw = sm.buf[map.addr(i)];
                const u32 bits = (u32)(raw >> 32);
                nan |= E::is_nan(bits);
                const u64 e = compose<E>(E::key(bits), (u32)raw);
                const u32 d = top_digit(e);
                if (live > 0 && d >= dl) {
                    const u32 pos = atomicAdd(&sm.hist[hidx(d)], 1u);
                    if (pos < cap) st_agent(&cand[pos], e);  // pos < live by the histogram invariant
                }
            }
            if (nan) sm.nan = 1;  // benign race: every writer stores 1
        } else {
            for (u32 i = tid; i < total; i += WG) {
                const u64 e = sm.buf[moved ? i : map.addr(i)];
                const u32 d = top_digit(e);
                if (live > 0 && d >= dl) {
                    const u32 pos = atomicAdd(&sm.hist[hidx(d)], 1u);
                    if (pos < cap) st_agent(&cand[pos], e);  // pos < live by the histogram invariant
                }
            }
        }
    }
    // Hand-off: this wave's device-coherent stores have completed; once every
    // wave is past the barrier, one relaxed ticket increment publishes the
    // segment.  The last of the row's segments merges.
    DSTK_T(sm, kPhPublish);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const u32 prev = __hip_atomic_fetch_add(&ws_ticket[row], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm.last = prev == S - 1;
    }
    __syncthreads();
    DSTK_T(sm, kPhTicket);
    if (!sm.last) {
        if (tid == 0 && sm.nan) *flag = flag_value;
        DSTK_T_FLUSH(sm, timing);
        return;
    }

    // ---- merge.  Every element of the row's top-k is in some segment's
    // published list.  One round trip reads every segment's metadata and the
    // head of its directory; the row histogram, a one-wave walk to the bin of
    // the row's k-th entry and the segments' shares follow, then the shares
    // are loaded and the selection finishes as for a single segment.
    const gptr<const u64> rc = ws_cand + (u64)row * S * cap;
    const gptr<const u32> rdir = ws_dir + (u64)row * S * kBins;
    constexpr u32 kDirCache = 16;  // directory entries read with the metadata
    u64* mc = sm.buf;                                 // [S][4] metadata
    u32* dc = (u32*)(sm.buf + 4 * S);                 // [S][kDirCache] directory heads
    for (u32 i = tid; i < S * 4; i += WG) mc[i] = ld_agent(&ws_meta[(u64)row * S * 4 + i]);
    for (u32 i = tid; i < S * kDirCache; i += WG)
        dc[i] = ld_agent(&rdir[(u64)(i / kDirCache) * kBins + (i % kDirCache)]);
    for (u32 i = tid; i < (u32)kHistWords; i += WG) sm.hist[i] = 0;
    if (tid == 0) {
        st_agent(&ws_ticket[row], 0u);  // ready for the next call
        sm.d_hi = 0;
    }
    __syncthreads();
    auto dirv = [&](u32 s_, u32 j) -> u32 {  // entries of segment s_ with digit >= d_hi - j
        return j < kDirCache ? dc[s_ * kDirCache + j] : ld_agent(&rdir[(u64)s_ * kBins + j]);
    };
    DSTK_T(sm, kPhHeaders);
    // Each segment's list head is requested now, up to its published count
    // (the share, a prefix of the list, is known only after the row bin), so
    // the row bin is worked out while the loads are in flight.
    const u32 G = (u32)WG / S;  // threads per segment in the list load (S <= 256: two or more)
    const u32 ls = tid / G, lj0 = tid - ls * G;
    const gptr<const u64> src = rc + (u64)(ls < S ? ls : 0u) * cap;
    constexpr int kLB = 4;  // loads in flight per thread
    u64 v[kLB];
    auto load = [&](u32 j, u32 lim) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kLB; ++u) {
            const u32 jj = j + (u32)u * G;
            v[u] = jj < lim ? ld_agent(&src[jj]) : 0ull;
        }
    };
    {
        const u32 lv = ls < S ? (u32)mc[ls * 4] : 0u;
        load(lj0, lv < cap ? lv : cap);
    }
    // With few segments, each directory within its cached head, every wave
    // works out the row's k-th bin and the shares itself from the segments'
    // cumulative counts (lane s holds segment s's metadata): no row histogram
    // and no barrier before the list load.
    constexpr u32 kDirectS = 16;
    bool direct = false;
    u32 lv_l = 0, dl_l = 0, dh_l = 0;
    if (S <= kDirectS) {
        if (lane_id() < S) {
            const u64 m0 = mc[lane_id() * 4];
            lv_l = (u32)m0;
            dl_l = (u32)(m0 >> 32);
            dh_l = (u32)mc[lane_id() * 4 + 1];
        }
        direct = __ballot(lv_l > 0 && dh_l - dl_l >= kDirCache) == 0;
    }
    u32 b1 = 0, r1 = 0, c1 = 0, total = 0, d_off = 0, d_share = 0;
    if (direct) {
        const u32 l = lane_id();
        const u32 dhm = wave_max(lv_l > 0 ? dh_l : 0u);  // highest published bin
        // C(b): entries of the row published with top digit >= b, for this
        // lane's bin b; the first bin (walking down) with C(b) >= k holds the
        // k-th.
        u32 prev = 0;  // C of the bin above the current 64
        for (u32 j0 = 0; j0 <= dhm; j0 += kWave) {
            const bool in = j0 + l <= dhm;
            const u32 b = dhm - j0 - l;
            u32 C = 0;
            for (u32 s_ = 0; s_ < S; ++s_) {
                const u32 lv = __builtin_amdgcn_readlane(lv_l, s_);
                if (lv == 0) continue;
                const u32 dl = __builtin_amdgcn_readlane(dl_l, s_), dh = __builtin_amdgcn_readlane(dh_l, s_);
                const bool mid = b > dl && b <= dh;  // then dh - b < kDirCache
                const u32 dv = dc[s_ * kDirCache + (mid ? dh - b : 0u)];
                C += b > dh ? 0u : (mid ? dv : lv);
            }
            const u64 hit = __ballot(in && C >= k);
            if (hit) {
                const u32 hl = (u32)__builtin_ctzll(hit);
                const u32 ch = __builtin_amdgcn_readlane(C, hl);
                const u32 cp = hl ? __builtin_amdgcn_readlane(C, hl - 1) : prev;
                b1 = dhm - j0 - hl;
                c1 = ch - cp;
                r1 = k - cp;
                break;
            }
            prev = __builtin_amdgcn_readlane(C, kWave - 1);
        }
        // segment l's share: its entries at or above b1
        const bool mid = lv_l > 0 && dh_l >= b1 && b1 > dl_l;
        const u32 dv = dc[(l < S ? l : 0u) * kDirCache + (mid ? dh_l - b1 : 0u)];
        const u32 m = lv_l > 0 && dh_l >= b1 ? (mid ? dv : lv_l) : 0u;
        const u32 incl = wave_incl_scan(m);
        total = __builtin_amdgcn_readlane(incl, kWave - 1);
        const u32 s_ = ls;
        d_off = (u32)__builtin_amdgcn_ds_bpermute((int)((s_ & (kWave - 1)) * 4), (int)(incl - m));
        d_share = (u32)__builtin_amdgcn_ds_bpermute((int)((s_ & (kWave - 1)) * 4), (int)m);
        if (s_ >= S) d_share = 0;
    } else {
        // Row histogram of the published entries, from the directories: one
        // thread per (segment, cached directory entry), then the entries of
        // segments with more bins than the cache holds.
        for (u32 i = tid; i < S * kDirCache; i += WG) {
            const u32 s_ = i / kDirCache, j = i % kDirCache;
            const u64 m0 = mc[s_ * 4];
            const u32 lv = (u32)m0, dl = (u32)(m0 >> 32), dh = (u32)mc[s_ * 4 + 1];
            if (lv > 0 && j <= dh - dl) {
                const u32 c = dc[i] - (j ? dc[i - 1] : 0u);
                if (c) atomicAdd(&sm.hist[hidx(dh - j)], c);
                if (j == 0) atomicMax(&sm.d_hi, dh);
            }
        }
        {
            // Below the row bound (the largest segment bound, or the smallest
            // q-bound if that is larger: either leaves k entries of the row at or
            // above it) no bin is needed; it is worked out by a wave that meets
            // such a segment.
            u32 dL = 0;
            bool have_dL = false;
            for (u32 s_ = wave; s_ < S; s_ += WG / kWave) {
                const u64 m0 = mc[s_ * 4];
                const u32 lv = (u32)m0, dl = (u32)(m0 >> 32), dh = (u32)mc[s_ * 4 + 1];
                if (lv == 0 || dh - dl < kDirCache) continue;
                if (!have_dL) {
                    u64 lmax = 0, qmin = ~0ull;
                    for (u32 t = lane_id(); t < S; t += kWave) {
                        lmax = mc[t * 4 + 2] > lmax ? mc[t * 4 + 2] : lmax;
                        qmin = mc[t * 4 + 3] < qmin ? mc[t * 4 + 3] : qmin;
                    }
                    lmax = wave_max64(lmax);
                    qmin = wave_min64(qmin);
                    dL = top_digit(lmax > qmin ? lmax : qmin);
                    have_dL = true;
                }
                const u32 lo = dl > dL ? dl : dL;
                for (u32 j = kDirCache + lane_id(); dh >= lo && j <= dh - lo; j += kWave) {
                    const u32 c = dirv(s_, j) - dirv(s_, j - 1);
                    if (c) atomicAdd(&sm.hist[hidx(dh - j)], c);
                }
            }
        }
        __syncthreads();
        if (wave == 0) {
            // One wave walks the bins down from the highest published one to
            // the bin of the row's k-th entry (the counts at and above it are
            // complete: every segment publishes all of its entries at or above
            // its own k-th's bin, which lies at or below the row's), then gives
            // each segment's share (its entries at or above that bin, a prefix
            // of its list) and their offsets.
            const u32 l = lane_id();
            const u32 dhm = __builtin_amdgcn_readfirstlane(sm.d_hi);  // highest published bin
            // (the first 64 segments' metadata, read ahead of the walk)
            const u64 m0a = l < S ? mc[l * 4] : 0ull;
            const u32 dha = l < S ? (u32)mc[l * 4 + 1] : 0u;
            u32 b1 = 0, r1 = 0, c1 = 0, above = 0;
            for (u32 j0 = 0; j0 <= dhm; j0 += kWave) {
                const u32 c = j0 + l <= dhm ? sm.hist[hidx(dhm - j0 - l)] : 0u;
                const u32 incl = wave_incl_scan(c);
                const u64 hit = __ballot(above + incl >= k);
                if (hit) {
                    const u32 hl = hit ? (u32)__builtin_ctzll(hit) : 0u;
                    b1 = dhm - j0 - hl;
                    c1 = __builtin_amdgcn_readlane(c, hl);
                    r1 = k - (above + __builtin_amdgcn_readlane(incl, hl) - c1);
                    break;
                }
                above += __builtin_amdgcn_readlane(incl, kWave - 1);
            }
            u32 carry = 0;
            for (u32 s0 = 0; s0 < S; s0 += kWave) {
                const u32 s_ = s0 + l;
                u32 m = 0;
                if (s_ < S) {
                    const u64 m0 = s0 ? mc[s_ * 4] : m0a;
                    const u32 lv = (u32)m0, dl = (u32)(m0 >> 32), dh = s0 ? (u32)mc[s_ * 4 + 1] : dha;
                    if (lv > 0 && dh >= b1) m = b1 <= dl ? lv : dirv(s_, dh - b1);
                }
                const u32 incl = wave_incl_scan(m);
                if (s_ < S) sm.seg_count[s_] = carry + incl - m;
                carry += __builtin_amdgcn_readlane(incl, kWave - 1);
            }
            if (l == 0) {
                sm.loc_digit[0] = b1;
                sm.loc_r[0] = r1;
                sm.loc_c[0] = c1;
                sm.newtotal = carry;
            }
        }
        __syncthreads();

        b1 = sm.loc_digit[0];
        r1 = sm.loc_r[0];
        c1 = sm.loc_c[0];
        total = sm.newtotal;
    }
    DSTK_T(sm, kPhLoad);
    if (total > (u32)CAP) {
        if (direct) __syncthreads();  // (mc and dc are still being read)
        merge_fallback<E, WG, CAP>(sm, ws_meta + (u64)row * S * 4, rdir, rc, S, cap, digit_floor(b1), k, n,
                                   sorted, retval,
                                   flags, row_idx.p, row_val, flag, flag_value);
        if (k < kout) write_tail<E, WG>(row_idx, row_val, k, kout);
        if constexpr (kSample) {
            __syncthreads();
            sample_sorted<E, WG, CAP>(sm, k, k > (u32)WG, sample_io<kSample>(p, row));
        }
        DSTK_T(sm, kPhEmit);
        DSTK_T_FLUSH(sm, timing);
        return;
    }
    // The shares are loaded, and the entries of the k-th entry's bin are
    // counted for the refine's first level (and chained) as they arrive: no
    // pass over the buffer afterwards.
    u64 fo = 0, fa = ~0ull;  // OR / AND of this thread's entries of bin b1
    {
        // G threads per segment load its share (no search for the source);
        // the first loads are in flight since the metadata arrived
        const u32 s_ = ls, j0 = lj0;
        const u32 off = direct ? d_off : s_ < S ? sm.seg_count[s_] : 0u;
        const u32 share = direct ? d_share : s_ < S ? (s_ + 1 < S ? sm.seg_count[s_ + 1] : total) - off : 0u;
        for (u32 i = tid; i < (u32)kHistWords; i += WG) sm.hist[i] = 0;  // zero for the selection
        __syncthreads();
        const FirstLevel<kFirstOf<E>, CAP> fl(sm, total, col_bits(n));
        for (u32 j = j0; j < share; j += G * kLB) {
#pragma unroll
            for (int u = 0; u < kLB; ++u) {
                const u32 jj = j + (u32)u * G;
                if (jj < share) {
                    sm.buf[off + jj] = v[u];
                    if (top_digit(v[u]) == b1) fl.add(sm, v[u], off + jj, fo, fa);
                }
            }
            if (j + G * kLB < share) load(j + G * kLB, share);
        }
    }
    __syncthreads();
    DSTK_T(sm, kPhMergeLocate);
    select_and_emit<E, WG, CAP, kSample, true>(sm, total, b1, r1, c1, k, kout, n, sorted, retval, flags, row_idx.p,
                                               row_val, flag, flag_value, timing, sample_io<kSample>(p, row), fo, fa);
}

// The selection kernel, and the same with the sampling step after a row's
// value-ordered output (one token per row: ds_topk_sample in one launch).
template <int EB, int WG, int NV, int CAP>
__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(WG / 256)))
void topk_rows(Params p) {
    topk_rows_body<EB, WG, NV, CAP, false>(p);
}
template <int EB, int WG, int NV, int CAP>
__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(WG / 256)))
void topk_sample_rows(Params p) {
    topk_rows_body<EB, WG, NV, CAP, true>(p);
}

}  // namespace dstk

namespace dstk {

// ------------------------------------------------------------------ short rows
// Rows of at most kSmallN columns: one wave per row, kSmallWG / 64 rows per
// workgroup (the one-workgroup-per-row kernel would leave most of a 512-lane
// workgroup idle).  Lane l keeps the composites of columns l, l + 64, ... in
// registers; a radix select over kB-bit digits, in the wave's own LDS
// histogram, narrows the k-th composite from the top bits down until its
// digit's whole sub-bin is kept, which gives T with exactly k composites at
// or above it; between levels the window moves past the bits that every
// remaining candidate shares (their OR and AND), so runs of equal bits
// (high column bits, tied values) cost no level.  Kept entries are written
// in column order by ballot (that is index order too), or gathered and
// sorted by value.  Only the wave's own LDS is touched, so no workgroup
// barrier is needed.  Two instances: 11-bit digits for rows up to kSmallN
// columns, and 8-bit digits with a quarter of the LDS per wave for rows up
// to kTinyN (a 2048-bin histogram to clear and scan per level, for a few
// elements per lane, and 8 KB per wave that limit how many waves a CU
// holds, cost more than a level or two more).
constexpr int kSmallN = 2048;
constexpr int kTinyN = 256;
constexpr int kSmallWG = 256;
constexpr int kSmallValueMax = kBins / 2;        // value order: k the LDS list holds (u64 in the histogram)

template <int EB, int kB>
__global__ __launch_bounds__(kSmallWG) void topk_small_rows(Params p, int64_t rows) {
    using E = Elem<EB>;
    using VT = typename std::conditional<EB == 2, uint16_t, uint32_t>::type;
    constexpr u32 kWaves = kSmallWG / kWave;
    constexpr u32 kNB = 1u << kB;                            // digit bins
    constexpr u32 kPerLane = kNB / kWave;                    // bins a lane sums
    constexpr int kSmallJ = (kB == kHistBits ? kSmallN : kTinyN) / kWave;  // columns per lane
    // the histogram, and for value order the list of kept composites (u64)
    constexpr u32 kWords = kB == kHistBits ? (u32)kBins : 2u * (u32)kTinyN;
    static_assert(kPerLane >= 1 && kPerLane <= (u32)kWave && kWords >= kNB, "digit bins per lane");
    __shared__ u32 hist_all[kWaves][kWords];
    const u32 wave = threadIdx.x / kWave, l = lane_id();
    const int64_t row = (int64_t)blockIdx.x * kWaves + wave;
    if (row >= rows) return;  // the whole wave
    u32* const hist = hist_all[wave];
    const u32 kout = (u32)p.k;
    u32 n = (u32)p.n;
    if (p.lengths) {
        const int32_t len = p.lengths[row];
        n = len < 0 ? 0u : (u32)len < n ? (u32)len : n;
    }
    const u32 k = kout < n ? kout : n;
    const IdxOut out = IdxOut{(gptr<void>)p.out_idx, p.flags & kFlagIdx64}.at((u64)row * kout);
    const gptr<VT> ov = p.retval ? (gptr<VT>)((gptr<uint8_t>)p.out_val + (u64)row * kout * EB) : nullptr;
    for (u32 j = k + l; j < kout; j += kWave) {  // -inf columns past a short row (see write_tail)
        out.put(j, j);
        if (ov) ov[j] = EB == 2 ? (VT)0xFF80u : (VT)0xFF800000u;
    }
    if (k == 0) return;

    const uint8_t* rin = p.in + row * p.row_stride_bytes;
    const u32 jn = (n + kWave - 1) / kWave;
    u64 comp[kSmallJ];
    bool nan = false;
#pragma unroll
    for (u32 j = 0; j < (u32)kSmallJ; ++j) {
        const u32 col = j * kWave + l;
        u64 c = 0;
        if (j < jn && col < n) {
            const u32 b = EB == 2 ? (u32)((const uint16_t*)rin)[col] : ((const u32*)rin)[col];
            nan |= E::is_nan(b);
            c = compose<E>(E::key(b), col);  // never 0
        }
        comp[j] = c;
    }
    if (__ballot(nan) && l == 0) *p.flag = p.flag_value;

    // radix select: window [sh, fixed) of the composites whose bits at or
    // above `fixed` equal P's; r = rank of the k-th among them
    u64 P = 0;
    int fixed = 64;
    u32 r = k;
    for (int level = 0; level < 64; ++level) {
        const int sh = fixed > kB ? fixed - kB : 0;
        const u64 pm = ~low_mask(fixed), wm = low_mask(fixed - sh);
        for (u32 i = l; i < kNB; i += kWave) hist[i] = 0;
#pragma unroll
        for (u32 j = 0; j < (u32)kSmallJ; ++j)
            if (j < jn && comp[j] != 0 && (comp[j] & pm) == P) atomicAdd(&hist[(u32)((comp[j] >> sh) & wm)], 1u);
        // lane l owns digits kNB - 1 - kPerLane l - i, i < kPerLane
        // (descending with the lane)
        u32 s = 0;
#pragma unroll
        for (u32 i = 0; i < kPerLane; ++i) s += hist[kNB - 1u - kPerLane * l - i];
        const u32 incl = wave_incl_scan(s);
        const u64 hm = __ballot(incl >= r);  // not empty: r <= the entries counted
        const u32 hl = hm ? (u32)__builtin_ctzll(hm) : (u32)kWave - 1u;
        const u32 above = __builtin_amdgcn_readlane(incl - s, hl);
        const u32 ci = l < kPerLane ? hist[kNB - 1u - kPerLane * hl - l] : 0u;
        const u32 in2 = wave_incl_scan(ci);
        const u64 jm = __ballot(above + in2 >= r);
        const u32 jl = jm ? (u32)__builtin_ctzll(jm) : kPerLane - 1u;
        const u32 cc = __builtin_amdgcn_readlane(ci, jl);
        const u32 rr = r - (above + __builtin_amdgcn_readlane(in2, jl) - cc);
        P |= (u64)(kNB - 1u - kPerLane * hl - jl) << sh;
        if (rr >= cc || sh == 0) break;  // the whole sub-bin is kept: exactly k at or above P
        r = rr;
        // The next window starts at the highest bit below sh where the
        // sub-bin's entries (two or more: rr < cc) differ; the bits above it
        // are the same in all of them.
        const u64 pm2 = ~low_mask(sh);
        u64 o = 0, a = ~0ull;
#pragma unroll
        for (u32 j = 0; j < (u32)kSmallJ; ++j)
            if (j < jn && comp[j] != 0 && (comp[j] & pm2) == P) {
                o |= comp[j];
                a &= comp[j];
            }
        const u64 O = ((u64)wave_or((u32)(o >> 32)) << 32) | wave_or((u32)o);
        const u64 A = ((u64)wave_and((u32)(a >> 32)) << 32) | wave_and((u32)a);
        const u64 D = (O ^ A) & low_mask(sh);
        const int hb = D ? 63 - __clzll((long long)D) : 0;
        P |= A & low_mask(sh) & ~low_mask(hb + 1);
        fixed = hb + 1;
    }
    const u64 T = P;

    if (p.sorted != kOrderValue) {  // column order: index order, and any order
        u32 run = 0;
#pragma unroll
        for (u32 j = 0; j < (u32)kSmallJ; ++j) {
            const bool keep = j < jn && comp[j] >= T && comp[j] != 0;
            const u64 m = __ballot(keep);
            const u32 pos = run + mbcnt(m);
            if (keep && pos < k) {
                out.put(pos, comp_col<E>(comp[j]));
                if (ov) ov[pos] = (VT)E::bits(comp_key<E>(comp[j]));
            }
            run += (u32)__popcll(m);
        }
        return;
    }
    // value order: gather the kept composites (complemented: ascending sort
    // puts the largest first, padding ~0 last) into the wave's LDS, then
    // ranks by lane broadcasts when one lane each suffices, else a bitonic
    // sort there
    u64* const list = (u64*)hist;
    u32 run = 0;
#pragma unroll
    for (u32 j = 0; j < (u32)kSmallJ; ++j) {
        const bool keep = j < jn && comp[j] >= T && comp[j] != 0;
        const u64 m = __ballot(keep);
        const u32 pos = run + mbcnt(m);
        if (keep && pos < kWords / 2u) list[pos] = ~comp[j];
        run += (u32)__popcll(m);
    }
    u32 Pn = 1;
    while (Pn < k) Pn <<= 1;
    for (u32 i = k + l; i < Pn; i += kWave) list[i] = ~0ull;
    if (k <= (u32)kWave) {
        // one entry per lane: the complemented composites are distinct, so
        // an entry's slot is the number of entries below it, counted over
        // lane broadcasts
        const u64 key = l < k ? list[l] : ~0ull;
        const u32 khi = (u32)(key >> 32), klo = (u32)key;
        u32 rank = 0;
        for (u32 j = 0; j < k; ++j) {
            const u64 o = ((u64)(u32)__builtin_amdgcn_readlane((int)khi, (int)j) << 32) |
                          (u32)__builtin_amdgcn_readlane((int)klo, (int)j);
            rank += o < key ? 1u : 0u;
        }
        if (l < k) {
            out.put(rank, comp_col<E>(~key));
            if (ov) ov[rank] = (VT)E::bits(comp_key<E>(~key));
        }
        return;
    }
    for (u32 size = 2; size <= Pn; size <<= 1)
        for (u32 stride = size >> 1; stride > 0; stride >>= 1)
            for (u32 t = l; t < Pn / 2; t += kWave) {
                const u32 i = 2 * t - (t & (stride - 1)), j = i + stride;
                const bool up = (i & size) == 0;
                const u64 x = list[i], y = list[j];
                if ((x > y) == up) {
                    list[i] = y;
                    list[j] = x;
                }
            }
    for (u32 i = l; i < k; i += kWave) {
        const u64 c = ~list[i];
        out.put(i, comp_col<E>(c));
        if (ov) ov[i] = (VT)E::bits(comp_key<E>(c));
    }
}

}  // namespace dstk
