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
//   * one workgroup streams one row segment with 16-byte loads, the next tile
//     in flight while the current one is filtered;
//   * every element is mapped to a 64-bit composite key
//         (order-preserving value key << ...) | (~column << ...)
//     so that the operator's total order (value, then +0 over -0, then the
//     lower column) is plain unsigned order and all keys are distinct;
//   * a float compare against the threshold's value rejects most elements
//     in one VALU op (it also lets NaN through, to be caught exactly);
//   * survivors are checked exactly and appended to an LDS buffer with one
//     ballot and one LDS atomic per wave and tile;
//   * the buffer is reduced to k by an MSD radix select in LDS; the k-th
//     composite becomes the new admission bound;
//   * short batches split each row over several workgroups; each writes its
//     local top-k to a workspace and the last one to finish (agent-scope
//     ticket) merges them with the same filter/compaction machinery;
//   * index-ordered output is a bitonic sort of the k survivors in LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dstk {

using u32 = uint32_t;
using u64 = uint64_t;

constexpr int kWave = 64;
// Word 3 of a raw buffer resource on CDNA (32-bit data format, no swizzle,
// no index stride): byte-addressed loads with a range check.
constexpr int kBufferWord3 = 0x00020000;
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

template <>
struct PreFilter<Elem<2>> {
    float t_lo;  // for the low half of a dword: exact bf16 value << 16
    float t_hi;  // for the high half read as a whole dword (low half is noise):
                 // the least float whose upper 16 bits are the threshold's
    __device__ void set(u64 L) {
        u32 b = Elem<2>::bits(comp_key<Elem<2>>(L));
        t_lo = __uint_as_float(b << 16);
        t_hi = __uint_as_float((b << 16) | ((b & 0x8000u) ? 0xFFFFu : 0u));
    }
    __device__ u32 any(u32 d) const {
        return (u32)!(__uint_as_float(d) < t_hi) | (u32)!(__uint_as_float(d << 16) < t_lo);
    }
};

template <>
struct PreFilter<Elem<4>> {
    float t;
    __device__ void set(u64 L) { t = __uint_as_float(Elem<4>::bits(comp_key<Elem<4>>(L))); }
    __device__ u32 any(u32 d) const { return (u32)!(__uint_as_float(d) < t); }
};

// ------------------------------------------------------------------ shared
constexpr int kHistBits = 11;  // radix-select digit width
constexpr int kBins = 1 << kHistBits;
constexpr int kFlagBitonic = 1;  // Params::flags: always use the bitonic index sort

template <int CAP>
struct Smem {
    u64 buf[CAP];      // candidate composites
    u32 hist[kBins];   // radix-select histogram
    u64 red[16][3];    // per-wave OR / AND / MIN
    u64 L;             // admission bound: admit iff composite >= L
    u64 kth;           // k-th composite after the last compaction
    u32 count;         // entries in buf
    u32 sel_digit, sel_r, sel_c, sel_above, sel_total;
    u32 d_hi;
    u32 wsum[16];      // per-wave partial sums
    u32 nan;
    u32 last;
    u32 newtotal;
    u32 seg_count[256];  // merge: offset of each segment's list
};

// Optional instrumentation hook (phase timestamps); compiled out by default.
#ifndef DSTK_PHASE
#define DSTK_PHASE(i) ((void)0)
#endif

// ------------------------------------------------------------------ wave helpers
// Cross-lane steps use DPP (row_shr, quad_perm, row mirrors, row_bcast15/31),
// which stay in the VALU; __shfl_* would be an LDS round trip per step.
__device__ __forceinline__ u32 lane_id() { return __lane_id(); }

__device__ __forceinline__ u32 mbcnt(u64 m) {
    return __builtin_amdgcn_mbcnt_hi((u32)(m >> 32), __builtin_amdgcn_mbcnt_lo((u32)m, 0u));
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

// As wave_reserve, but never past `cap`: returns kFull (and reserves
// nothing) when the wave's entries do not fit.  Lock-free CAS by one lane.
constexpr u32 kFull = 0xFFFFFFFEu;
__device__ __forceinline__ u32 wave_reserve_cap(u32* counter, u32 c, u32 cap) {
    const u32 incl = wave_incl_scan(c);
    const u32 tot = __builtin_amdgcn_readlane(incl, 63);
    if (tot == 0) return ~0u;
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
    base = __builtin_amdgcn_readfirstlane(base);
    return base == kFull ? kFull : base + incl - c;
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

// MIN and MAX over the entries of buf[lo, hi) whose bits under `mask` equal
// `prefix` (MIN = ~0, MAX = 0 when none do).  Also zeroes the histogram for
// the block_hist_find that follows.  Separate consecutive calls by a barrier.
template <int WG, int CAP>
__device__ __forceinline__ void block_minmax(Smem<CAP>& sm, u32 lo, u32 hi, u64 prefix, u64 mask, u64& mn, u64& mx) {
    const u32 tid = threadIdx.x;
    for (u32 i = tid; i < kBins; i += WG) sm.hist[i] = 0;
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
        h[j] = sm.hist[kBins - 1 - tid * kPer - j];
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
            if (i < hi && (v[u] & mask) == prefix) atomicAdd(&sm.hist[(u32)(v[u] >> shift) & (kBins - 1)], 1u);
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
    for (u32 i = tid; i < kBins; i += WG) sm.hist[i] = 0;
    __syncthreads();
    for (u32 i = tid; i < cnt; i += WG) atomicAdd(&sm.hist[top_digit(sm.buf[i])], 1u);
    __syncthreads();
}

// Free room for `room` more entries: drop entries below the histogram
// bound's bin edge, or, if that is not enough, reduce exactly to k.
template <class E, int WG, int CAP>
__device__ __forceinline__ void make_room(Smem<CAP>& sm, u32 cnt, u32 k, u32 room) {
    const u32 tid = threadIdx.x;
    hist_locate<WG, CAP>(sm, k);
    const u32 d = sm.sel_digit, keep = sm.sel_above + sm.sel_c;
    if (sm.sel_c > 0 && keep + room <= (u32)CAP) {
        const u32 kept = keep_at_least<WG, CAP>(sm, 0, cnt, digit_floor(d));
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
__device__ __forceinline__ void final_select(Smem<CAP>& sm, u32 cnt, u32 k) {
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
// Writes the k entries of buf[0, k).  Index order, when asked for, comes
// from a bitmap of the selected columns and a prefix popcount over it (when
// the row's bitmap fits in the free LDS), else from a bitonic sort.
template <class E, int WG, int CAP>
__device__ __forceinline__ void emit(Smem<CAP>& sm, u32 k, u32 n, int sorted, int retval, int flags, int32_t* out_idx,
                     void* out_val) {
    const u32 tid = threadIdx.x;
    using VT = typename std::conditional<E::kKeyBits == 16, uint16_t, uint32_t>::type;
    VT* ov = (VT*)out_val;
    if (!sorted) {
        for (u32 i = tid; i < k; i += WG) {
            const u64 e = sm.buf[i];
            out_idx[i] = (int32_t)comp_col<E>(e);
            if (retval) ov[i] = (VT)E::bits(comp_key<E>(e));
        }
        return;
    }
    const u32 words = (n + 31) / 32;
    if (!(flags & kFlagBitonic) && (u64)k * 8 + (u64)words * 8 <= (u64)CAP * 8) {
        u32* bm = (u32*)(sm.buf + k);
        u32* pre = bm + words;
        for (u32 w = tid; w < words; w += WG) bm[w] = 0;
        __syncthreads();
        for (u32 i = tid; i < k; i += WG) {
            const u32 c = comp_col<E>(sm.buf[i]);
            atomicOr(&bm[c >> 5], 1u << (c & 31));
        }
        __syncthreads();
        const u32 per = (words + WG - 1) / WG;
        const u32 w0 = tid * per;
        u32 s = 0;
        for (u32 j = 0; j < per; ++j)
            if (w0 + j < words) s += __popc(bm[w0 + j]);
        u32 tot;
        u32 run = block_excl_scan<WG, CAP>(sm, s, &tot);
        for (u32 j = 0; j < per; ++j)
            if (w0 + j < words) {
                pre[w0 + j] = run;
                run += __popc(bm[w0 + j]);
            }
        __syncthreads();
        for (u32 i = tid; i < k; i += WG) {
            const u64 e = sm.buf[i];
            const u32 c = comp_col<E>(e);
            const u32 pos = pre[c >> 5] + __popc(bm[c >> 5] & ((1u << (c & 31)) - 1u));
            out_idx[pos] = (int32_t)c;
            if (retval) ov[pos] = (VT)E::bits(comp_key<E>(e));
        }
        return;
    }
    u32 P = 1;
    while (P < k) P <<= 1;
    for (u32 i = tid; i < P; i += WG) {
        const u64 e = i < k ? sm.buf[i] : 0ull;
        sm.buf[i] = i < k ? (((u64)comp_col<E>(e) << 32) | comp_key<E>(e)) : ~0ull;
    }
    __syncthreads();
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
            __syncthreads();
        }
    }
    for (u32 i = tid; i < k; i += WG) {
        const u64 s = sm.buf[i];
        out_idx[i] = (int32_t)(u32)(s >> 32);
        if (retval) ov[i] = (VT)E::bits((u32)s);
    }
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
    int32_t sorted;
    int32_t retval;
    int32_t* out_idx;
    void* out_val;
    u64* ws_cand;      // [batch][segs][pub_cap]: a segment's live candidates, by top digit
    u64* ws_meta;      // [batch][segs][4]: count | low digit, high digit, bound, q-bound
    u32* ws_dir;       // [batch][segs][kBins]: entries with top digit >= d, from the low digit
    u32* ws_ticket;    // [batch], zero between calls
    int32_t pub_cap;   // most candidates a segment publishes
    int32_t* flag;     // set to flag_value when a NaN is seen
    int32_t flag_value;
    int32_t flags;     // kFlag* bits
};

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
    __device__ static __forceinline__ void get(const uint4 (&v)[VPT], int s, int vb, u32 tid, int v1, u32 n,
                                               u32& bits, u32& col, bool& valid) {
        const int j = s / E::kPerVec;
        const int w = (s % E::kPerVec) / kPerDword;
        const int hh = s % kPerDword;
        const u32 d = w == 0 ? v[j].x : w == 1 ? v[j].y : w == 2 ? v[j].z : v[j].w;
        bits = kPerDword == 2 ? ((d >> (16 * hh)) & 0xFFFFu) : d;
        const int vi = vb + j * WG + (int)tid;
        col = (u32)vi * E::kPerVec + (u32)(w * kPerDword + hh);
        valid = vi < v1 && col < n;
    }
};

// One workgroup per (row, segment).  EB: element bytes; WG: threads; NV:
// tiles per chunk (16-byte loads each thread has in flight); CAP:
// candidate-buffer entries.
// A "tile" is one vector per thread, WG * 16 bytes; tiles are visited in a
// pseudo-random order, a chunk at a time.
template <int EB, int WG, int NV, int CAP>
__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu((CAP <= 8192 ? 2 : 1) * WG / 256)))
void topk_rows(Params p) {
    using E = Elem<EB>;
    using SL = Slot<E, 1, WG>;
    constexpr int kTileVecs = WG;
    constexpr int kTileElems = kTileVecs * E::kPerVec;
    static_assert(CAP % WG == 0, "capacity must be a multiple of the workgroup size");
    static_assert(CAP >= 2 * NV * kTileElems || NV * kTileElems >= 8192, "capacity must hold two chunks");
    __shared__ Smem<CAP> sm;

    const u32 tid = threadIdx.x;
    const u32 row = blockIdx.x / (u32)p.segs;
    const u32 seg = blockIdx.x % (u32)p.segs;
    const u32 k = (u32)p.k;
    const u32 n = (u32)p.n;
    const uint8_t* row_in = p.in + (int64_t)row * p.row_stride_bytes;

    const int v0 = (int)seg * p.seg_vecs;
    const int v1 = min(p.n_vec, v0 + p.seg_vecs);
    // The segment as a raw buffer resource: loads take one 32-bit offset
    // (vector index relative to v0, times 16) and the hardware range check
    // returns zeros past the segment's end instead of faulting.
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(row_in + (int64_t)v0 * 16), (short)0, (int)((u32)(v1 - v0) * 16u), kBufferWord3);
    auto load_vec = [&](int vi) -> uint4 {  // vi: absolute vector index in the row
        const auto r = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (u32)(vi - v0) * 16u, 0, 0);
        return uint4{r[0], r[1], r[2], r[3]};
    };
    const u32 ntiles = (u32)((v1 - v0 + kTileVecs - 1) / kTileVecs);

    // Tile visiting order: t -> (a t + b) mod ntiles with gcd(a, ntiles) = 1.
    const u32 h = hash32(blockIdx.x * 0x9E3779B9u ^ p.seed);
    u32 a = 1, b = 0;
    if (ntiles > 1) {
        a = (u32)(((u64)ntiles * 0x9E3779B9ull) >> 32) | 1u;
        if (a >= ntiles) a = 1;
        while (gcd_u32(a, ntiles) != 1) ++a;
        b = h % ntiles;
    }

    for (u32 i = tid; i < kBins; i += WG) sm.hist[i] = 0;
    if (tid == 0) {
        sm.count = 0;
        sm.L = 0;
        sm.nan = 0;
        sm.last = 0;
    }
    DSTK_PHASE(0);

    PreFilter<E> pf;
    u64 L = 0;
    pf.set(L);
    bool saw_nan = false;
    __syncthreads();

    u32 pr = b;  // permuted index of the next tile to request
    constexpr int kSeed = NV < 2 ? NV : 2;  // tiles counted to seed the bound
    static_assert(CAP >= kSeed * kTileElems, "the seed tiles must fit an empty buffer");

    // Filter one tile (one vector per thread) against the bound, appending
    // admitted elements and counting them in the histogram.  Returns false,
    // appending nothing, when the wave's admitted elements do not fit.
    auto filter = [&](const uint4& x, int vbi) -> bool {
        const u32 any = pf.any(x.x) | pf.any(x.y) | pf.any(x.z) | pf.any(x.w);
        if (__ballot(any != 0) == 0) return true;
        const uint4 xs[1] = {x};
        u32 pm = 0, c = 0;
#pragma unroll
        for (int s = 0; s < SL::kSlots; ++s) {
            u32 bits, col;
            bool valid;
            SL::get(xs, s, vbi, tid, v1, n, bits, col, valid);
            saw_nan |= valid && E::is_nan(bits);
            const bool ok = valid && compose<E>(E::key(bits), col) >= L;
            pm |= (u32)ok << s;
            c += ok;
        }
        u32 pos = wave_reserve_cap(&sm.count, c, (u32)CAP);
        if (pos == kFull) return false;
        if (pos != ~0u) {
#pragma unroll
            for (int s = 0; s < SL::kSlots; ++s) {
                if ((pm >> s) & 1u) {
                    u32 bits, col;
                    bool valid;
                    SL::get(xs, s, vbi, tid, v1, n, bits, col, valid);
                    const u64 e = compose<E>(E::key(bits), col);
                    sm.buf[pos++] = e;
                    atomicAdd(&sm.hist[top_digit(e)], 1u);
                }
            }
        }
        return true;
    };

    // Phase A, per chunk of NV tiles: all NV loads requested at once and
    // filtered in request order (straight-line code, so each tile waits only
    // for its own load; lanes past the segment read zeros and are masked out).  After the seed, filtering
    // takes no workgroup barrier: waves run independently and hide each
    // other's load latency.  A wave whose entries do not fit records the
    // tile; phase B makes room and filters those tiles again.
    for (u32 t0 = 0; t0 < ntiles; t0 += NV) {
        uint4 v[NV];
        int vb[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            vb[i] = t0 + (u32)i < ntiles ? v0 + (int)pr * kTileVecs : v1;
            v[i] = load_vec(vb[i] + (int)tid);
            __builtin_amdgcn_sched_barrier(0);  // keep requests in slot order
            pr += a;
            if (pr >= ntiles) pr -= ntiles;
        }
        u32 pending = 0;  // wave-uniform: tiles this wave still has to append
        if (t0 == 0) {
            // Seed: count every element of the first kSeed tiles, take the
            // bin edge of the k-th counted as the bound, then admit those
            // tiles' elements at or above it (they always fit).
#pragma unroll
            for (int i = 0; i < kSeed; ++i) {
                const uint4 xs[1] = {v[i]};
#pragma unroll
                for (int s = 0; s < SL::kSlots; ++s) {
                    u32 bits, col;
                    bool valid;
                    SL::get(xs, s, vb[i], tid, v1, n, bits, col, valid);
                    if (valid) {
                        saw_nan |= E::is_nan(bits);
                        atomicAdd(&sm.hist[top_digit(compose<E>(E::key(bits), col))], 1u);
                    }
                }
            }
            __syncthreads();
            hist_locate<WG, CAP>(sm, k);
            if (sm.sel_c > 0) L = digit_floor(sm.sel_digit);
            pf.set(L);
#pragma unroll
            for (int i = 0; i < kSeed; ++i) {
                const uint4 xs[1] = {v[i]};
                u32 pm = 0, c = 0;
#pragma unroll
                for (int s = 0; s < SL::kSlots; ++s) {
                    u32 bits, col;
                    bool valid;
                    SL::get(xs, s, vb[i], tid, v1, n, bits, col, valid);
                    const bool ok = valid && compose<E>(E::key(bits), col) >= L;
                    pm |= (u32)ok << s;
                    c += ok;
                }
                u32 pos = wave_reserve(&sm.count, c);
                if (pos != ~0u) {
#pragma unroll
                    for (int s = 0; s < SL::kSlots; ++s) {
                        if ((pm >> s) & 1u) {
                            u32 bits, col;
                            bool valid;
                            SL::get(xs, s, vb[i], tid, v1, n, bits, col, valid);
                            sm.buf[pos++] = compose<E>(E::key(bits), col);
                        }
                    }
                }
            }
#pragma unroll
            for (int i = kSeed; i < NV; ++i)
                if (!filter(v[i], vb[i])) pending |= 1u << i;
        } else {
#pragma unroll
            for (int i = 0; i < NV; ++i)
                if (!filter(v[i], vb[i])) pending |= 1u << i;
        }

        // Phase B (rare): make room, raise the bound, filter what did not fit.
        for (int round = 0; round < 64; ++round) {
            __syncthreads();
            if (lane_id() == 0 && pending) atomicOr(&sm.last, 1u);
            __syncthreads();
            const bool again = sm.last != 0;
            __syncthreads();
            if (!again) break;
            if (tid == 0) sm.last = 0;
            make_room<E, WG, CAP>(sm, sm.count, k, kTileElems);
            hist_locate<WG, CAP>(sm, k);
            if (sm.sel_c > 0 && digit_floor(sm.sel_digit) > L) L = digit_floor(sm.sel_digit);
            if (sm.L > L) L = sm.L;
            pf.set(L);
            const u32 todo = pending;
            pending = 0;
            for (int i = 0; i < NV; ++i) {
                if ((todo >> i) & 1u) {
                    const uint4 x = load_vec(vb[i] + (int)tid);  // cached: read moments ago
                    if (!filter(x, vb[i])) pending |= 1u << i;
                }
            }
        }
        // Between chunks (long segments only): tidy up and raise the bound.
        if (t0 + NV < ntiles) {
            if (sm.count > (u32)CAP / 2) make_room<E, WG, CAP>(sm, sm.count, k, 0);
            hist_locate<WG, CAP>(sm, k);
            if (sm.sel_c > 0 && digit_floor(sm.sel_digit) > L) L = digit_floor(sm.sel_digit);
            if (sm.L > L) L = sm.L;
            pf.set(L);
        }
    }
    if (saw_nan) sm.nan = 1;  // benign race: every writer stores 1
    if (tid == 0) sm.L = L;
    DSTK_PHASE(1);
    __syncthreads();
    u32 cnt = sm.count;

    if (p.segs == 1) {
        final_select<E, WG, CAP>(sm, cnt, k);
        DSTK_PHASE(2);
        emit<E, WG, CAP>(sm, k, n, p.sorted, p.retval, p.flags, p.out_idx + (int64_t)row * k,
                         p.retval ? (void*)((uint8_t*)p.out_val + (int64_t)row * k * EB) : nullptr);
        __syncthreads();
        if (tid == 0 && sm.nan) *p.flag = p.flag_value;
        DSTK_PHASE(6);
        return;
    }

    // ---- split row: publish this segment's live candidates, sorted by top
    // digit, with a directory of cumulative counts per digit.
    const u32 S = (u32)p.segs;
    const u32 slot = row * S + seg;
    {
        // bound for rank q = ceil(k / S): with every segment's list holding
        // q entries at or above its own such bound, the smallest of them is
        // a valid bound for the row
        const u32 q = (k + S - 1) / S;
        hist_locate<WG, CAP>(sm, q);
        const u64 bq = sm.sel_c > 0 ? digit_floor(sm.sel_digit) : 0ull;
        hist_locate<WG, CAP>(sm, k);
        u32 dl = sm.sel_c > 0 ? sm.sel_digit : 0u;
        u32 live = sm.sel_c > 0 ? sm.sel_above + sm.sel_c : sm.sel_total;
        if (live > (u32)p.pub_cap) {
            // too many to publish: reduce this segment exactly to k first
            compact_to_k<E, WG, CAP>(sm, cnt, k);
            rebuild_hist<WG, CAP>(sm, k);
            cnt = k;
            hist_locate<WG, CAP>(sm, k);
            dl = sm.sel_digit;
            live = sm.sel_above + sm.sel_c;
            if (L < sm.L) L = sm.L;
        }
        // hist[d] -> number of live entries in higher bins (for d >= dl);
        // directory: entries with digit >= d, written for d in [dl, d_hi]
        constexpr int kPer = kBins / WG;
        u32 hv[kPer];
        u32 sum = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const u32 d = kBins - 1 - tid * kPer - j;
            hv[j] = d >= dl ? sm.hist[d] : 0u;
            sum += hv[j];
        }
        u32 tot;
        u32 run = block_excl_scan<WG, CAP>(sm, sum, &tot);
        u32* dir = p.ws_dir + (u64)slot * kBins;
        if (run == 0 && sum > 0) {
#pragma unroll
            for (int j = kPer - 1; j >= 0; --j)
                if (hv[j]) sm.d_hi = kBins - 1 - tid * kPer - j;
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const u32 d = kBins - 1 - tid * kPer - j;
            if (d >= dl) {
                sm.hist[d] = run;
                run += hv[j];
                if (run > 0) dir[d - dl] = run;
            }
        }
        __syncthreads();
        u64* cand = p.ws_cand + (u64)slot * (u32)p.pub_cap;
        constexpr int kItems = CAP / WG;
        u64 mine[kItems];
        u32 at[kItems];
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            const u32 i = tid + j * WG;
            mine[j] = i < cnt ? sm.buf[i] : 0ull;
            at[j] = (i < cnt && top_digit(mine[j]) >= dl) ? atomicAdd(&sm.hist[top_digit(mine[j])], 1u) : ~0u;
        }
#pragma unroll
        for (int j = 0; j < kItems; ++j)
            if (at[j] != ~0u) cand[at[j]] = mine[j];
        if (tid == 0) {
            u64* meta = p.ws_meta + (u64)slot * 4;
            meta[0] = (u64)live | ((u64)dl << 32);
            meta[1] = (u64)(live ? sm.d_hi : 0u);
            meta[2] = L;
            meta[3] = bq;
        }
    }
    DSTK_PHASE(2);
    __syncthreads();
    if (tid == 0) {
        // release this workgroup's stores (ordered before by the barrier) to
        // the device, then take a ticket; the last ticket merges
        __threadfence();
        const u32 prev = atomicAdd(&p.ws_ticket[row], 1u);
        sm.last = prev == S - 1;
        if (sm.last) __threadfence();
    }
    __syncthreads();
    if (!sm.last) {
        if (tid == 0 && sm.nan) *p.flag = p.flag_value;
        DSTK_PHASE(3);
        return;
    }
    DSTK_PHASE(4);

    // Merge.  Every element of the row's top-k is among some segment's live
    // list.  Bounds: a segment with at least k elements has k of them at or
    // above its bound; every segment has q = ceil(k/S) at or above its
    // q-bound, so the smallest q-bound over the row is valid as well.
    const u32 cap = (u32)p.pub_cap;
    const u64* rc = p.ws_cand + (u64)row * S * cap;
    for (u32 i = tid; i < kBins; i += WG) sm.hist[i] = 0;
    {
        u64 m0 = 0, m1 = 0, m2 = 0, m3 = ~0ull;
        if (tid < S) {
            const u64* meta = p.ws_meta + (u64)(row * S + tid) * 4;
            m0 = meta[0];
            m1 = meta[1];
            m2 = meta[2];
            m3 = meta[3];
        }
        // row bound: max over segment bounds, max with min over q-bounds
        u64 vmax = wave_max64(m2), vmin = wave_min64(m3);
        const u32 wave = tid / kWave;
        if (lane_id() == 0) {
            sm.red[wave][0] = vmax;
            sm.red[wave][1] = vmin;
        }
        __syncthreads();
        u64 lmax = 0, qmin = ~0ull;
#pragma unroll
        for (u32 w = 0; w < WG / kWave; ++w) {
            lmax = sm.red[w][0] > lmax ? sm.red[w][0] : lmax;
            qmin = sm.red[w][1] < qmin ? sm.red[w][1] : qmin;
        }
        L = lmax > qmin ? lmax : qmin;
        const u32 df = top_digit(L);
        u32 m = 0;
        if (tid < S) {
            const u32 live = (u32)m0, dl = (u32)(m0 >> 32), dh = (u32)m1;
            if (live == 0 || df > dh) m = 0;
            else if (df <= dl) m = live;
            else m = p.ws_dir[(u64)(row * S + tid) * kBins + (df - dl)];
        }
        u32 total;
        const u32 off = block_excl_scan<WG, CAP>(sm, m, &total);
        if (tid < S) sm.seg_count[tid] = off;
        if (tid == 0) {
            sm.newtotal = total;
            sm.count = 0;
            p.ws_ticket[row] = 0;  // ready for the next call
        }
        __syncthreads();
    }
    const u32 total = sm.newtotal;
    constexpr int kMI = kTileElems / WG;  // merge entries per thread per step
    for (u32 base = 0; base < total; base += WG * kMI) {
        u64 e[kMI];
        u32 pm = 0, c = 0;
#pragma unroll
        for (int j = 0; j < kMI; ++j) {
            const u32 f = base + j * WG + tid;
            e[j] = 0;
            if (f < total) {
                u32 lo = 0, hi = S;  // last segment whose offset is <= f
                while (hi - lo > 1) {
                    const u32 mid = (lo + hi) >> 1;
                    if (sm.seg_count[mid] <= f) lo = mid; else hi = mid;
                }
                e[j] = rc[(u64)lo * cap + (f - sm.seg_count[lo])];
            }
            const bool ok = f < total && e[j] >= L;
            pm |= (u32)ok << j;
            c += ok;
        }
        u32 pos = wave_reserve(&sm.count, c);
        if (pos != ~0u) {
#pragma unroll
            for (int j = 0; j < kMI; ++j)
                if ((pm >> j) & 1u) {
                    sm.buf[pos++] = e[j];
                    atomicAdd(&sm.hist[top_digit(e[j])], 1u);
                }
        }
        __syncthreads();
        const u32 c2 = sm.count;
        if (c2 > (u32)(CAP - kTileElems)) make_room<E, WG, CAP>(sm, c2, k, kTileElems);
    }
    cnt = sm.count;
    final_select<E, WG, CAP>(sm, cnt, k);
    DSTK_PHASE(5);
    emit<E, WG, CAP>(sm, k, n, p.sorted, p.retval, p.flags, p.out_idx + (int64_t)row * k,
                     p.retval ? (void*)((uint8_t*)p.out_val + (int64_t)row * k * EB) : nullptr);
    __syncthreads();
    if (tid == 0 && sm.nan) *p.flag = p.flag_value;
    DSTK_PHASE(6);
}

}  // namespace dstk
