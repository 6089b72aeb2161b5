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
    u32 sel_digit, sel_r, sel_c, sel_above;
    u32 wsum[16];      // per-wave partial sums
    u32 nan;
    u32 last;
    u32 seg_count[256];  // merge: entries per segment
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
DSTK_WAVE_REDUCE(wave_or, (v | t), 0u)
DSTK_WAVE_REDUCE(wave_and, (v & t), 0xFFFFFFFFu)
DSTK_WAVE_REDUCE(wave_min, (t < v ? t : v), 0xFFFFFFFFu)
#undef DSTK_WAVE_REDUCE

__device__ __forceinline__ u64 wave_or64(u64 v) { return ((u64)wave_or((u32)(v >> 32)) << 32) | wave_or((u32)v); }
__device__ __forceinline__ u64 wave_and64(u64 v) {
    return ((u64)wave_and((u32)(v >> 32)) << 32) | wave_and((u32)v);
}
__device__ __forceinline__ u64 wave_min64(u64 v) {
    const u32 hi = wave_min((u32)(v >> 32));
    const u32 lo = wave_min((u32)(v >> 32) == hi ? (u32)v : 0xFFFFFFFFu);
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

// ------------------------------------------------------------------ block helpers
// Exclusive prefix sum of one value per thread, in thread order; *total gets
// the block sum.  Separate consecutive calls by a barrier.
template <int WG, int CAP>
__device__ u32 block_excl_scan(Smem<CAP>& sm, u32 v, u32* total) {
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

// OR, AND and MIN over the entries of buf[lo, hi) whose bits under `mask`
// equal `prefix`.  Separate consecutive calls by a barrier.
template <int WG, int CAP>
__device__ void block_reduce(Smem<CAP>& sm, u32 lo, u32 hi, u64 prefix, u64 mask, u64& o, u64& a, u64& mn) {
    const u32 tid = threadIdx.x;
    u64 vo = 0, va = ~0ull, vm = ~0ull;
    for (u32 i = lo + tid; i < hi; i += WG) {
        const u64 e = sm.buf[i];
        if ((e & mask) == prefix) {
            vo |= e;
            va &= e;
            vm = e < vm ? e : vm;
        }
    }
    vo = wave_or64(vo);
    va = wave_and64(va);
    vm = wave_min64(vm);
    const u32 wave = tid / kWave;
    if (lane_id() == 0) {
        sm.red[wave][0] = vo;
        sm.red[wave][1] = va;
        sm.red[wave][2] = vm;
    }
    __syncthreads();
    o = 0;
    a = ~0ull;
    mn = ~0ull;
#pragma unroll
    for (u32 w = 0; w < WG / kWave; ++w) {
        o |= sm.red[w][0];
        a &= sm.red[w][1];
        mn = sm.red[w][2] < mn ? sm.red[w][2] : mn;
    }
}

// Histogram of the digit (e >> shift) & (kBins-1) over the entries of
// buf[lo, hi) matching (prefix, mask); then the bin holding the r-th largest
// (r >= 1).  Leaves sel_digit, sel_r (rank inside the bin), sel_c (bin size)
// and sel_above (entries in higher bins) in shared memory.
template <int WG, int CAP>
__device__ void block_hist_find(Smem<CAP>& sm, u32 lo, u32 hi, u64 prefix, u64 mask, int shift, u32 r) {
    const u32 tid = threadIdx.x;
    for (u32 i = tid; i < kBins; i += WG) sm.hist[i] = 0;
    if (tid == 0) {  // overwritten below unless r exceeds the matching count
        sm.sel_digit = 0;
        sm.sel_r = 0;
        sm.sel_c = 0;
        sm.sel_above = 0;
    }
    __syncthreads();
    for (u32 i = lo + tid; i < hi; i += WG) {
        const u64 e = sm.buf[i];
        if ((e & mask) == prefix) atomicAdd(&sm.hist[(u32)(e >> shift) & (kBins - 1)], 1u);
    }
    __syncthreads();
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

// Window of kHistBits bits whose top bit is the highest bit set in diff.
__device__ __forceinline__ int window_shift(u64 diff) {
    const int msb = 63 - __clzll((long long)diff);
    return msb >= kHistBits - 1 ? msb - (kHistBits - 1) : 0;
}
__device__ __forceinline__ u64 bits_above(int shift) {
    return shift + kHistBits >= 64 ? 0ull : (~0ull << (shift + kHistBits));
}

// ------------------------------------------------------------------ compaction
// Reduce buf[0, cnt) (distinct composites, cnt > k) to its k largest, in
// buf[0, k); sets kth (the least kept) and L = kth + 1.
//
// Radix select with 11-bit digits.  Each level's window starts at the
// highest bit where the still-undecided entries differ, so concentrated
// value distributions still spread over the bins.  After the first level
// the buffer is partitioned once: entries in higher bins are kept outright,
// the boundary bin is moved next to them, and later levels only look at that
// boundary list.  Placement uses block prefix sums, not atomics, so the
// result order is a deterministic function of the buffer order.
template <class E, int WG, int CAP>
__device__ void compact_to_k(Smem<CAP>& sm, u32 cnt, u32 k) {
    const u32 tid = threadIdx.x;
    constexpr int kItems = CAP / WG;
    u64 o, a, mn;
    block_reduce<WG, CAP>(sm, 0, cnt, 0ull, 0ull, o, a, mn);
    int shift = window_shift(o ^ a);
    u64 mask = bits_above(shift);
    u64 prefix = a & mask;
    block_hist_find<WG, CAP>(sm, 0, cnt, prefix, mask, shift, k);
    const u32 b = sm.sel_digit, above = sm.sel_above, c = sm.sel_c;
    u32 r = sm.sel_r;

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
    u64 T;
    if (r == c) {
        block_reduce<WG, CAP>(sm, lo, hi, prefix, mask, o, a, mn);
        T = mn;
    } else {
        // Each level fixes at least one more bit, so 64 / kHistBits + 1
        // levels always suffice; the bound only guards the loop.
        T = 0;
        for (int level = 0; level < 64 / kHistBits + 2; ++level) {
            block_reduce<WG, CAP>(sm, lo, hi, prefix, mask, o, a, mn);
            shift = window_shift(o ^ a);
            // Keep the bits fixed so far: a window clamped at bit 0 can
            // overlap them.
            mask |= bits_above(shift);
            prefix = a & mask;
            block_hist_find<WG, CAP>(sm, lo, hi, prefix, mask, shift, r);
            const u32 d2 = sm.sel_digit, c2 = sm.sel_c, r2 = sm.sel_r;
            prefix |= (u64)d2 << shift;
            mask |= (u64)(kBins - 1) << shift;
            if (r2 == c2) {
                block_reduce<WG, CAP>(sm, lo, hi, prefix, mask, o, a, mn);
                T = mn;
                break;
            }
            r = r2;
        }
        // keep the boundary entries >= T, packed right after the definite ones
        u32 nk = 0;
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            const u32 i = lo + tid + j * WG;
            mine[j] = i < hi ? sm.buf[i] : 0ull;
            nk += (i < hi && mine[j] >= T) ? 1u : 0u;
        }
        __syncthreads();  // wsum reuse
        u32 pk = lo + block_excl_scan<WG, CAP>(sm, nk, &tot);
#pragma unroll
        for (int j = 0; j < kItems; ++j) {
            const u32 i = lo + tid + j * WG;
            if (i < hi && mine[j] >= T) sm.buf[pk++] = mine[j];
        }
    }
    if (tid == 0) {
        sm.count = k;
        sm.kth = T;
        sm.L = T + 1;
    }
    __syncthreads();
}

// ------------------------------------------------------------------ output
// Writes the k entries of buf[0, k).  Index order, when asked for, comes
// from a bitmap of the selected columns and a prefix popcount over it (when
// the row's bitmap fits in the free LDS), else from a bitonic sort.
template <class E, int WG, int CAP>
__device__ void emit(Smem<CAP>& sm, u32 k, u32 n, int sorted, int retval, int flags, int32_t* out_idx,
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
    int32_t idx_bits;  // columns < 2^idx_bits
    uint32_t seed;
    int32_t sorted;
    int32_t retval;
    int32_t* out_idx;
    void* out_val;
    u64* ws_cand;      // [batch][segs][k]
    u64* ws_kth;       // [batch][segs]
    u32* ws_count;     // [batch][segs]
    u32* ws_ticket;    // [batch], zero between calls
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

template <int EB, int WG, int VPT, int CAP>
__global__ __launch_bounds__(WG) void topk_rows(Params p) {
    using E = Elem<EB>;
    constexpr int kTileVecs = WG * VPT;
    constexpr int kTileElems = kTileVecs * E::kPerVec;
    static_assert(CAP % WG == 0, "capacity must be a multiple of the workgroup size");
    __shared__ Smem<CAP> sm;

    const u32 tid = threadIdx.x;
    const u32 row = blockIdx.x / (u32)p.segs;
    const u32 seg = blockIdx.x % (u32)p.segs;
    const u32 k = (u32)p.k;
    const uint4* vin = (const uint4*)(p.in + (int64_t)row * p.row_stride_bytes);

    const int v0 = (int)seg * p.seg_vecs;
    const int v1 = min(p.n_vec, v0 + p.seg_vecs);
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

    if (tid == 0) {
        sm.count = 0;
        sm.L = 0;
        sm.kth = 0;
        sm.nan = 0;
    }
    DSTK_PHASE(0);
    __syncthreads();

    PreFilter<E> pf;
    u64 L = 0;
    pf.set(L);
    bool saw_nan = false;

    uint4 cur[VPT], nxt[VPT];
    auto load_tile = [&](uint4 (&v)[VPT], u32 t) {
        const int vb = v0 + (int)(((u64)a * t + b) % ntiles) * kTileVecs;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int vi = vb + j * WG + (int)tid;
            v[j] = vi < v1 ? vin[vi] : make_uint4(0u, 0u, 0u, 0u);
        }
    };

    load_tile(cur, 0);
    for (u32 t = 0; t < ntiles; ++t) {
        if (t + 1 < ntiles) load_tile(nxt, t + 1);
        const int vb = v0 + (int)(((u64)a * t + b) % ntiles) * kTileVecs;
        u32 any = 0;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            any |= pf.any(cur[j].x) | pf.any(cur[j].y) | pf.any(cur[j].z) | pf.any(cur[j].w);
        }
        if (__ballot(any != 0) != 0) {
            // Exact test on every element slot; one LDS reservation per wave.
            constexpr int kSlots = VPT * E::kPerVec;
            constexpr int kPerDword = EB == 2 ? 2 : 1;
            u32 pm = 0, c = 0;
#pragma unroll
            for (int s = 0; s < kSlots; ++s) {
                const int j = s / E::kPerVec;
                const int w = (s % E::kPerVec) / kPerDword;
                const int hh = s % kPerDword;
                const u32 d = w == 0 ? cur[j].x : w == 1 ? cur[j].y : w == 2 ? cur[j].z : cur[j].w;
                const u32 bits = EB == 2 ? ((d >> (16 * hh)) & 0xFFFFu) : d;
                const int vi = vb + j * WG + (int)tid;
                const u32 col = (u32)vi * E::kPerVec + (u32)(w * kPerDword + hh);
                const bool valid = vi < v1 && col < (u32)p.n;
                saw_nan |= valid && E::is_nan(bits);
                const bool ok = valid && compose<E>(E::key(bits), col) >= L;
                pm |= (u32)ok << s;
                c += ok;
            }
            u32 pos = wave_reserve(&sm.count, c);
            if (pos != ~0u) {
#pragma unroll
                for (int s = 0; s < kSlots; ++s) {
                    if ((pm >> s) & 1u) {
                        const int j = s / E::kPerVec;
                        const int w = (s % E::kPerVec) / kPerDword;
                        const int hh = s % kPerDword;
                        const u32 d = w == 0 ? cur[j].x : w == 1 ? cur[j].y : w == 2 ? cur[j].z : cur[j].w;
                        const u32 bits = EB == 2 ? ((d >> (16 * hh)) & 0xFFFFu) : d;
                        const int vi = vb + j * WG + (int)tid;
                        const u32 col = (u32)vi * E::kPerVec + (u32)(w * kPerDword + hh);
                        sm.buf[pos++] = compose<E>(E::key(bits), col);
                    }
                }
            }
        }
        __syncthreads();
        const u32 cnt = sm.count;
        if (cnt > (u32)(CAP - kTileElems)) {
            compact_to_k<E, WG, CAP>(sm, cnt, k);
            L = sm.L;
            pf.set(L);
        }
#pragma unroll
        for (int j = 0; j < VPT; ++j) cur[j] = nxt[j];
    }

    DSTK_PHASE(1);
    // Final reduction of this segment to at most k entries.
    u32 cnt = sm.count;
    if (cnt > k) {
        compact_to_k<E, WG, CAP>(sm, cnt, k);
        cnt = k;
    } else if (cnt == k && p.segs > 1) {
        // k-th = least entry; a valid lower bound for the whole row
        u64 o, a, mn;
        block_reduce<WG, CAP>(sm, 0, cnt, 0ull, 0ull, o, a, mn);
        if (tid == 0) sm.kth = mn;
        __syncthreads();
    }
    DSTK_PHASE(2);

    if (saw_nan) sm.nan = 1;  // benign race: every writer stores 1

    if (p.segs == 1) {
        emit<E, WG, CAP>(sm, k, (u32)p.n, p.sorted, p.retval, p.flags, p.out_idx + (int64_t)row * k,
                         p.retval ? (void*)((uint8_t*)p.out_val + (int64_t)row * k * EB) : nullptr);
        __syncthreads();
        if (tid == 0 && sm.nan) *p.flag = p.flag_value;
        DSTK_PHASE(6);
        return;
    }

    // ---- split row: publish this segment's survivors, last arriver merges
    const u32 slot = row * (u32)p.segs + seg;
    u64* cand = p.ws_cand + (u64)slot * k;
    for (u32 i = tid; i < cnt; i += WG) cand[i] = sm.buf[i];
    if (tid == 0) {
        p.ws_count[slot] = cnt;
        p.ws_kth[slot] = cnt == k ? sm.kth : 0ull;
    }
    __syncthreads();
    if (tid == 0) {
        // release this workgroup's stores (ordered before by the barrier) to
        // the device, then take a ticket; the last ticket merges
        __threadfence();
        const u32 prev = atomicAdd(&p.ws_ticket[row], 1u);
        sm.last = prev == (u32)p.segs - 1;
        if (sm.last) __threadfence();
    }
    __syncthreads();
    if (!sm.last) {
        if (tid == 0 && sm.nan) *p.flag = p.flag_value;
        DSTK_PHASE(3);
        return;
    }
    DSTK_PHASE(4);

    // Merge: every element of the row's top-k is in some segment's list, and
    // no segment's k-th composite exceeds the row's k-th, so the largest of
    // them is a valid admission bound.
    const u32 S = (u32)p.segs;
    const u64* rc = p.ws_cand + (u64)row * S * k;
    for (u32 s = tid; s < S; s += WG) sm.seg_count[s] = p.ws_count[row * S + s];
    if (tid < kWave) {
        u64 mx = 0;
        for (u32 s = tid; s < S; s += kWave) {
            const u64 v = p.ws_kth[row * S + s];
            mx = v > mx ? v : mx;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const u64 t = __shfl_xor(mx, o, kWave);
            mx = t > mx ? t : mx;
        }
        if (tid == 0) {
            sm.L = mx;
            sm.count = 0;
            p.ws_ticket[row] = 0;  // ready for the next call
        }
    }
    __syncthreads();
    L = sm.L;
    constexpr int kMI = kTileElems / WG;  // merge entries per thread per step
    const u32 total = S * k;
    for (u32 base = 0; base < total; base += WG * kMI) {
        u64 e[kMI];
        u32 pm = 0, c = 0;
#pragma unroll
        for (int j = 0; j < kMI; ++j) {
            const u32 f = base + j * WG + tid;
            e[j] = 0;
            if (f < total) {
                const u32 s = f / k, jj = f - s * k;
                if (jj < sm.seg_count[s]) e[j] = rc[f];
            }
            const bool ok = e[j] != 0 && e[j] >= L;  // composites of real elements are nonzero
            pm |= (u32)ok << j;
            c += ok;
        }
        u32 pos = wave_reserve(&sm.count, c);
        if (pos != ~0u) {
#pragma unroll
            for (int j = 0; j < kMI; ++j)
                if ((pm >> j) & 1u) sm.buf[pos++] = e[j];
        }
        __syncthreads();
        const u32 c2 = sm.count;
        if (c2 > (u32)(CAP - kTileElems)) {
            compact_to_k<E, WG, CAP>(sm, c2, k);
            L = sm.L;
        }
    }
    cnt = sm.count;
    if (cnt > k) compact_to_k<E, WG, CAP>(sm, cnt, k);
    DSTK_PHASE(5);
    emit<E, WG, CAP>(sm, k, (u32)p.n, p.sorted, p.retval, p.flags, p.out_idx + (int64_t)row * k,
                     p.retval ? (void*)((uint8_t*)p.out_val + (int64_t)row * k * EB) : nullptr);
    __syncthreads();
    if (tid == 0 && sm.nan) *p.flag = p.flag_value;
    DSTK_PHASE(6);
}

}  // namespace dstk
