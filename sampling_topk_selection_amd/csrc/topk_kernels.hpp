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
template <int CAP>
struct Smem {
    u64 buf[CAP];     // candidate composites
    u32 hist[256];    // radix-select histogram
    u64 L;            // admission bound: admit iff composite >= L
    u64 kth;          // k-th composite after the last compaction
    u64 tmin;
    u32 count;        // entries in buf
    u32 newcount;
    u32 sel_digit, sel_r, sel_c;
    u32 nan;
    u32 last;
    u32 seg_count[256];  // merge: entries per segment
};

// ------------------------------------------------------------------ wave helpers
__device__ __forceinline__ u32 lane_id() { return __lane_id(); }

__device__ __forceinline__ u32 mbcnt(u64 m) {
    return __builtin_amdgcn_mbcnt_hi((u32)(m >> 32), __builtin_amdgcn_mbcnt_lo((u32)m, 0u));
}

__device__ __forceinline__ u32 wave_incl_scan(u32 v) {
    const u32 lane = lane_id();
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        u32 t = __shfl_up(v, o, kWave);
        if (lane >= (u32)o) v += t;
    }
    return v;
}

__device__ __forceinline__ u64 wave_min_u64(u64 v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        u64 t = __shfl_xor(v, o, kWave);
        v = t < v ? t : v;
    }
    return v;
}

// Append v (where pred) to buf, one LDS atomic per wave.
__device__ __forceinline__ void wave_append(u64* buf, u32* counter, u64 v, bool pred) {
    const u64 m = __ballot(pred);
    if (m == 0) return;
    u32 base = 0;
    if (lane_id() == 0) base = atomicAdd(counter, (u32)__popcll(m));
    base = __builtin_amdgcn_readfirstlane(base);
    if (pred) buf[base + mbcnt(m)] = v;
}

// ------------------------------------------------------------------ radix select
// The r-th largest (r >= 1) of the distinct composites buf[0, cnt).  MSD
// radix over 8-bit digits: first the value-key bits, then the column bits
// that can differ (column < 2^idx_bits).  Stops as soon as the bin holding
// the answer is needed whole; the answer is then that bin's minimum.
template <class E, int WG, int CAP>
__device__ u64 select_rth(Smem<CAP>& sm, u32 cnt, u32 r, int idx_bits) {
    const u32 tid = threadIdx.x;
    const int key_lo = 64 - E::kKeyBits;
    u64 prefix = 0, mask = 0;
    int hi = 64;
    for (;;) {
        int width, shift;
        if (hi > key_lo) {
            width = 8;
            shift = hi - 8;
        } else {
            if (hi == key_lo) {
                // ~column has all-one bits above idx_bits for every entry
                const u64 ones = idx_bits >= 32 ? 0ull
                                                : ((((u64)1 << (32 - idx_bits)) - 1) << (E::kIdxShift + idx_bits));
                prefix |= ones;
                mask |= ones;
                hi = E::kIdxShift + idx_bits;
            }
            if (hi <= E::kIdxShift) break;  // unreachable for distinct entries
            width = hi - E::kIdxShift < 8 ? hi - E::kIdxShift : 8;
            shift = hi - width;
        }
        for (u32 i = tid; i < 256; i += WG) sm.hist[i] = 0;
        __syncthreads();
        const u32 wmask = (1u << width) - 1u;
        for (u32 i = tid; i < cnt; i += WG) {
            const u64 e = sm.buf[i];
            if ((e & mask) == prefix) atomicAdd(&sm.hist[(u32)(e >> shift) & wmask], 1u);
        }
        __syncthreads();
        if (tid < kWave) {
            // lane l owns bins 255-4l .. 252-4l (descending)
            const u32 l = tid;
            const u32 h0 = sm.hist[255 - 4 * l], h1 = sm.hist[254 - 4 * l];
            const u32 h2 = sm.hist[253 - 4 * l], h3 = sm.hist[252 - 4 * l];
            const u32 s = h0 + h1 + h2 + h3;
            const u32 incl = wave_incl_scan(s);
            const u32 excl = incl - s;
            if (excl < r && r <= incl) {
                u32 rr = r - excl, d, c;
                if (rr <= h0) {
                    d = 255 - 4 * l; c = h0;
                } else if (rr <= h0 + h1) {
                    rr -= h0; d = 254 - 4 * l; c = h1;
                } else if (rr <= h0 + h1 + h2) {
                    rr -= h0 + h1; d = 253 - 4 * l; c = h2;
                } else {
                    rr -= h0 + h1 + h2; d = 252 - 4 * l; c = h3;
                }
                sm.sel_digit = d;
                sm.sel_r = rr;
                sm.sel_c = c;
            }
            if (l == 0) sm.tmin = ~0ull;
        }
        __syncthreads();
        const u32 d = sm.sel_digit, c = sm.sel_c;
        r = sm.sel_r;
        prefix |= (u64)d << shift;
        mask |= (u64)wmask << shift;
        if (c == r) break;
        hi = shift;
    }
    // The answer is the least entry matching prefix under mask.
    u64 lm = ~0ull;
    for (u32 i = tid; i < cnt; i += WG) {
        const u64 e = sm.buf[i];
        if ((e & mask) == prefix && e < lm) lm = e;
    }
    lm = wave_min_u64(lm);
    if (lane_id() == 0 && lm != ~0ull) atomicMin((unsigned long long*)&sm.tmin, (unsigned long long)lm);
    __syncthreads();
    return sm.tmin;
}

// Reduce buf[0, cnt) to its k largest entries (cnt > k); sets L and kth.
template <class E, int WG, int CAP>
__device__ void compact_to_k(Smem<CAP>& sm, u32 cnt, u32 k, int idx_bits) {
    const u32 tid = threadIdx.x;
    const u64 T = select_rth<E, WG, CAP>(sm, cnt, k, idx_bits);
    constexpr int kItems = CAP / WG;
    u64 mine[kItems];
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const u32 i = tid + j * WG;
        mine[j] = i < cnt ? sm.buf[i] : 0ull;
    }
    if (tid == 0) sm.newcount = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const u32 i = tid + j * WG;
        wave_append(sm.buf, &sm.newcount, mine[j], i < cnt && mine[j] >= T);
    }
    __syncthreads();
    if (tid == 0) {
        sm.count = k;
        sm.kth = T;
        sm.L = T + 1;
    }
    __syncthreads();
}

// ------------------------------------------------------------------ output
template <class E, int WG, int CAP>
__device__ void emit(Smem<CAP>& sm, u32 k, int sorted, int retval, int32_t* out_idx, void* out_val) {
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
                const u64 a = sm.buf[i], b = sm.buf[j];
                if ((a > b) == up) {
                    sm.buf[i] = b;
                    sm.buf[j] = a;
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
            constexpr int kSlots = VPT * 4 * (EB == 2 ? 2 : 1);
            u64 masks[kSlots];
            u32 total = 0;
#pragma unroll
            for (int s = 0; s < kSlots; ++s) {
                const int j = s / (kSlots / VPT);
                const int w = (s % (kSlots / VPT)) / (EB == 2 ? 2 : 1);
                const int hh = EB == 2 ? (s & 1) : 0;
                const u32 d = w == 0 ? cur[j].x : w == 1 ? cur[j].y : w == 2 ? cur[j].z : cur[j].w;
                const u32 bits = EB == 2 ? ((d >> (16 * hh)) & 0xFFFFu) : d;
                const int vi = vb + j * WG + (int)tid;
                const u32 col = (u32)vi * E::kPerVec + (u32)(w * (EB == 2 ? 2 : 1) + hh);
                const bool valid = vi < v1 && col < (u32)p.n;
                saw_nan |= valid && E::is_nan(bits);
                const u64 c = compose<E>(E::key(bits), col);
                masks[s] = __ballot(valid && c >= L);
                total += (u32)__popcll(masks[s]);
            }
            if (total) {
                u32 base = 0;
                if (lane_id() == 0) base = atomicAdd(&sm.count, total);
                base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
                for (int s = 0; s < kSlots; ++s) {
                    const u64 m = masks[s];
                    if (m == 0) continue;
                    if ((m >> lane_id()) & 1ull) {
                        const int j = s / (kSlots / VPT);
                        const int w = (s % (kSlots / VPT)) / (EB == 2 ? 2 : 1);
                        const int hh = EB == 2 ? (s & 1) : 0;
                        const u32 d = w == 0 ? cur[j].x : w == 1 ? cur[j].y : w == 2 ? cur[j].z : cur[j].w;
                        const u32 bits = EB == 2 ? ((d >> (16 * hh)) & 0xFFFFu) : d;
                        const int vi = vb + j * WG + (int)tid;
                        const u32 col = (u32)vi * E::kPerVec + (u32)(w * (EB == 2 ? 2 : 1) + hh);
                        sm.buf[base + mbcnt(m)] = compose<E>(E::key(bits), col);
                    }
                    base += (u32)__popcll(m);
                }
            }
        }
        __syncthreads();
        const u32 cnt = sm.count;
        if (cnt > (u32)(CAP - kTileElems)) {
            compact_to_k<E, WG, CAP>(sm, cnt, k, p.idx_bits);
            L = sm.L;
            pf.set(L);
        }
#pragma unroll
        for (int j = 0; j < VPT; ++j) cur[j] = nxt[j];
    }

    // Final reduction of this segment to at most k entries.
    u32 cnt = sm.count;
    if (cnt > k) {
        compact_to_k<E, WG, CAP>(sm, cnt, k, p.idx_bits);
        cnt = k;
    } else if (cnt == k && p.segs > 1) {
        // k-th = least entry; a valid lower bound for the whole row
        if (tid == 0) sm.tmin = ~0ull;
        __syncthreads();
        u64 lm = ~0ull;
        for (u32 i = tid; i < cnt; i += WG) lm = sm.buf[i] < lm ? sm.buf[i] : lm;
        lm = wave_min_u64(lm);
        if (lane_id() == 0) atomicMin((unsigned long long*)&sm.tmin, (unsigned long long)lm);
        __syncthreads();
        if (tid == 0) sm.kth = sm.tmin;
        __syncthreads();
    }

    if (saw_nan) sm.nan = 1;  // benign race: every writer stores 1

    if (p.segs == 1) {
        emit<E, WG, CAP>(sm, k, p.sorted, p.retval, p.out_idx + (int64_t)row * k,
                         p.retval ? (void*)((uint8_t*)p.out_val + (int64_t)row * k * EB) : nullptr);
        __syncthreads();
        if (tid == 0 && sm.nan) *p.flag = p.flag_value;
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
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const u32 prev = atomicAdd(&p.ws_ticket[row], 1u);
        sm.last = prev == (u32)p.segs - 1;
    }
    __syncthreads();
    if (!sm.last) {
        if (tid == 0 && sm.nan) *p.flag = p.flag_value;
        return;
    }
    __threadfence();

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
#pragma unroll
        for (int j = 0; j < kMI; ++j) {
            const u32 f = base + j * WG + tid;
            bool ok = f < total;
            u64 e = 0;
            if (ok) {
                const u32 s = f / k, jj = f - s * k;
                ok = jj < sm.seg_count[s];
                if (ok) e = rc[f];
            }
            wave_append(sm.buf, &sm.count, e, ok && e >= L);
        }
        __syncthreads();
        const u32 c2 = sm.count;
        if (c2 > (u32)(CAP - kTileElems)) {
            compact_to_k<E, WG, CAP>(sm, c2, k, p.idx_bits);
            L = sm.L;
        }
    }
    cnt = sm.count;
    if (cnt > k) compact_to_k<E, WG, CAP>(sm, cnt, k, p.idx_bits);
    emit<E, WG, CAP>(sm, k, p.sorted, p.retval, p.out_idx + (int64_t)row * k,
                     p.retval ? (void*)((uint8_t*)p.out_val + (int64_t)row * k * EB) : nullptr);
    __syncthreads();
    if (tid == 0 && sm.nan) *p.flag = p.flag_value;
}

}  // namespace dstk
