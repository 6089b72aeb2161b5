// One token per row from its top-k candidates: the step after the selection
// on the sampler path.  The pages name temperature and top-p as generation
// parameters (CSDN page, section 二 接入层; zh-TW page, the deepseek-recipe
// section) without a formula; this is the textbook one.  With c_1 .. c_k a
// row's top-k in value order, x_j their values:
//   w_j = exp((x_j - x_1) / T)  (1 where x_j == x_1, 0 for a -inf below it),
//   W_j = w_1 + ... + w_j,
//   m   = the smallest j with W_j >= top_p W_k (the nucleus; m = k if none),
//   the token is c_j for the smallest j <= m with W_j > u W_m (inverse CDF
//   at the caller's uniform u, clamped to [0, 1)).  T <= 0: greedy, c_1.
// fp32 throughout; the weights, prefix sums and both searches take one
// workgroup per row.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dssample {

typedef uint32_t u32;
constexpr int kWG = 256;     // threads per row
constexpr int kMaxPer = 16;  // candidates per thread: k <= 4096

__device__ __forceinline__ float to_float(const uint16_t* v, u32 j) { return __uint_as_float((u32)v[j] << 16); }
__device__ __forceinline__ float to_float(const float* v, u32 j) { return v[j]; }

// vals/idx: [batch][k], each row's top-k in value order (largest first).
template <class VT>
__global__ __launch_bounds__(kWG) void sample_rows(const VT* __restrict__ vals, const int32_t* __restrict__ idx,
                                                   int k, const float* __restrict__ temperature,
                                                   const float* __restrict__ top_p,
                                                   const float* __restrict__ uniform, int32_t* __restrict__ out) {
    __shared__ float wsum[kWG / 64];
    __shared__ float w_at_m;
    __shared__ u32 m_s, pick_s;
    const u32 row = blockIdx.x, tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    const VT* v = vals + (uint64_t)row * (u32)k;
    const int32_t* c = idx + (uint64_t)row * (u32)k;
    const float T = temperature[row];
    if (!(T > 0.0f)) {  // greedy (also for NaN)
        if (tid == 0) out[row] = c[0];
        return;
    }
    const float invT = 1.0f / T;
    const float x1 = to_float(v, 0);
    const u32 per = ((u32)k + kWG - 1) / kWG;
    const u32 j0 = tid * per;
    // this thread's candidates j0 .. j0 + per - 1: weights and inclusive sums
    float W[kMaxPer];
    float run = 0.0f;
#pragma unroll
    for (u32 i = 0; i < (u32)kMaxPer; ++i) {
        float w = 0.0f;
        if (i < per && j0 + i < (u32)k) {
            const float x = to_float(v, j0 + i);
            w = x == x1 ? 1.0f : (x == -__builtin_huge_valf() ? 0.0f : expf((x - x1) * invT));
        }
        run += w;
        W[i] = run;
    }
    // block exclusive scan of the thread sums (wave scan, then wave totals)
    float incl = run;
#pragma unroll
    for (u32 d = 1; d < 64; d <<= 1) {
        const float o = __shfl_up(incl, d, 64);
        if (lane >= d) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
    if (tid == 0) {
        m_s = (u32)k - 1u;
        pick_s = ~0u;
    }
    __syncthreads();
    float base = incl - run, total = 0.0f;
#pragma unroll
    for (u32 q = 0; q < (u32)(kWG / 64); ++q) {
        base += q < wave ? wsum[q] : 0.0f;
        total += wsum[q];
    }
    // nucleus: the first j with W_j >= top_p W_k
    const float thresh = top_p[row] * total;
#pragma unroll
    for (u32 i = 0; i < (u32)kMaxPer; ++i)
        if (i < per && j0 + i < (u32)k && base + W[i] >= thresh) {
            atomicMin(&m_s, j0 + i);
            break;
        }
    __syncthreads();
    const u32 m = m_s;
    if (m >= j0 && m < j0 + per) w_at_m = base + W[m - j0];
    __syncthreads();
    float u = uniform[row];
    if (!(u >= 0.0f)) u = 0.0f;
    if (u >= 1.0f) u = 0x1.fffffep-1f;  // the largest float below 1
    const float t = u * w_at_m;
#pragma unroll
    for (u32 i = 0; i < (u32)kMaxPer; ++i)
        if (i < per && j0 + i <= m && base + W[i] > t) {
            atomicMin(&pick_s, j0 + i);
            break;
        }
    __syncthreads();
    if (tid == 0) out[row] = c[pick_s <= m ? pick_s : m];
}

}  // namespace dssample
