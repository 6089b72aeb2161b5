// Calibration kernels for the benchmark (not part of the top-k path):
//   calib_empty  -- an empty kernel on a given grid: the launch/dispatch floor;
//   calib_read   -- a pure streaming read of `bytes` on a given grid of
//                   512-thread workgroups, each reading one contiguous slice
//                   with 2 x NV 16-byte loads in flight per thread (the
//                   top-k scan's own access shape: one slice per workgroup,
//                   chunks of NV loads, double buffered), so it bounds what
//                   a scan on that grid can reach at that size;
//   calib_copy   -- a plain copy of `bytes`: a kernel of known traffic, used to
//                   scale the FETCH_SIZE / WRITE_SIZE hardware counters.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kWG = 512;
constexpr int kNV = 4;  // 16-byte loads per thread per chunk

__global__ __launch_bounds__(kWG) void k_empty() {}

__device__ __forceinline__ uint32_t fold(const uint4 (&v)[kNV]) {
    uint32_t a = 0;
#pragma unroll
    for (int i = 0; i < kNV; ++i) a ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    return a;
}

// Workgroup b reads vectors [b * per, min((b + 1) * per, nvec)).
__global__ __launch_bounds__(kWG) void k_read(const uint4* __restrict__ in, int64_t nvec, int64_t per,
                                              uint32_t* out) {
    const int64_t v0 = (int64_t)blockIdx.x * per;
    const int64_t v1 = v0 + per < nvec ? v0 + per : nvec;
    constexpr int64_t kChunk = (int64_t)kWG * kNV;
    uint4 a[kNV], b[kNV];
    auto load = [&](int64_t base, uint4 (&v)[kNV]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kNV; ++i) {
            const int64_t j = base + (int64_t)i * kWG + threadIdx.x;
            v[i] = j < v1 ? in[j] : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    uint32_t acc = 0;
    load(v0, a);
    for (int64_t base = v0; base < v1; base += 2 * kChunk) {
        load(base + kChunk, b);
        acc ^= fold(a);
        load(base + 2 * kChunk, a);
        acc ^= fold(b);
    }
    acc ^= fold(a);  // (zeros or the loads past the slice: keeps every load used)
    // one word per workgroup: a wave reduction, then one LDS atomic per wave
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
    __shared__ uint32_t s;
    if (threadIdx.x == 0) s = 0;
    __syncthreads();
    if ((threadIdx.x & 63u) == 0) atomicXor(&s, acc);
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = s;
}

__global__ __launch_bounds__(kWG) void k_copy(const uint4* __restrict__ in, uint4* __restrict__ out, int64_t nvec) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) out[i] = in[i];
}

}  // namespace

extern "C" {

// `n` empty kernels of `grid` workgroups, back to back.
int calib_empty(int64_t grid, int64_t n, void* stream) {
    for (int64_t i = 0; i < n; ++i)
        hipLaunchKernelGGL(k_empty, dim3((uint32_t)grid), dim3(kWG), 0, (hipStream_t)stream);
    return (int)hipGetLastError();
}

// `out` must hold `grid` uint32 words; `bytes` is a multiple of 16.
int calib_read(const void* in, int64_t bytes, int64_t grid, uint32_t* out, void* stream) {
    const int64_t nvec = bytes / 16;
    const int64_t per = (nvec + grid - 1) / grid;
    hipLaunchKernelGGL(k_read, dim3((uint32_t)grid), dim3(kWG), 0, (hipStream_t)stream, (const uint4*)in, nvec, per,
                       out);
    return (int)hipGetLastError();
}

int calib_copy(const void* in, void* out, int64_t bytes, int64_t grid, void* stream) {
    hipLaunchKernelGGL(k_copy, dim3((uint32_t)grid), dim3(kWG), 0, (hipStream_t)stream, (const uint4*)in,
                       (uint4*)out, bytes / 16);
    return (int)hipGetLastError();
}

}  // extern "C"
