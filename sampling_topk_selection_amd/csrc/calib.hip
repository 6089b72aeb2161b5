// Calibration kernels for the benchmark (not part of the top-k path):
//   calib_empty  -- an empty kernel on a given grid: the launch/dispatch floor;
//   calib_read   -- a pure 16-byte streaming read of `bytes` with a given grid:
//                   the achievable read roofline at that size and shape;
//   calib_copy   -- a plain copy of `bytes`: a kernel of known traffic, used to
//                   scale the FETCH_SIZE / WRITE_SIZE hardware counters.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(512) void k_empty() {}

__global__ __launch_bounds__(512) void k_read(const uint4* __restrict__ in, int64_t nvec, uint32_t* out) {
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
        const uint4 v = in[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // keep the loads alive; one word per workgroup
    __shared__ uint32_t s;
    if (threadIdx.x == 0) s = 0;
    __syncthreads();
    atomicXor(&s, acc);
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = s;
}

__global__ __launch_bounds__(512) void k_copy(const uint4* __restrict__ in, uint4* __restrict__ out, int64_t nvec) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) out[i] = in[i];
}

}  // namespace

extern "C" {

int calib_empty(int64_t grid, void* stream) {
    hipLaunchKernelGGL(k_empty, dim3((uint32_t)grid), dim3(512), 0, (hipStream_t)stream);
    return (int)hipGetLastError();
}

// `out` must hold `grid` uint32 words; `bytes` is a multiple of 16.
int calib_read(const void* in, int64_t bytes, int64_t grid, uint32_t* out, void* stream) {
    hipLaunchKernelGGL(k_read, dim3((uint32_t)grid), dim3(512), 0, (hipStream_t)stream, (const uint4*)in,
                       bytes / 16, out);
    return (int)hipGetLastError();
}

int calib_copy(const void* in, void* out, int64_t bytes, int64_t grid, void* stream) {
    hipLaunchKernelGGL(k_copy, dim3((uint32_t)grid), dim3(512), 0, (hipStream_t)stream, (const uint4*)in,
                       (uint4*)out, bytes / 16);
    return (int)hipGetLastError();
}

}  // extern "C"
