// The selection kernel with the sampling step after each row's value-ordered
// output (dstk::topk_sample_rows), for ds_topk_sample with k <= 1024 on the
// workgroup-per-row plans.  Compiled apart from ds_topk.hip so that the
// selection kernels there share no out-of-line function with these
// instances: shared callees change their register allocation.
#include <hip/hip_runtime.h>

#include "ds_topk.h"
#include "topk_kernels.hpp"

hipError_t ds_topk_launch_sample_fused(int eb, const dstk::Params& prm, int64_t grid, hipStream_t s) {
    if (eb == 4)
        hipLaunchKernelGGL((dstk::topk_sample_rows<4, 512, DS_TOPK_TILES_PER_CHUNK_F32, 8192>), dim3((uint32_t)grid),
                           dim3(512), 0, s, prm);
    else
        hipLaunchKernelGGL((dstk::topk_sample_rows<2, 512, DS_TOPK_TILES_PER_CHUNK_BF16, 8192>), dim3((uint32_t)grid),
                           dim3(512), 0, s, prm);
    return hipGetLastError();
}
