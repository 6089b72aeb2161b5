// The selection kernels with the 16384-entry buffer (k above 1024), compiled
// apart from ds_topk.hip: their scheduling options differ (the build adds the
// AMDGPU register-pressure trackers for this unit only; they schedule these
// instances better and the 8192-entry ones worse), and the two units share
// no out-of-line function, so each keeps its own register allocation.
#include <hip/hip_runtime.h>

#include "ds_topk.h"
#include "topk_kernels.hpp"

hipError_t ds_topk_launch_bigk(int eb, const dstk::Params& prm, int64_t grid, hipStream_t s) {
    if (eb == 4)
        hipLaunchKernelGGL((dstk::topk_rows<4, 512, DS_TOPK_TILES_PER_CHUNK_F32, 16384>), dim3((uint32_t)grid),
                           dim3(512), 0, s, prm);
    else
        hipLaunchKernelGGL((dstk::topk_rows<2, 512, DS_TOPK_TILES_PER_CHUNK_BF16_BIGK, 16384>), dim3((uint32_t)grid),
                           dim3(512), 0, s, prm);
    return hipGetLastError();
}
