// The bf16 selection kernel with the 8192-entry buffer, compiled apart from
// ds_topk.hip: the build lets the control-flow structurizer of this unit
// leave wave-uniform regions as plain branches, which schedules this
// instance better (bf16 4 x 204800 k = 1024 and 128 x 65536 k = 512) and the
// fp32 one worse; the two units share no out-of-line function.
#include <hip/hip_runtime.h>

#include "ds_topk.h"
#include "topk_kernels.hpp"

hipError_t ds_topk_launch_bf16(const dstk::Params& prm, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((dstk::topk_rows<2, 512, DS_TOPK_TILES_PER_CHUNK_BF16, 8192>), dim3((uint32_t)grid), dim3(512),
                       0, s, prm);
    return hipGetLastError();
}
