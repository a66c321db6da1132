// 2:4 sparse-A kernel instances for BF16 inputs (sp24_kernel.inc), FP32 or BF16 output,
// either layout of B.  One input type per translation unit: the compile time of a unit grows
// faster than its number of sparse kernels.
#include "sp24_kernel.inc"

namespace mpg {

template __global__ void sp24_kernel<IN_BF16, OUT_F32, false>(SpParams);
template __global__ void sp24_kernel<IN_BF16, OUT_F32, true>(SpParams);
template __global__ void sp24_kernel<IN_BF16, OUT_BF16, false>(SpParams);
template __global__ void sp24_kernel<IN_BF16, OUT_BF16, true>(SpParams);

hipError_t launch_sp24_bf16(int out, bool tb, const SpParams &sp, hipStream_t s) {
    if (out == OUT_F32) return by_layout<IN_BF16, OUT_F32>(tb, sp, s);
    if (out == OUT_BF16) return by_layout<IN_BF16, OUT_BF16>(tb, sp, s);
    return hipErrorInvalidValue;
}

}  // namespace mpg
