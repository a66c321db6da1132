// 2:4 sparse-A kernel instances for FP16 inputs (sp24_kernel.inc), FP32 or FP16 output,
// either layout of B.  One input type per translation unit: the compile time of a unit grows
// faster than its number of sparse kernels.
#include "sp24_kernel.inc"

namespace mpg {

template __global__ void sp24_kernel<IN_F16, OUT_F32, false>(SpParams);
template __global__ void sp24_kernel<IN_F16, OUT_F32, true>(SpParams);
template __global__ void sp24_kernel<IN_F16, OUT_F16, false>(SpParams);
template __global__ void sp24_kernel<IN_F16, OUT_F16, true>(SpParams);

hipError_t launch_sp24_f16(int out, bool tb, const SpParams &sp, hipStream_t s) {
    if (out == OUT_F32) return by_layout<IN_F16, OUT_F32>(tb, sp, s);
    if (out == OUT_F16) return by_layout<IN_F16, OUT_F16>(tb, sp, s);
    return hipErrorInvalidValue;
}

}  // namespace mpg
