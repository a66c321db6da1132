// 2:4 sparse-A kernel instances for INT8 inputs (sp24_kernel.inc), INT32 output, either layout
// of B.
#include "sp24_kernel.inc"

namespace mpg {

template __global__ void sp24_kernel<IN_I8, OUT_I32, false>(SpParams);
template __global__ void sp24_kernel<IN_I8, OUT_I32, true>(SpParams);

hipError_t launch_sp24_i8(int out, bool tb, const SpParams &sp, hipStream_t s) {
    if (out == OUT_I32) return by_layout<IN_I8, OUT_I32>(tb, sp, s);
    return hipErrorInvalidValue;
}

}  // namespace mpg
