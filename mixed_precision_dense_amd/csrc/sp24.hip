// sp24.hip -- the 2:4 sparse-A kernels for FP16, BF16 and INT8 inputs (sp24_kernel.inc), and
// the launcher for every input type (FP8 instances in sp24_fp8.hip).
#include "sp24_kernel.inc"

namespace mpg {

template __global__ void sp24_kernel<IN_F16, OUT_F32, false>(SpParams);
template __global__ void sp24_kernel<IN_F16, OUT_F32, true>(SpParams);
template __global__ void sp24_kernel<IN_F16, OUT_F16, false>(SpParams);
template __global__ void sp24_kernel<IN_F16, OUT_F16, true>(SpParams);
template __global__ void sp24_kernel<IN_BF16, OUT_F32, false>(SpParams);
template __global__ void sp24_kernel<IN_BF16, OUT_F32, true>(SpParams);
template __global__ void sp24_kernel<IN_BF16, OUT_BF16, false>(SpParams);
template __global__ void sp24_kernel<IN_BF16, OUT_BF16, true>(SpParams);
template __global__ void sp24_kernel<IN_I8, OUT_I32, false>(SpParams);
template __global__ void sp24_kernel<IN_I8, OUT_I32, true>(SpParams);

hipError_t launch_sp24(int in, int out, bool tb, const SpParams &sp, hipStream_t s) {
    if (in == IN_F16 && out == OUT_F32) return by_layout<IN_F16, OUT_F32>(tb, sp, s);
    if (in == IN_F16 && out == OUT_F16) return by_layout<IN_F16, OUT_F16>(tb, sp, s);
    if (in == IN_BF16 && out == OUT_F32) return by_layout<IN_BF16, OUT_F32>(tb, sp, s);
    if (in == IN_BF16 && out == OUT_BF16) return by_layout<IN_BF16, OUT_BF16>(tb, sp, s);
    if (in == IN_I8 && out == OUT_I32) return by_layout<IN_I8, OUT_I32>(tb, sp, s);
    if (is_fp8(in)) return launch_sp24_fp8(in, out, tb, sp, s);
    return hipErrorInvalidValue;
}

}  // namespace mpg
