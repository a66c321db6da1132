// sp24_fp8.hip -- the 2:4 sparse-A kernels for FP8 inputs (E4M3 / E5M2, either pairing),
// FP32 or BF16 output (sp24_kernel.inc).
#include "sp24_kernel.inc"

namespace mpg {

template __global__ void sp24_kernel<IN_FP8_FP8, OUT_F32, false>(SpParams);
template __global__ void sp24_kernel<IN_FP8_FP8, OUT_F32, true>(SpParams);
template __global__ void sp24_kernel<IN_FP8_FP8, OUT_BF16, false>(SpParams);
template __global__ void sp24_kernel<IN_FP8_FP8, OUT_BF16, true>(SpParams);
template __global__ void sp24_kernel<IN_FP8_BF8, OUT_F32, false>(SpParams);
template __global__ void sp24_kernel<IN_FP8_BF8, OUT_F32, true>(SpParams);
template __global__ void sp24_kernel<IN_FP8_BF8, OUT_BF16, false>(SpParams);
template __global__ void sp24_kernel<IN_FP8_BF8, OUT_BF16, true>(SpParams);
template __global__ void sp24_kernel<IN_BF8_FP8, OUT_F32, false>(SpParams);
template __global__ void sp24_kernel<IN_BF8_FP8, OUT_F32, true>(SpParams);
template __global__ void sp24_kernel<IN_BF8_FP8, OUT_BF16, false>(SpParams);
template __global__ void sp24_kernel<IN_BF8_FP8, OUT_BF16, true>(SpParams);
template __global__ void sp24_kernel<IN_BF8_BF8, OUT_F32, false>(SpParams);
template __global__ void sp24_kernel<IN_BF8_BF8, OUT_F32, true>(SpParams);
template __global__ void sp24_kernel<IN_BF8_BF8, OUT_BF16, false>(SpParams);
template __global__ void sp24_kernel<IN_BF8_BF8, OUT_BF16, true>(SpParams);

hipError_t launch_sp24_fp8(int in, int out, bool tb, const SpParams &sp, hipStream_t s) {
    if (in == IN_FP8_FP8 && out == OUT_F32) return by_layout<IN_FP8_FP8, OUT_F32>(tb, sp, s);
    if (in == IN_FP8_FP8 && out == OUT_BF16) return by_layout<IN_FP8_FP8, OUT_BF16>(tb, sp, s);
    if (in == IN_FP8_BF8 && out == OUT_F32) return by_layout<IN_FP8_BF8, OUT_F32>(tb, sp, s);
    if (in == IN_FP8_BF8 && out == OUT_BF16) return by_layout<IN_FP8_BF8, OUT_BF16>(tb, sp, s);
    if (in == IN_BF8_FP8 && out == OUT_F32) return by_layout<IN_BF8_FP8, OUT_F32>(tb, sp, s);
    if (in == IN_BF8_FP8 && out == OUT_BF16) return by_layout<IN_BF8_FP8, OUT_BF16>(tb, sp, s);
    if (in == IN_BF8_BF8 && out == OUT_F32) return by_layout<IN_BF8_BF8, OUT_F32>(tb, sp, s);
    if (in == IN_BF8_BF8 && out == OUT_BF16) return by_layout<IN_BF8_BF8, OUT_BF16>(tb, sp, s);
    return hipErrorInvalidValue;
}

}  // namespace mpg
