// sp24.hip -- the launcher of the 2:4 sparse-A kernels for every input type; the instances
// are in sp24_<type>.hip (one input type per translation unit).
#include "mpgemm_kernel.hpp"

namespace mpg {

hipError_t launch_sp24(int in, int out, bool tb, const SpParams &sp, hipStream_t s) {
    switch (in) {
    case IN_F16: return launch_sp24_f16(out, tb, sp, s);
    case IN_BF16: return launch_sp24_bf16(out, tb, sp, s);
    case IN_I8: return launch_sp24_i8(out, tb, sp, s);
    case IN_FP8_FP8: return launch_sp24_fp8_fp8(out, tb, sp, s);
    case IN_FP8_BF8: return launch_sp24_fp8_bf8(out, tb, sp, s);
    case IN_BF8_FP8: return launch_sp24_bf8_fp8(out, tb, sp, s);
    case IN_BF8_BF8: return launch_sp24_bf8_bf8(out, tb, sp, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace mpg
