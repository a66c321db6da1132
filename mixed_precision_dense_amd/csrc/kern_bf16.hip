// Instances of the GEMM kernel for bf16 inputs (one translation unit per input type so the
// instances compile in parallel).  Every kernel is instantiated explicitly: host code that
// only reaches a kernel through an inlined launcher does not reliably emit its launch stub.
#include "mpgemm_kernel.hpp"

namespace mpg {

template __global__ void gemm_kernel<IN_BF16, OUT_F32, false, false, 256, 256>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_F32, false, false, 128, 128>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_F32, false, false, 64, 64>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_F32, false, true, 256, 256>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_F32, false, true, 128, 128>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_F32, false, true, 64, 64>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_F32, true, false, 256, 256>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_F32, true, false, 128, 128>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_F32, true, false, 64, 64>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_F32, true, true, 256, 256>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_F32, true, true, 128, 128>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_F32, true, true, 64, 64>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_BF16, false, false, 256, 256>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_BF16, false, false, 128, 128>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_BF16, false, false, 64, 64>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_BF16, false, true, 256, 256>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_BF16, false, true, 128, 128>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_BF16, false, true, 64, 64>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_BF16, true, false, 256, 256>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_BF16, true, false, 128, 128>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_BF16, true, false, 64, 64>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_BF16, true, true, 256, 256>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_BF16, true, true, 128, 128>(Params);
template __global__ void gemm_kernel<IN_BF16, OUT_BF16, true, true, 64, 64>(Params);

template <int OUT, bool TA, bool TB>
static hipError_t by_tile(int tile, const Params &p, hipStream_t s) {
    switch (tile) {
    case 256: return launch<IN_BF16, OUT, TA, TB, 256, 256>(p, s);
    case 128: return launch<IN_BF16, OUT, TA, TB, 128, 128>(p, s);
    case 64: return launch<IN_BF16, OUT, TA, TB, 64, 64>(p, s);
    default: return hipErrorInvalidValue;
    }
}

template <int OUT>
static hipError_t by_layout(bool ta, bool tb, int tile, const Params &p, hipStream_t s) {
    if (!ta && !tb) return by_tile<OUT, false, false>(tile, p, s);
    if (!ta && tb) return by_tile<OUT, false, true>(tile, p, s);
    if (ta && !tb) return by_tile<OUT, true, false>(tile, p, s);
    return by_tile<OUT, true, true>(tile, p, s);
}

hipError_t launch_bf16(int out, bool ta, bool tb, int tile, const Params &p, hipStream_t s) {
    if (out == OUT_F32) return by_layout<OUT_F32>(ta, tb, tile, p, s);
    if (out == OUT_BF16) return by_layout<OUT_BF16>(ta, tb, tile, p, s);
    return hipErrorInvalidValue;
}

}  // namespace mpg
