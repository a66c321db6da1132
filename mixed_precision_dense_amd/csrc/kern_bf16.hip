// Instances of the GEMM kernel for bf16 inputs (one translation unit per input type so the
// instances compile in parallel).
#include "mpgemm_kernel.hpp"

namespace mpg {

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
