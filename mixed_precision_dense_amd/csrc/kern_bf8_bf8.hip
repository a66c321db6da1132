// GEMM kernel instances for FP8 inputs: A E5M2, B E5M2 (see kern_fp8.inc).
#define MPG_FP8_KIND IN_BF8_BF8
#define MPG_FP8_LAUNCH launch_bf8_bf8
#include "kern_fp8.inc"
