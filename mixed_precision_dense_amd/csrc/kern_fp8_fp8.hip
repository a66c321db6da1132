// GEMM kernel instances for FP8 inputs: A E4M3, B E4M3 (see kern_fp8.inc).
#define MPG_FP8_KIND IN_FP8_FP8
#define MPG_FP8_LAUNCH launch_fp8_fp8
#include "kern_fp8.inc"
