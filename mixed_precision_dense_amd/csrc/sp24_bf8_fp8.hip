// 2:4 sparse-A kernel instances for FP8 inputs: A E5M2, B E4M3 (see sp24_fp8.inc).
#define MPG_SP_KIND IN_BF8_FP8
#define MPG_SP_LAUNCH launch_sp24_bf8_fp8
#include "sp24_fp8.inc"
