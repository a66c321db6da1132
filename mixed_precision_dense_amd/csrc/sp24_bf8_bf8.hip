// 2:4 sparse-A kernel instances for FP8 inputs: A E5M2, B E5M2 (see sp24_fp8.inc).
#define MPG_SP_KIND IN_BF8_BF8
#define MPG_SP_LAUNCH launch_sp24_bf8_bf8
#include "sp24_fp8.inc"
