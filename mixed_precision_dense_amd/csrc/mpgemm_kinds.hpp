// mpgemm_kinds.hpp -- names shared by the host-side argument checks and the kernels: the
// input and output kinds a kernel instance is built for, and the launch geometry the checks
// bound (plain C++, no HIP headers, so the checks also build as ordinary host code).
#pragma once

namespace mpg {

// FP8 kinds name the A and B formats (OCP E4M3 "fp8", E5M2 "bf8").
enum InKind { IN_F16 = 0, IN_BF16 = 1, IN_I8 = 2, IN_FP8_FP8 = 3, IN_FP8_BF8 = 4, IN_BF8_FP8 = 5,
              IN_BF8_BF8 = 6 };
constexpr bool is_fp8(int in) { return in >= IN_FP8_FP8 && in <= IN_BF8_BF8; }
enum OutKind { OUT_F32 = 0, OUT_F16 = 1, OUT_BF16 = 2, OUT_I32 = 3 };

constexpr int kThreads = 256;                  // lanes per workgroup (4 waves)
constexpr int kSpTileM = 256, kSpTileN = 256;  // tile of the 2:4 sparse-A kernel

}  // namespace mpg
