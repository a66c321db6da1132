// mpgemm_host.hpp -- the host-side part of the C ABI that touches no device: argument checks,
// the tile rule and the three-product GEMM's workspace layout (mpgemm_host.cpp).  Plain
// C++17 with no HIP dependency, so it also builds as ordinary host code (for instance with
// the address and undefined-behaviour sanitizers).
#pragma once

#include <stdint.h>

#include "mpgemm.h"

namespace mpg_host {

int elem_bytes(mpgemm_dtype_t t);
bool is_fp8_type(mpgemm_dtype_t t);
// Kernel input kind of an FP8 pair (A format, B format).
int fp8_kind(mpgemm_dtype_t a, mpgemm_dtype_t b);
// Kernel output kind for any supported combination, or -1.
int kernel_out_kind(mpgemm_dtype_t a, mpgemm_dtype_t b, mpgemm_dtype_t c, mpgemm_dtype_t compute);
// Tile edge (256, 128 or 64) for an m x n output on a device with num_cus compute units.
int pick_tile(int64_t m, int64_t n, bool one_byte, int num_cus);
// *beta == 0 in the compute type (-0 counts as zero, NaN does not).
bool beta_is_zero(const void *beta, mpgemm_dtype_t compute);

// Workspace layout of mpgemm_run_bf16x3 (see include/mpgemm.h).
struct Bf16x3Layout {
    int64_t k3;            // 3 * (k rounded up to 8)
    int64_t lda3, ldb3;    // leading dimensions (elements) of the BF16 operands
    uint64_t off_b;        // byte offset of B3 in the workspace
    uint64_t total;        // workspace bytes (0 when nothing is split)
};
bool bf16x3_layout(bool ta, bool tb, int64_t m, int64_t n, int64_t k, Bf16x3Layout &L);

}  // namespace mpg_host
