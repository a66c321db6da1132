// bf16x3.hip -- splitting FP32 operands into the BF16 pieces of the three-product GEMM.
//
// Multiword emulation ("NVIDIA Tensor Core mixed-precision computing: principles and
// applications", section 5.1): an FP32 element x becomes x_hi = RN_bf16(x) and
// x_lo = RN_bf16(x - x_hi) (x_lo = 0 when x_hi is not finite), and the three products
// A_hi B_hi + A_lo B_hi + A_hi B_lo are one BF16 GEMM over k3 = 3 kp (kp = k rounded up to a
// multiple of 8, zero padded), the pieces concatenated along k in that order.
//
// This kernel writes one operand's pieces.  The FP32 input is row-major (rows x cols, ld
// elements).  k runs along its columns (A with transa == N, B with transb == T) or along its
// rows (A with transa == T, B with transb == N):
//   k along columns: output row r = [piece0(r, :) 0-pad | piece1 | piece2], each piece
//                    cols_pad = roundup(cols, 8) wide; ld_out = 3 cols_pad.
//   k along rows:    output rows [piece0 rows, zero rows up to rows_pad | piece1 | piece2],
//                    rows_pad = roundup(rows, 8); ld_out = roundup(cols, 8), the columns
//                    from cols up to ld_out written as zeros.
// A thread handles 8 consecutive columns of one row: two 16-byte loads, three 16-byte stores
// (one per piece).  The work is a pure HBM stream (4 bytes read, 6 written per element).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "mpgemm_kernel.hpp"

namespace mpg {

namespace {

struct Split8 {
    uint32_t hi[4], lo[4];  // 8 BF16 values each, packed in pairs (element 2i in the low half)
};

__device__ __forceinline__ uint32_t bf16_bits(__bf16 v) {
    return (uint32_t)__builtin_bit_cast(unsigned short, v);
}

// x_hi = RN_bf16(x); x_lo = RN_bf16(x - x_hi), or 0 when x_hi is not finite.
__device__ __forceinline__ void split1(float x, uint32_t &hi, uint32_t &lo) {
    const __bf16 h = (__bf16)x;                    // v_cvt_pk_bf16_f32: nearest even
    const float hf = (float)h;
    const float r = x - hf;                        // exact: the rounding error of x
    hi = bf16_bits(h);
    lo = __builtin_isfinite(hf) ? bf16_bits((__bf16)r) : 0u;
}

__device__ __forceinline__ Split8 split8(const float (&x)[8]) {
    Split8 s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t h0, l0, h1, l1;
        split1(x[2 * i], h0, l0);
        split1(x[2 * i + 1], h1, l1);
        s.hi[i] = h0 | (h1 << 16);
        s.lo[i] = l0 | (l1 << 16);
    }
    return s;
}

// Eight consecutive FP32 values of a row starting at column c (zeros past `cols`).
__device__ __forceinline__ void load8(const float *row, int64_t c, int64_t cols, float (&x)[8]) {
    if (c + 8 <= cols) {
        const float4 a = *(const float4 *)(row + c);
        const float4 b = *(const float4 *)(row + c + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (c + i < cols) ? row[c + i] : 0.0f;
    }
}

__device__ __forceinline__ void store8(__bf16 *dst, const uint32_t (&v)[4]) {
    *(uint4 *)dst = make_uint4(v[0], v[1], v[2], v[3]);
}

// pieces: bit i set means piece i is the low part (A: 0b010 = hi, lo, hi; B: 0b100 = hi, hi, lo)
__global__ void __launch_bounds__(256) split_bf16x3_kernel(
    const float *__restrict__ in, int64_t rows, int64_t cols, int64_t ld_in,
    __bf16 *__restrict__ out, int64_t ld_out, int k_along_cols, int pieces, int64_t row_groups,
    int64_t iter_rows) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= iter_rows * row_groups) return;
    const int64_t r = t / row_groups;
    const int64_t c = (t - r * row_groups) * 8;
    float x[8];
    if (r < rows)
        load8(in + r * ld_in, c, cols, x);
    else
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = 0.0f;     // zero rows of a k-along-rows piece
    const Split8 s = split8(x);
    const int64_t cols_pad = row_groups * 8;
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        const bool lo = (pieces >> p) & 1;
        __bf16 *dst = k_along_cols ? out + r * ld_out + p * cols_pad + c
                                   : out + (p * iter_rows + r) * ld_out + c;
        store8(dst, lo ? s.lo : s.hi);
    }
}

}  // namespace

hipError_t launch_split_bf16x3(const float *in, int64_t rows, int64_t cols, int64_t ld_in,
                               void *out, int64_t ld_out, bool k_along_cols, int pieces,
                               hipStream_t stream) {
    const int64_t row_groups = (cols + 7) / 8;
    const int64_t iter_rows = k_along_cols ? rows : (rows + 7) / 8 * 8;
    const int64_t threads = iter_rows * row_groups;
    if (threads == 0) return hipSuccess;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks * 256 > (int64_t)UINT32_MAX) return hipErrorInvalidValue;   // 32-bit dispatch size
    // arguments with the kernel's exact parameter types, for hipLaunchKernel (which returns
    // this launch's own status)
    const float *a_in = in;
    __bf16 *a_out = (__bf16 *)out;
    int a_kc = k_along_cols ? 1 : 0, a_pieces = pieces;
    int64_t a_rows = rows, a_cols = cols, a_ld_in = ld_in, a_ld_out = ld_out;
    int64_t a_groups = row_groups, a_iter = iter_rows;
    void *args[] = {&a_in, &a_rows, &a_cols, &a_ld_in, &a_out, &a_ld_out, &a_kc, &a_pieces,
                    &a_groups, &a_iter};
    return hipLaunchKernel(reinterpret_cast<const void *>(&split_bf16x3_kernel),
                           dim3((unsigned)blocks), dim3(256), args, 0, stream);
}

}  // namespace mpg
