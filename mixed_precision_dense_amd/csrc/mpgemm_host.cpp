// mpgemm_host.cpp -- host-only part of the C ABI declared in include/mpgemm.h: argument
// checks (mpgemm_check, mpgemm_check_sp24), the tile rule, the three-product GEMM's workspace
// layout, status strings.  No device call and no HIP header: the same source is linked into
// the HIP library and builds with a plain C++ compiler.
#include "mpgemm_host.hpp"

#include <string.h>

#include "mpgemm_kinds.hpp"

namespace mpg_host {
namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Largest k of mpgemm_run: the kernel's stage count (k + stage - 1) / stage is formed in
// 32-bit arithmetic, so k + 255 must not overflow.
constexpr int64_t kMaxK = (int64_t)INT32_MAX - 255;

// Largest leading dimension (elements of `eb` bytes) whose 256 rows span at most the
// 2^31 - 4096 bytes that the kernels' 32-bit buffer offsets reach.  Strides are compared with
// this bound rather than multiplied out, so that no stride a caller passes can overflow.
int64_t max_ld(int eb) { return (((int64_t)1 << 31) - 4096) / (256 * (int64_t)eb); }

// Kernel output kind for a supported FP16/BF16/INT8 combination, or -1.
int out_kind(mpgemm_dtype_t a, mpgemm_dtype_t b, mpgemm_dtype_t c, mpgemm_dtype_t compute) {
    if (a != b) return -1;
    if (a == MPGEMM_R_16F && compute == MPGEMM_R_32F) {
        if (c == MPGEMM_R_32F) return mpg::OUT_F32;
        if (c == MPGEMM_R_16F) return mpg::OUT_F16;
    }
    if (a == MPGEMM_R_16BF && compute == MPGEMM_R_32F) {
        if (c == MPGEMM_R_32F) return mpg::OUT_F32;
        if (c == MPGEMM_R_16BF) return mpg::OUT_BF16;
    }
    if (a == MPGEMM_R_8I && compute == MPGEMM_R_32I && c == MPGEMM_R_32I) return mpg::OUT_I32;
    return -1;
}

bool valid_dtype(int t) { return t >= MPGEMM_R_16F && t <= MPGEMM_R_8F_E5M2; }

}  // namespace

int elem_bytes(mpgemm_dtype_t t) {
    switch (t) {
    case MPGEMM_R_16F:
    case MPGEMM_R_16BF: return 2;
    case MPGEMM_R_8I:
    case MPGEMM_R_8F_E4M3:
    case MPGEMM_R_8F_E5M2: return 1;
    case MPGEMM_R_32F:
    case MPGEMM_R_32I: return 4;
    }
    return 0;
}

bool is_fp8_type(mpgemm_dtype_t t) { return t == MPGEMM_R_8F_E4M3 || t == MPGEMM_R_8F_E5M2; }

int fp8_kind(mpgemm_dtype_t a, mpgemm_dtype_t b) {
    const bool a5 = a == MPGEMM_R_8F_E5M2, b5 = b == MPGEMM_R_8F_E5M2;
    return a5 ? (b5 ? mpg::IN_BF8_BF8 : mpg::IN_BF8_FP8) : (b5 ? mpg::IN_FP8_BF8 : mpg::IN_FP8_FP8);
}

int kernel_out_kind(mpgemm_dtype_t a, mpgemm_dtype_t b, mpgemm_dtype_t c, mpgemm_dtype_t compute) {
    if (is_fp8_type(a) && is_fp8_type(b)) {
        if (compute != MPGEMM_R_32F) return -1;
        if (c == MPGEMM_R_32F) return mpg::OUT_F32;
        if (c == MPGEMM_R_16BF) return mpg::OUT_BF16;
        return -1;
    }
    return out_kind(a, b, c, compute);
}

// Tile edge with the least estimated time: the rounds of one workgroup per CU (the kernel
// runs one per CU) times the cost of a round, a tile's area over its speed per output
// element.  Measured on FP16 GEMMs that fill one round: 128 x 128 tiles produce output
// elements at about half the rate of 256 x 256 ones and 64 x 64 tiles at about a quarter
// (a fixed prologue and epilogue per tile, more loads per flop).  Ties go to the larger
// tile.  INT8 and FP8 tiles are at least 128 wide (a transposed 1-byte operand is staged in
// 128-column groups).
int pick_tile(int64_t m, int64_t n, bool one_byte, int num_cus) {
    struct Option { int edge; double round_cost; };
    static const Option kOptions[] = {{256, 1.0}, {128, 0.25 / 0.5}, {64, 0.0625 / 0.24}};
    const int64_t cus = num_cus > 0 ? num_cus : 256;
    int best = 256;
    double best_cost = 0.0;
    for (const Option &o : kOptions) {
        if (one_byte && o.edge < 128) continue;
        const int64_t tiles = ((m + o.edge - 1) / o.edge) * ((n + o.edge - 1) / o.edge);
        const double cost = (double)((tiles + cus - 1) / cus) * o.round_cost;
        if (o.edge == 256 || cost < best_cost) {
            best = o.edge;
            best_cost = cost;
        }
    }
    return best;
}

bool beta_is_zero(const void *beta, mpgemm_dtype_t compute) {
    if (compute == MPGEMM_R_32I) {
        int32_t b;
        memcpy(&b, beta, sizeof b);
        return b == 0;
    }
    float b;
    memcpy(&b, beta, sizeof b);
    return b == 0.0f;  // -0 counts as zero; NaN does not
}

bool bf16x3_layout(bool ta, bool tb, int64_t m, int64_t n, int64_t k, Bf16x3Layout &L) {
    if (m < 0 || n < 0 || k < 0) return false;
    const int64_t lim = (int64_t)1 << 40;  // keeps every product below 2^63
    if (m > lim || n > lim || k > lim) return false;
    L.k3 = 3 * ((k + 7) / 8 * 8);
    const int64_t m8 = (m + 7) / 8 * 8, n8 = (n + 7) / 8 * 8;
    // (at least 8: with k == 0 nothing is split, but the BF16 call still checks its strides)
    L.lda3 = ta ? m8 : (L.k3 > 8 ? L.k3 : 8);
    L.ldb3 = tb ? (L.k3 > 8 ? L.k3 : 8) : n8;
    if (m == 0 || n == 0 || k == 0) {
        L.off_b = L.total = 0;
        return true;
    }
    const unsigned __int128 bytes_a = (unsigned __int128)(ta ? L.k3 : m) * (uint64_t)L.lda3 * 2;
    const unsigned __int128 bytes_b = (unsigned __int128)(tb ? n : L.k3) * (uint64_t)L.ldb3 * 2;
    const unsigned __int128 off_b = (bytes_a + 255) / 256 * 256;
    const unsigned __int128 total = off_b + bytes_b;
    if (total > (unsigned __int128)UINT64_MAX) return false;
    L.off_b = (uint64_t)off_b;
    L.total = (uint64_t)total;
    return true;
}

}  // namespace mpg_host

using namespace mpg_host;

extern "C" {

uint64_t mpgemm_bf16x3_workspace_size(mpgemm_op_t transa, mpgemm_op_t transb, int64_t m,
                                      int64_t n, int64_t k) {
    if ((transa != MPGEMM_OP_N && transa != MPGEMM_OP_T) ||
        (transb != MPGEMM_OP_N && transb != MPGEMM_OP_T))
        return 0;
    Bf16x3Layout L;
    if (!bf16x3_layout(transa == MPGEMM_OP_T, transb == MPGEMM_OP_T, m, n, k, L)) return 0;
    return L.total;
}

mpgemm_status_t mpgemm_check_bf16x3(mpgemm_op_t transa, mpgemm_op_t transb, int64_t m,
                                    int64_t n, int64_t k, const float *alpha, const float *A,
                                    int64_t lda, const float *B, int64_t ldb, const float *beta,
                                    const float *C, int64_t ldc, const float *D,
                                    const void *workspace, uint64_t workspace_bytes) {
    if ((transa != MPGEMM_OP_N && transa != MPGEMM_OP_T) ||
        (transb != MPGEMM_OP_N && transb != MPGEMM_OP_T))
        return MPGEMM_STATUS_INVALID_VALUE;
    if (m < 0 || n < 0 || k < 0 || !alpha || !beta) return MPGEMM_STATUS_INVALID_VALUE;
    const bool ta = transa == MPGEMM_OP_T, tb = transb == MPGEMM_OP_T;
    const int64_t min_lda = ta ? m : k, min_ldb = tb ? k : n;
    if (lda < (min_lda > 1 ? min_lda : 1) || ldb < (min_ldb > 1 ? min_ldb : 1) ||
        ldc < (n > 1 ? n : 1))
        return MPGEMM_STATUS_INVALID_VALUE;
    if (m == 0 || n == 0) return MPGEMM_STATUS_SUCCESS;  // nothing to do, nothing is read
    const bool read_c = !beta_is_zero(beta, MPGEMM_R_32F);
    if (!D || (k > 0 && (!A || !B)) || (read_c && !C)) return MPGEMM_STATUS_INVALID_VALUE;
    if (m > INT32_MAX || n > INT32_MAX || k > INT32_MAX / 3 - 8) return MPGEMM_STATUS_NOT_SUPPORTED;
    if (!aligned16(D) || (read_c && !aligned16(C))) return MPGEMM_STATUS_NOT_SUPPORTED;
    if (k > 0 && (!aligned16(A) || !aligned16(B))) return MPGEMM_STATUS_NOT_SUPPORTED;
    if (lda % 4 || ldb % 4 || ldc % 4) return MPGEMM_STATUS_NOT_SUPPORTED;
    Bf16x3Layout L;
    if (!bf16x3_layout(ta, tb, m, n, k, L)) return MPGEMM_STATUS_NOT_SUPPORTED;
    if (L.total > 0) {
        if (!workspace || workspace_bytes < L.total) return MPGEMM_STATUS_INVALID_VALUE;
        if ((uintptr_t)workspace & 255u) return MPGEMM_STATUS_NOT_SUPPORTED;
    }
    // the GEMM on the pieces must itself be within mpgemm_run's contract (strides, sizes)
    const char *ws = (const char *)workspace;
    const void *A3 = ws, *B3 = ws ? ws + L.off_b : nullptr;
    return mpgemm_check(transa, transb, m, n, L.k3, alpha, A3, MPGEMM_R_16BF, L.lda3, B3,
                        MPGEMM_R_16BF, L.ldb3, beta, C, MPGEMM_R_32F, ldc, D, MPGEMM_R_32F);
}

mpgemm_status_t mpgemm_check(mpgemm_op_t transa, mpgemm_op_t transb, int64_t m, int64_t n,
                             int64_t k, const void *alpha, const void *A, mpgemm_dtype_t a_type,
                             int64_t lda, const void *B, mpgemm_dtype_t b_type, int64_t ldb,
                             const void *beta, const void *C, mpgemm_dtype_t c_type, int64_t ldc,
                             const void *D, mpgemm_dtype_t compute_type) {
    if ((transa != MPGEMM_OP_N && transa != MPGEMM_OP_T) ||
        (transb != MPGEMM_OP_N && transb != MPGEMM_OP_T))
        return MPGEMM_STATUS_INVALID_VALUE;
    if (m < 0 || n < 0 || k < 0) return MPGEMM_STATUS_INVALID_VALUE;
    if (!alpha || !beta) return MPGEMM_STATUS_INVALID_VALUE;
    if (!valid_dtype(a_type) || !valid_dtype(b_type) || !valid_dtype(c_type) ||
        !valid_dtype(compute_type))
        return MPGEMM_STATUS_NOT_SUPPORTED;
    if (kernel_out_kind(a_type, b_type, c_type, compute_type) < 0) return MPGEMM_STATUS_NOT_SUPPORTED;
    const bool ta = transa == MPGEMM_OP_T, tb = transb == MPGEMM_OP_T;
    const int64_t min_lda = ta ? m : k, min_ldb = tb ? k : n, min_ldc = n;
    if (lda < (min_lda > 1 ? min_lda : 1) || ldb < (min_ldb > 1 ? min_ldb : 1) ||
        ldc < (min_ldc > 1 ? min_ldc : 1))
        return MPGEMM_STATUS_INVALID_VALUE;
    if (m == 0 || n == 0) return MPGEMM_STATUS_SUCCESS;  // nothing to do, nothing is read
    const bool read_c = !beta_is_zero(beta, compute_type);
    if (!D) return MPGEMM_STATUS_INVALID_VALUE;
    if (k > 0 && (!A || !B)) return MPGEMM_STATUS_INVALID_VALUE;
    if (read_c && !C) return MPGEMM_STATUS_INVALID_VALUE;
    // sizes the kernel indexes with 32-bit integers; k also leaves room for the kernel's
    // stage count, k rounded up to a whole 128-byte stage
    if (m > INT32_MAX || n > INT32_MAX || k > kMaxK) return MPGEMM_STATUS_NOT_SUPPORTED;
    // one workgroup of kThreads per tile (smallest tile), within a 32-bit dispatch size
    const int64_t tiles = ((m + 63) / 64) * ((n + 63) / 64);
    if (tiles > (int64_t)UINT32_MAX / mpg::kThreads) return MPGEMM_STATUS_NOT_SUPPORTED;
    // alignment contract
    const int ea = elem_bytes(a_type), ec = elem_bytes(c_type);
    if (!aligned16(D) || (read_c && !aligned16(C))) return MPGEMM_STATUS_NOT_SUPPORTED;
    if (k > 0 && (!aligned16(A) || !aligned16(B))) return MPGEMM_STATUS_NOT_SUPPORTED;
    // every buffer offset the kernel forms spans at most 256 rows of one operand
    if (lda > max_ld(ea) || ldb > max_ld(ea) || ldc > max_ld(ec)) return MPGEMM_STATUS_NOT_SUPPORTED;
    if ((lda * ea) % 16 || (ldb * ea) % 16 || (ldc * ec) % 16) return MPGEMM_STATUS_NOT_SUPPORTED;
    return MPGEMM_STATUS_SUCCESS;
}

mpgemm_status_t mpgemm_check_sp24(mpgemm_op_t transb, int64_t m, int64_t n, int64_t k,
                                  const void *alpha, const void *Ac, mpgemm_dtype_t a_type,
                                  int64_t lda, const void *meta, int64_t ld_meta, const void *B,
                                  mpgemm_dtype_t b_type, int64_t ldb, const void *beta,
                                  const void *C, mpgemm_dtype_t c_type, int64_t ldc,
                                  const void *D, mpgemm_dtype_t compute_type) {
    if (transb != MPGEMM_OP_N && transb != MPGEMM_OP_T) return MPGEMM_STATUS_INVALID_VALUE;
    if (m < 0 || n < 0 || k < 0 || !alpha || !beta) return MPGEMM_STATUS_INVALID_VALUE;
    if (!valid_dtype(a_type) || !valid_dtype(b_type) || !valid_dtype(c_type) ||
        !valid_dtype(compute_type))
        return MPGEMM_STATUS_NOT_SUPPORTED;
    if (is_fp8_type(a_type) && is_fp8_type(b_type)) {
        if (kernel_out_kind(a_type, b_type, c_type, compute_type) < 0)
            return MPGEMM_STATUS_NOT_SUPPORTED;
    } else if (a_type != b_type) {
        return MPGEMM_STATUS_NOT_SUPPORTED;
    } else if (a_type == MPGEMM_R_8I) {
        if (compute_type != MPGEMM_R_32I || c_type != MPGEMM_R_32I) return MPGEMM_STATUS_NOT_SUPPORTED;
    } else if (a_type == MPGEMM_R_16F || a_type == MPGEMM_R_16BF) {
        if (compute_type != MPGEMM_R_32F || (c_type != MPGEMM_R_32F && c_type != a_type))
            return MPGEMM_STATUS_NOT_SUPPORTED;
    } else {
        return MPGEMM_STATUS_NOT_SUPPORTED;
    }
    const int ea = elem_bytes(a_type);
    if (k % 128) return MPGEMM_STATUS_NOT_SUPPORTED;
    const bool tb = transb == MPGEMM_OP_T;
    const int64_t min_ldb = tb ? k : n;
    if (lda < (k / 2 > 1 ? k / 2 : 1) || ld_meta < (k / 8 > 1 ? k / 8 : 1) ||
        ldb < (min_ldb > 1 ? min_ldb : 1) || ldc < (n > 1 ? n : 1))
        return MPGEMM_STATUS_INVALID_VALUE;
    if (m == 0 || n == 0) return MPGEMM_STATUS_SUCCESS;
    const bool read_c = !beta_is_zero(beta, compute_type);
    if (!D || (k > 0 && (!Ac || !meta || !B)) || (read_c && !C)) return MPGEMM_STATUS_INVALID_VALUE;
    if (m > INT32_MAX || n > INT32_MAX || k > INT32_MAX) return MPGEMM_STATUS_NOT_SUPPORTED;
    const int64_t tiles = ((m + mpg::kSpTileM - 1) / mpg::kSpTileM) *
                          ((n + mpg::kSpTileN - 1) / mpg::kSpTileN);
    if (tiles > (int64_t)UINT32_MAX / mpg::kThreads) return MPGEMM_STATUS_NOT_SUPPORTED;
    const int ec = elem_bytes(c_type);
    if (!aligned16(D) || (read_c && !aligned16(C))) return MPGEMM_STATUS_NOT_SUPPORTED;
    if (k > 0 && (!aligned16(Ac) || !aligned16(meta) || !aligned16(B))) return MPGEMM_STATUS_NOT_SUPPORTED;
    if (lda > max_ld(ea) || ldb > max_ld(ea) || ld_meta > max_ld(1) || ldc > max_ld(ec))
        return MPGEMM_STATUS_NOT_SUPPORTED;
    if ((lda * ea) % 16 || (ldb * ea) % 16 || ld_meta % 16 || (ldc * ec) % 16)
        return MPGEMM_STATUS_NOT_SUPPORTED;
    return MPGEMM_STATUS_SUCCESS;
}

const char *mpgemm_status_string(mpgemm_status_t status) {
    switch (status) {
    case MPGEMM_STATUS_SUCCESS: return "success";
    case MPGEMM_STATUS_NOT_INITIALIZED: return "handle not initialized or already destroyed";
    case MPGEMM_STATUS_INVALID_VALUE: return "invalid value (null pointer, negative size or leading dimension too small)";
    case MPGEMM_STATUS_NOT_SUPPORTED: return "not supported (type combination, alignment or stride outside the contract)";
    case MPGEMM_STATUS_ALLOC_FAILED: return "host allocation failed";
    case MPGEMM_STATUS_NO_DEVICE: return "no gfx950 HIP device";
    case MPGEMM_STATUS_LAUNCH_FAILED: return "kernel launch failed";
    case MPGEMM_STATUS_INTERNAL_ERROR: return "internal error";
    case MPGEMM_STATUS_WRONG_DEVICE: return "current HIP device is not the handle's device";
    case MPGEMM_STATUS_SCRATCH_TOO_SMALL: return "the problem needs more than the library's fixed 64 MiB scratch buffer";
    }
    return "unknown status";
}

mpgemm_status_t mpgemm_tile_shape(int64_t m, int64_t n, mpgemm_dtype_t a_type, int *tile_m,
                                  int *tile_n) {
    if (m < 0 || n < 0 || !tile_m || !tile_n) return MPGEMM_STATUS_INVALID_VALUE;
    const int t = pick_tile(m, n, elem_bytes(a_type) == 1, 256);
    *tile_m = t;
    *tile_n = t;
    return MPGEMM_STATUS_SUCCESS;
}

}  // extern "C"
