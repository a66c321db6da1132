// mpgemm_api.hip -- host side of the C ABI declared in include/mpgemm.h: argument checks,
// handles, tile choice and kernel dispatch.  No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <mutex>
#include <new>
#include <set>
#include <string.h>

#include "mpgemm.h"
#include "mpgemm_kernel.hpp"

struct mpgemm_handle_s {
    int device;
    int num_cus;
};

namespace {

std::mutex g_handles_mu;
std::set<mpgemm_handle_t> g_handles;  // live handles; lets destroyed ones be recognised

bool handle_live(mpgemm_handle_t h) {
    std::lock_guard<std::mutex> lock(g_handles_mu);
    return g_handles.count(h) != 0;
}

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

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Largest leading dimension (elements of `eb` bytes) whose 256 rows span at most the
// 2^31 - 4096 bytes that the kernels' 32-bit buffer offsets reach.  Strides are compared with
// this bound rather than multiplied out, so that no stride a caller passes can overflow.
int64_t max_ld(int eb) { return (((int64_t)1 << 31) - 4096) / (256 * (int64_t)eb); }

// Kernel output kind for a supported type combination, or -1.
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

bool is_fp8_type(mpgemm_dtype_t t) { return t == MPGEMM_R_8F_E4M3 || t == MPGEMM_R_8F_E5M2; }

// Kernel input kind of an FP8 pair (A format, B format).
int fp8_kind(mpgemm_dtype_t a, mpgemm_dtype_t b) {
    const bool a5 = a == MPGEMM_R_8F_E5M2, b5 = b == MPGEMM_R_8F_E5M2;
    return a5 ? (b5 ? mpg::IN_BF8_BF8 : mpg::IN_BF8_FP8) : (b5 ? mpg::IN_FP8_BF8 : mpg::IN_FP8_FP8);
}

// Output kind for any supported combination, or -1.
int kernel_out_kind(mpgemm_dtype_t a, mpgemm_dtype_t b, mpgemm_dtype_t c, mpgemm_dtype_t compute) {
    if (is_fp8_type(a) && is_fp8_type(b)) {
        if (compute != MPGEMM_R_32F) return -1;
        if (c == MPGEMM_R_32F) return mpg::OUT_F32;
        if (c == MPGEMM_R_16BF) return mpg::OUT_BF16;
        return -1;
    }
    return out_kind(a, b, c, compute);
}

bool valid_dtype(int t) { return t >= MPGEMM_R_16F && t <= MPGEMM_R_8F_E5M2; }

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
    if (compute == MPGEMM_R_32I) return *(const int32_t *)beta == 0;
    float b;
    memcpy(&b, beta, sizeof b);
    return b == 0.0f;  // -0 counts as zero; NaN does not
}

// Workspace layout of mpgemm_run_bf16x3 (see include/mpgemm.h).
struct Bf16x3Layout {
    int64_t k3;            // 3 * (k rounded up to 8)
    int64_t lda3, ldb3;    // leading dimensions (elements) of the BF16 operands
    uint64_t off_b;        // byte offset of B3 in the workspace
    uint64_t total;        // workspace bytes (0 when nothing is split)
};

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

}  // namespace

namespace mpg {
hipError_t launch_fp8(int in, int out, bool ta, bool tb, int tile, const Params &p, hipStream_t s) {
    switch (in) {
    case IN_FP8_FP8: return launch_fp8_fp8(out, ta, tb, tile, p, s);
    case IN_FP8_BF8: return launch_fp8_bf8(out, ta, tb, tile, p, s);
    case IN_BF8_FP8: return launch_bf8_fp8(out, ta, tb, tile, p, s);
    case IN_BF8_BF8: return launch_bf8_bf8(out, ta, tb, tile, p, s);
    default: return hipErrorInvalidValue;
    }
}
}  // namespace mpg

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

mpgemm_status_t mpgemm_run_bf16x3(mpgemm_handle_t handle, mpgemm_op_t transa,
                                  mpgemm_op_t transb, int64_t m, int64_t n, int64_t k,
                                  const float *alpha, const float *A, int64_t lda,
                                  const float *B, int64_t ldb, const float *beta,
                                  const float *C, int64_t ldc, float *D, void *workspace,
                                  uint64_t workspace_bytes, void *stream) {
    if (!handle || !handle_live(handle)) return MPGEMM_STATUS_NOT_INITIALIZED;
    if ((transa != MPGEMM_OP_N && transa != MPGEMM_OP_T) ||
        (transb != MPGEMM_OP_N && transb != MPGEMM_OP_T))
        return MPGEMM_STATUS_INVALID_VALUE;
    if (m < 0 || n < 0 || k < 0 || !alpha || !beta) return MPGEMM_STATUS_INVALID_VALUE;
    const bool ta = transa == MPGEMM_OP_T, tb = transb == MPGEMM_OP_T;
    const int64_t min_lda = ta ? m : k, min_ldb = tb ? k : n;
    if (lda < (min_lda > 1 ? min_lda : 1) || ldb < (min_ldb > 1 ? min_ldb : 1) ||
        ldc < (n > 1 ? n : 1))
        return MPGEMM_STATUS_INVALID_VALUE;
    if (m == 0 || n == 0) return MPGEMM_STATUS_SUCCESS;
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
    char *ws = (char *)workspace;
    const void *A3 = ws, *B3 = ws ? ws + L.off_b : nullptr;
    // the GEMM on the pieces must itself be within mpgemm_run's contract (strides, sizes)
    const mpgemm_status_t st =
        mpgemm_check(transa, transb, m, n, L.k3, alpha, A3, MPGEMM_R_16BF, L.lda3, B3,
                     MPGEMM_R_16BF, L.ldb3, beta, C, MPGEMM_R_32F, ldc, D, MPGEMM_R_32F);
    if (st != MPGEMM_STATUS_SUCCESS) return st;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MPGEMM_STATUS_INTERNAL_ERROR;
    if (dev != handle->device) return MPGEMM_STATUS_WRONG_DEVICE;
    hipStream_t s = (hipStream_t)stream;
    if (k > 0) {
        // A: pieces (hi, lo, hi); B: pieces (hi, hi, lo)
        hipError_t e = ta ? mpg::launch_split_bf16x3(A, k, m, lda, ws, L.lda3, false, 0b010, s)
                          : mpg::launch_split_bf16x3(A, m, k, lda, ws, L.lda3, true, 0b010, s);
        if (e != hipSuccess) return MPGEMM_STATUS_LAUNCH_FAILED;
        e = tb ? mpg::launch_split_bf16x3(B, n, k, ldb, ws + L.off_b, L.ldb3, true, 0b100, s)
               : mpg::launch_split_bf16x3(B, k, n, ldb, ws + L.off_b, L.ldb3, false, 0b100, s);
        if (e != hipSuccess) return MPGEMM_STATUS_LAUNCH_FAILED;
    }
    return mpgemm_run(handle, transa, transb, m, n, L.k3, alpha, A3, MPGEMM_R_16BF, L.lda3, B3,
                      MPGEMM_R_16BF, L.ldb3, beta, C, MPGEMM_R_32F, ldc, D, MPGEMM_R_32F,
                      stream);
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
    // sizes the kernel indexes with 32-bit integers
    if (m > INT32_MAX || n > INT32_MAX || k > INT32_MAX) return MPGEMM_STATUS_NOT_SUPPORTED;
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

mpgemm_status_t mpgemm_create(mpgemm_handle_t *handle) {
    if (!handle) return MPGEMM_STATUS_INVALID_VALUE;
    *handle = nullptr;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return MPGEMM_STATUS_NO_DEVICE;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MPGEMM_STATUS_NO_DEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MPGEMM_STATUS_NO_DEVICE;
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MPGEMM_STATUS_NO_DEVICE;
    mpgemm_handle_t h = new (std::nothrow) mpgemm_handle_s;
    if (!h) return MPGEMM_STATUS_ALLOC_FAILED;
    h->device = dev;
    h->num_cus = prop.multiProcessorCount;
    {
        std::lock_guard<std::mutex> lock(g_handles_mu);
        g_handles.insert(h);
    }
    *handle = h;
    return MPGEMM_STATUS_SUCCESS;
}

mpgemm_status_t mpgemm_destroy(mpgemm_handle_t handle) {
    {
        std::lock_guard<std::mutex> lock(g_handles_mu);
        if (!handle || g_handles.erase(handle) == 0) return MPGEMM_STATUS_NOT_INITIALIZED;
    }
    delete handle;
    return MPGEMM_STATUS_SUCCESS;
}

mpgemm_status_t mpgemm_run(mpgemm_handle_t handle, mpgemm_op_t transa, mpgemm_op_t transb,
                           int64_t m, int64_t n, int64_t k, const void *alpha,
                           const void *A, mpgemm_dtype_t a_type, int64_t lda,
                           const void *B, mpgemm_dtype_t b_type, int64_t ldb,
                           const void *beta, const void *C, mpgemm_dtype_t c_type, int64_t ldc,
                           void *D, mpgemm_dtype_t compute_type, void *stream) {
    if (!handle || !handle_live(handle)) return MPGEMM_STATUS_NOT_INITIALIZED;
    const mpgemm_status_t st = mpgemm_check(transa, transb, m, n, k, alpha, A, a_type, lda, B,
                                            b_type, ldb, beta, C, c_type, ldc, D, compute_type);
    if (st != MPGEMM_STATUS_SUCCESS) return st;
    if (m == 0 || n == 0) return MPGEMM_STATUS_SUCCESS;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MPGEMM_STATUS_INTERNAL_ERROR;
    if (dev != handle->device) return MPGEMM_STATUS_WRONG_DEVICE;

    mpg::Params p;
    p.A = A;
    p.B = B;
    p.D = D;
    p.lda = lda;
    p.ldb = ldb;
    p.ldc = ldc;
    p.m = (int)m;
    p.n = (int)n;
    p.k = (int)k;
    p.read_c = beta_is_zero(beta, compute_type) ? 0 : 1;
    p.C = p.read_c ? C : nullptr;
    p.alpha_f = p.beta_f = 0.0f;
    p.alpha_i = p.beta_i = 0;
    if (compute_type == MPGEMM_R_32I) {
        p.alpha_i = *(const int32_t *)alpha;
        p.beta_i = *(const int32_t *)beta;
    } else {
        memcpy(&p.alpha_f, alpha, sizeof(float));
        memcpy(&p.beta_f, beta, sizeof(float));
    }
    const int tile = pick_tile(m, n, elem_bytes(a_type) == 1, handle->num_cus);
    p.tiles_m = (int)((m + tile - 1) / tile);
    p.tiles_n = (int)((n + tile - 1) / tile);
    const int out = kernel_out_kind(a_type, b_type, c_type, compute_type);
    const bool ta = transa == MPGEMM_OP_T, tb = transb == MPGEMM_OP_T;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    switch (a_type) {
    case MPGEMM_R_16F: e = mpg::launch_f16(out, ta, tb, tile, p, s); break;
    case MPGEMM_R_16BF: e = mpg::launch_bf16(out, ta, tb, tile, p, s); break;
    case MPGEMM_R_8I: e = mpg::launch_i8(out, ta, tb, tile, p, s); break;
    case MPGEMM_R_8F_E4M3:
    case MPGEMM_R_8F_E5M2: e = mpg::launch_fp8(fp8_kind(a_type, b_type), out, ta, tb, tile, p, s); break;
    default: return MPGEMM_STATUS_INTERNAL_ERROR;
    }
    return e == hipSuccess ? MPGEMM_STATUS_SUCCESS : MPGEMM_STATUS_LAUNCH_FAILED;
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

mpgemm_status_t mpgemm_run_sp24(mpgemm_handle_t handle, mpgemm_op_t transb, int64_t m, int64_t n,
                                int64_t k, const void *alpha, const void *Ac,
                                mpgemm_dtype_t a_type, int64_t lda, const void *meta,
                                int64_t ld_meta, const void *B, mpgemm_dtype_t b_type,
                                int64_t ldb, const void *beta, const void *C,
                                mpgemm_dtype_t c_type, int64_t ldc, void *D,
                                mpgemm_dtype_t compute_type, void *stream) {
    if (!handle || !handle_live(handle)) return MPGEMM_STATUS_NOT_INITIALIZED;
    const mpgemm_status_t st =
        mpgemm_check_sp24(transb, m, n, k, alpha, Ac, a_type, lda, meta, ld_meta, B, b_type, ldb,
                          beta, C, c_type, ldc, D, compute_type);
    if (st != MPGEMM_STATUS_SUCCESS) return st;
    if (m == 0 || n == 0) return MPGEMM_STATUS_SUCCESS;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MPGEMM_STATUS_INTERNAL_ERROR;
    if (dev != handle->device) return MPGEMM_STATUS_WRONG_DEVICE;
    mpg::SpParams sp;
    mpg::Params &p = sp.p;
    p.A = Ac;
    p.B = B;
    p.D = D;
    p.lda = lda;
    p.ldb = ldb;
    p.ldc = ldc;
    p.m = (int)m;
    p.n = (int)n;
    p.k = (int)k;
    p.read_c = beta_is_zero(beta, compute_type) ? 0 : 1;
    p.C = p.read_c ? C : nullptr;
    p.alpha_f = p.beta_f = 0.0f;
    p.alpha_i = p.beta_i = 0;
    if (compute_type == MPGEMM_R_32I) {
        memcpy(&p.alpha_i, alpha, sizeof(int32_t));
        memcpy(&p.beta_i, beta, sizeof(int32_t));
    } else {
        memcpy(&p.alpha_f, alpha, sizeof(float));
        memcpy(&p.beta_f, beta, sizeof(float));
    }
    p.tiles_m = (int)((m + mpg::kSpTileM - 1) / mpg::kSpTileM);
    p.tiles_n = (int)((n + mpg::kSpTileN - 1) / mpg::kSpTileN);
    sp.meta = meta;
    sp.ld_meta = ld_meta;
    const int in = is_fp8_type(a_type) ? fp8_kind(a_type, b_type)
                   : a_type == MPGEMM_R_8I ? mpg::IN_I8
                   : (a_type == MPGEMM_R_16F ? mpg::IN_F16 : mpg::IN_BF16);
    const int out = c_type == MPGEMM_R_32I ? mpg::OUT_I32
                    : c_type == MPGEMM_R_32F ? mpg::OUT_F32
                    : (c_type == MPGEMM_R_16F ? mpg::OUT_F16 : mpg::OUT_BF16);
    const hipError_t e = mpg::launch_sp24(in, out, transb == MPGEMM_OP_T, sp, (hipStream_t)stream);
    return e == hipSuccess ? MPGEMM_STATUS_SUCCESS : MPGEMM_STATUS_LAUNCH_FAILED;
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
