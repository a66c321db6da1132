// mpgemm_api.hip -- the device-facing part of the C ABI declared in include/mpgemm.h:
// handles and kernel dispatch (the argument checks, the tile rule and the workspace layout
// are in mpgemm_host.cpp).  No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <new>
#include <set>
#include <string.h>

#include "mpgemm.h"
#include "mpgemm_host.hpp"
#include "mpgemm_kernel.hpp"

using namespace mpg_host;

struct mpgemm_handle_s {
    int device;
    int num_cus;
    void *scratch;   // this device's address of `scratch` (below), or nullptr
};

// Fixed scratch buffer of mpgemm_run_bf16x3_noalloc, for callers that cannot allocate: it
// holds the BF16 pieces of the split operands, laid out as mpgemm_run_bf16x3's workspace.
// Static device memory: every device the library runs on has its own copy, at its own
// address, until the process ends; all calls on one device share it.  In host code the name
// is only a stand-in for the symbol: kernels and copies use the address that
// hipGetSymbolAddress returns for the current device (scratch_address).
static __device__ __align__(256) unsigned char scratch[MPGEMM_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_handles_mu;
std::set<mpgemm_handle_t> g_handles;  // live handles; lets destroyed ones be recognised

bool handle_live(mpgemm_handle_t h) {
    std::lock_guard<std::mutex> lock(g_handles_mu);
    return g_handles.count(h) != 0;
}

std::mutex g_scratch_mu;
std::map<int, void *> g_scratch_addr;   // device -> address of `scratch` on that device

// Address of `scratch` on device `dev`, which must be the current device: looked up once per
// device (hipGetSymbolAddress, at handle creation) and kept; nullptr if the lookup fails.
void *scratch_address(int dev) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    const auto it = g_scratch_addr.find(dev);
    if (it != g_scratch_addr.end()) return it->second;
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
        (void)hipGetLastError();
        return nullptr;
    }
    g_scratch_addr[dev] = ptr;
    return ptr;
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

mpgemm_status_t mpgemm_run_bf16x3(mpgemm_handle_t handle, mpgemm_op_t transa,
                                  mpgemm_op_t transb, int64_t m, int64_t n, int64_t k,
                                  const float *alpha, const float *A, int64_t lda,
                                  const float *B, int64_t ldb, const float *beta,
                                  const float *C, int64_t ldc, float *D, void *workspace,
                                  uint64_t workspace_bytes, void *stream) {
    if (!handle || !handle_live(handle)) return MPGEMM_STATUS_NOT_INITIALIZED;
    const mpgemm_status_t st = mpgemm_check_bf16x3(transa, transb, m, n, k, alpha, A, lda, B,
                                                   ldb, beta, C, ldc, D, workspace,
                                                   workspace_bytes);
    if (st != MPGEMM_STATUS_SUCCESS) return st;
    if (m == 0 || n == 0) return MPGEMM_STATUS_SUCCESS;
    const bool ta = transa == MPGEMM_OP_T, tb = transb == MPGEMM_OP_T;
    Bf16x3Layout L;
    if (!bf16x3_layout(ta, tb, m, n, k, L)) return MPGEMM_STATUS_INTERNAL_ERROR;  // checked above
    char *ws = (char *)workspace;
    const void *A3 = ws, *B3 = ws ? ws + L.off_b : nullptr;
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

mpgemm_status_t mpgemm_run_bf16x3_noalloc(mpgemm_handle_t handle, mpgemm_op_t transa,
                                          mpgemm_op_t transb, int64_t m, int64_t n, int64_t k,
                                          const float *alpha, const float *A, int64_t lda,
                                          const float *B, int64_t ldb, const float *beta,
                                          const float *C, int64_t ldc, float *D, void *stream) {
    if (!handle || !handle_live(handle)) return MPGEMM_STATUS_NOT_INITIALIZED;
    if (!handle->scratch) return MPGEMM_STATUS_INTERNAL_ERROR;   // lookup at creation failed
    const uint64_t cap = MPGEMM_NOALLOC_SCRATCH_BYTES;
    const uint64_t need = mpgemm_bf16x3_workspace_size(transa, transb, m, n, k);
    // every other argument as mpgemm_run_bf16x3 checks it; then the scratch limit
    const mpgemm_status_t st =
        mpgemm_check_bf16x3(transa, transb, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, D,
                            handle->scratch, need > cap ? need : cap);
    if (st != MPGEMM_STATUS_SUCCESS) return st;
    if (need > cap) return MPGEMM_STATUS_SCRATCH_TOO_SMALL;
    return mpgemm_run_bf16x3(handle, transa, transb, m, n, k, alpha, A, lda, B, ldb, beta, C,
                             ldc, D, handle->scratch, cap, stream);
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
    h->scratch = scratch_address(dev);   // checked by mpgemm_run_bf16x3_noalloc
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
        memcpy(&p.alpha_i, alpha, sizeof(int32_t));
        memcpy(&p.beta_i, beta, sizeof(int32_t));
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

}  // extern "C"
