/*
 * mpgemm.h -- mixed-precision dense matrix multiply-accumulate on AMD Instinct MI355X (gfx950).
 *
 *     D = alpha * op(A) * op(B) + beta * C
 *
 * with FP16 or BF16 inputs accumulated in FP32, or INT8 inputs accumulated in INT32.
 *
 * The call follows the GEMM statement of "Programming Tensor Cores in CUDA 9"
 * (makelele.cn/d/1827294.html), section on using Tensor Cores through cuBLAS: a handle,
 * transpose flags, m, n, k, alpha, the A, B and C matrices each with an element type and a
 * leading dimension, beta, and a compute (accumulate) type; and its section "Finishing":
 * the product is scaled by alpha and added to C scaled by beta.  The type matrix follows
 * "Mixed-Precision Programming with CUDA 8" (m.ruidan.com/infomation/detail/138780),
 * section on cuBLAS: FP32 compute on FP16 inputs with FP32 or FP16 output, and INT8 inputs
 * with integer (DP4A-style) compute.
 *
 * STORAGE IS ROW-MAJOR.  op(A) is m x k, op(B) is k x n, C and D are m x n.
 *   transa == MPGEMM_OP_N: A is stored m x k, element (i,p) at A[i*lda + p], lda >= k.
 *   transa == MPGEMM_OP_T: A is stored k x m (the buffer holds op(A)^T), element (i,p) at
 *                          A[p*lda + i], lda >= m.
 *   transb == MPGEMM_OP_N: B is stored k x n, element (p,j) at B[p*ldb + j], ldb >= n.
 *   transb == MPGEMM_OP_T: B is stored n x k ("B column-major"), element (p,j) at
 *                          B[j*ldb + p], ldb >= k.
 *   C and D: element (i,j) at [i*ldc + j], ldc >= n.  D has C's type and leading dimension.
 * A column-major caller computes D^T = op(B)^T op(A)^T: it passes (transb, transa, n, m, k,
 * B, ldb, A, lda, C, ldc), which the row-major reading turns back into its own problem.
 *
 * Supported type combinations (anything else returns MPGEMM_STATUS_NOT_SUPPORTED):
 *   a_type = b_type = MPGEMM_R_16F,  compute MPGEMM_R_32F, c_type MPGEMM_R_32F or MPGEMM_R_16F
 *   a_type = b_type = MPGEMM_R_16BF, compute MPGEMM_R_32F, c_type MPGEMM_R_32F or MPGEMM_R_16BF
 *   a_type = b_type = MPGEMM_R_8I,   compute MPGEMM_R_32I, c_type MPGEMM_R_32I
 *   a_type, b_type each MPGEMM_R_8F_E4M3 or MPGEMM_R_8F_E5M2 (either pairing; the two FP8
 *     formats of "NVIDIA Tensor Core mixed-precision computing: principles and applications",
 *     section 4.3.1), compute MPGEMM_R_32F, c_type MPGEMM_R_32F or MPGEMM_R_16BF; here
 *     "compute MPGEMM_R_32F" means an FP32 accumulator between 128-deep instructions only:
 *     the sums inside each instruction keep about 13 bits (see below), so FP8 results are
 *     not FP32-accurate sums of the products
 * FP16/BF16 outputs are rounded once from the FP32 result, to nearest with ties to even.
 * INT32 accumulation and the epilogue wrap modulo 2^32.
 *
 * FP32 result (the rounding steps, which the pages leave to the hardware): the products are
 * accumulated in k order by the matrix cores' block FMA, 8 consecutive k per block ("NVIDIA
 * Tensor Core mixed-precision computing: principles and applications", sections 2.2-2.3
 * and 4.2.1, with gfx950's parameters: products aligned to the block's largest exponent
 * with 24 fraction bits, products cut toward zero and the running sum toward minus infinity
 * below that, the block sum kept to 32 significant bits, then rounded to FP32 to nearest
 * even), starting from zero; the epilogue is alpha * acc when beta == 0, else
 * fma(alpha, acc, beta * c) in FP32.  The result is deterministic: the same inputs give the
 * same bits on every call, tile shape and launch.
 * FP8 inputs accumulate on gfx950's v_mfma_f32_16x16x128_f8f6f4, whose intermediate sums are
 * narrower (measured: groups of 8 products keep about 13 fraction bits below the group's
 * largest exponent, blocks of 16 products in k order are added to the FP32 accumulator in a
 * 24-bit window and the sum rounded to FP32 after each block); results whose partial sums stay
 * on that grid (small integers, for instance) are exact, others carry an error up to about
 * 2^-9 of sum |a b|.
 *
 * Alignment contract (there is no slower fallback path): A, B, C (when read) and D must be
 * 16-byte aligned, and lda, ldb, ldc times the element size must be multiples of 16 bytes
 * (8 elements for FP16/BF16, 16 for INT8 and FP8, 4 for FP32/INT32).  m, n and k are
 * arbitrary up to 2^31 - 1 (k up to 2^31 - 256); larger sizes return
 * MPGEMM_STATUS_NOT_SUPPORTED.
 * Operands are read in whole aligned 16-byte blocks: each row of A and B must be readable up
 * to the end of the 16-byte block holding its last element (true of any buffer whose size is
 * rows * ld elements).  Elements beyond the logical row are never used in the result.
 * The distance in bytes spanned by 256 rows of any operand (256 * ld * element size) must be
 * below 2^31; larger strides return MPGEMM_STATUS_NOT_SUPPORTED.
 *
 * Ownership and ordering: the caller allocates and owns every matrix and keeps it alive and
 * unmodified until the work queued on `stream` has finished.  mpgemm_run allocates no device
 * memory, is asynchronous, and is ordered on `stream` (a hipStream_t; NULL means the null
 * stream).  A handle is bound to the device that was current at mpgemm_create and holds only
 * host state; use one handle per host thread (a handle is not thread-safe).
 *
 * Errors are returned as status codes; nothing aborts and no exception crosses this ABI.
 * Arguments are checked on the host before any device call.  Faults that happen while the
 * queued kernel runs surface at the caller's next synchronisation of `stream`.
 */
#ifndef MPGEMM_H
#define MPGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mpgemm_handle_s *mpgemm_handle_t;

typedef enum { MPGEMM_OP_N = 0, MPGEMM_OP_T = 1 } mpgemm_op_t;

typedef enum {
    MPGEMM_R_16F = 0,   /* IEEE binary16: 1 sign, 5 exponent, 10 fraction bits */
    MPGEMM_R_16BF = 1,  /* bfloat16: upper 16 bits of an IEEE binary32 */
    MPGEMM_R_8I = 2,    /* signed 8-bit integer */
    MPGEMM_R_32F = 3,   /* IEEE binary32 */
    MPGEMM_R_32I = 4,   /* signed 32-bit integer (two's complement) */
    MPGEMM_R_8F_E4M3 = 5, /* FP8 E4M3 (OCP): 1 sign, 4 exponent (bias 7), 3 fraction bits;
                             no infinities, S.1111.111 is NaN; largest 448, smallest 2^-9 */
    MPGEMM_R_8F_E5M2 = 6  /* FP8 E5M2 (OCP): 1 sign, 5 exponent (bias 15), 2 fraction bits;
                             IEEE-style infinities and NaNs; largest 57344, smallest 2^-16 */
} mpgemm_dtype_t;

typedef enum {
    MPGEMM_STATUS_SUCCESS = 0,
    MPGEMM_STATUS_NOT_INITIALIZED = 1, /* handle not created, or already destroyed */
    MPGEMM_STATUS_INVALID_VALUE = 2,   /* null pointer, negative size, ld below its minimum */
    MPGEMM_STATUS_NOT_SUPPORTED = 3,   /* type combination, alignment or stride outside the contract */
    MPGEMM_STATUS_ALLOC_FAILED = 4,    /* host allocation of the handle failed */
    MPGEMM_STATUS_NO_DEVICE = 5,       /* no HIP device, or the current device is not gfx950 */
    MPGEMM_STATUS_LAUNCH_FAILED = 6,   /* the kernel launch was rejected by the runtime */
    MPGEMM_STATUS_INTERNAL_ERROR = 7,
    MPGEMM_STATUS_WRONG_DEVICE = 8,    /* current device differs from the handle's device */
    MPGEMM_STATUS_SCRATCH_TOO_SMALL = 9 /* mpgemm_run_bf16x3_noalloc: the split operands need
                                           more than MPGEMM_NOALLOC_SCRATCH_BYTES */
} mpgemm_status_t;

/* Size of the library's fixed scratch buffer (per device) used by mpgemm_run_bf16x3_noalloc. */
#define MPGEMM_NOALLOC_SCRATCH_BYTES (64ull << 20)

/* Create a handle bound to the current HIP device.  Returns MPGEMM_STATUS_NO_DEVICE when no
 * device is present or the device is not a gfx950, MPGEMM_STATUS_INVALID_VALUE when
 * `handle` is NULL, MPGEMM_STATUS_ALLOC_FAILED when host memory runs out.  On failure
 * *handle is set to NULL (when handle is non-NULL). */
mpgemm_status_t mpgemm_create(mpgemm_handle_t *handle);

/* Queue D = alpha * op(A) * op(B) + beta * C on `stream` (see the contract above).
 *   alpha, beta: host pointers to a float (compute MPGEMM_R_32F) or an int32_t
 *                (compute MPGEMM_R_32I), read before the call returns.
 *   C:           read only when *beta != 0; may be NULL otherwise.  D == C (in place) is
 *                allowed; any other overlap of D with A, B or C is undefined.
 *   m == 0 or n == 0 returns MPGEMM_STATUS_SUCCESS without touching the device.
 *   k == 0 gives D = beta * C (D = 0 when beta == 0); A and B may then be NULL.
 *   alpha == 0 is not special-cased: NaN or Inf in A or B still reaches D.
 * The current HIP device must be the handle's (else MPGEMM_STATUS_WRONG_DEVICE). */
mpgemm_status_t mpgemm_run(mpgemm_handle_t handle, mpgemm_op_t transa, mpgemm_op_t transb,
                           int64_t m, int64_t n, int64_t k, const void *alpha,
                           const void *A, mpgemm_dtype_t a_type, int64_t lda,
                           const void *B, mpgemm_dtype_t b_type, int64_t ldb,
                           const void *beta, const void *C, mpgemm_dtype_t c_type, int64_t ldc,
                           void *D, mpgemm_dtype_t compute_type, void *stream);

/* FP32 GEMM from BF16 pieces (multiword emulation: "NVIDIA Tensor Core mixed-precision
 * computing: principles and applications", section 5.1, splits high-precision operands into
 * pieces the matrix cores take and sums the partial products; "The CUDA Handbook" section
 * 17.5 does FP32 GEMM on Tensor Cores by rounding inputs to TF32).  Queues on `stream`
 *
 *   D = alpha * op(A) * op(B) + beta * C        A, B, C, D, alpha, beta: FP32
 *
 * with every element x of A and B split into x_hi = RN_bf16(x) and x_lo = RN_bf16(x - x_hi)
 * (round to nearest even; x - x_hi is exact in FP32; x_lo = 0 when x_hi is Inf or NaN, so
 * Inf and NaN propagate as in an FP32 product, and finite x beyond BF16's largest value,
 * about 3.39e38, counts as infinite), and op(A) op(B) replaced by
 *
 *   A_hi B_hi + A_lo B_hi + A_hi B_lo
 *
 * computed as ONE BF16 GEMM of the kind mpgemm_run performs (FP32 accumulation, same
 * numerics and epilogue) over k3 = 3 kp, kp = k rounded up to a multiple of 8: the k index
 * runs through the three products in that order, each zero-padded from k to kp.  Per
 * element the representation error is at most about 3 * 2^-16 |a b| (A_lo B_lo and the
 * residuals are dropped), against 2^-11 for inputs rounded to TF32.
 *
 *   workspace:       device memory for the split operands, at least
 *                    mpgemm_bf16x3_workspace_size(transa, transb, m, n, k) bytes, 256-byte
 *                    aligned, not overlapping A, B, C or D; overwritten, owned by the caller,
 *                    and in use until the queued work finishes.  Layout (BF16, row-major):
 *                    A3 at offset 0: m x k3 (ld k3) for transa == N, k3 x m (ld m rounded up
 *                    to 8) for transa == T; B3 at the next 256-byte boundary: k3 x n (ld n
 *                    rounded up to 8) for transb == N, n x k3 (ld k3) for transb == T.
 *   Alignment:       A, B, C (when read), D 16-byte aligned; lda, ldb, ldc multiples of 4.
 *   Other arguments, ownership and errors as for mpgemm_run; a workspace that is NULL (with
 *   a nonzero requirement) or smaller than required returns MPGEMM_STATUS_INVALID_VALUE, a
 *   misaligned one MPGEMM_STATUS_NOT_SUPPORTED.  mpgemm_run_bf16x3 allocates nothing. */
mpgemm_status_t mpgemm_run_bf16x3(mpgemm_handle_t handle, mpgemm_op_t transa,
                                  mpgemm_op_t transb, int64_t m, int64_t n, int64_t k,
                                  const float *alpha, const float *A, int64_t lda,
                                  const float *B, int64_t ldb, const float *beta,
                                  const float *C, int64_t ldc, float *D, void *workspace,
                                  uint64_t workspace_bytes, void *stream);

/* mpgemm_run_bf16x3 without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and results, with the split operands kept in a fixed device array of
 * the library (MPGEMM_NOALLOC_SCRATCH_BYTES = 64 MiB per device, reserved when the library's
 * code is first loaded on a device and held until the process ends) instead of a
 * caller-provided workspace.  The call allocates nothing and frees nothing.
 *   - Problems whose workspace, mpgemm_bf16x3_workspace_size(transa, transb, m, n, k),
 *     exceeds MPGEMM_NOALLOC_SCRATCH_BYTES return MPGEMM_STATUS_SCRATCH_TOO_SMALL without
 *     launching anything (for example m x k + k x n up to about 11 million elements fits).
 *   - All calls on one device share that device's buffer, which keeps the last call's
 *     contents: calls that may overlap on one device (different streams, handles or host
 *     threads without ordering between them) race and give wrong results; calls ordered on
 *     one stream are safe.  No byte of it needs to start at zero: each call writes every
 *     byte its GEMM reads.
 *   - Other arguments, ownership and errors as for mpgemm_run_bf16x3; the handle must have
 *     been created on the current device (its creation looks the buffer's address up;
 *     MPGEMM_STATUS_INTERNAL_ERROR if that failed). */
mpgemm_status_t mpgemm_run_bf16x3_noalloc(mpgemm_handle_t handle, mpgemm_op_t transa,
                                          mpgemm_op_t transb, int64_t m, int64_t n, int64_t k,
                                          const float *alpha, const float *A, int64_t lda,
                                          const float *B, int64_t ldb, const float *beta,
                                          const float *C, int64_t ldc, float *D, void *stream);

/* Host-only argument check of mpgemm_run_bf16x3: returns exactly the status mpgemm_run_bf16x3
 * would return for these arguments before touching the device (the workspace's size and
 * alignment included); needs no handle and no device, and dereferences only alpha and beta. */
mpgemm_status_t mpgemm_check_bf16x3(mpgemm_op_t transa, mpgemm_op_t transb, int64_t m,
                                    int64_t n, int64_t k, const float *alpha, const float *A,
                                    int64_t lda, const float *B, int64_t ldb, const float *beta,
                                    const float *C, int64_t ldc, const float *D,
                                    const void *workspace, uint64_t workspace_bytes);

/* GEMM with a 2:4 structured-sparse A (the page "稀疏张量核心加速模板计算的技术解析" on sparse tensor
 * cores for stencils, sections
 * 1.2.1 and 1.3.2: at most two nonzeros in every group of 4 consecutive k, stored as the kept
 * values plus 2 bits of metadata per kept value; here on gfx950's v_smfmac sparse matrix
 * cores).  Queues on `stream`
 *
 *   D = alpha * A * op(B) + beta * C,   A(i, 4q + idx(i, j)) += Ac(i, j) for j = 2q, 2q + 1
 *
 * i.e. D(i, c) = alpha * sum_j Ac(i, j) * op(B)(4 (j / 2) + idx(i, j), c) + beta * C(i, c).
 *   Ac:     the kept values, m x k/2, row-major: Ac(i, j) at Ac[i*lda + j], lda >= k/2.
 *   meta:   m rows of ld_meta bytes, ld_meta >= k/8: idx(i, j) is bits 2 (j % 4) .. +1 of byte
 *           meta[i*ld_meta + j/4] (2 bits per kept value, in k order, little-endian).  The two
 *           indices of a group are normally distinct; equal ones make both values multiply
 *           the same row of op(B).
 *   B, C, D, transb, ldb, ldc, alpha, beta: as for mpgemm_run; A is never transposed.
 *   Types:  a_type = b_type = MPGEMM_R_16F or MPGEMM_R_16BF, compute MPGEMM_R_32F, c_type
 *           MPGEMM_R_32F or a_type: numerics as for the dense FP16/BF16 GEMM, over the k/2
 *           kept products (blocks of 8 kept products, in kept order); or a_type = b_type =
 *           MPGEMM_R_8I with compute and c_type MPGEMM_R_32I: exact, wrapping INT32 arithmetic
 *           as for the dense INT8 GEMM (alpha and beta point to int32_t); or a_type and b_type
 *           each MPGEMM_R_8F_E4M3 or MPGEMM_R_8F_E5M2, compute MPGEMM_R_32F, c_type
 *           MPGEMM_R_32F or MPGEMM_R_16BF: numerics as for the dense FP8 GEMM.
 *   Sizes:  k a multiple of 128 (else MPGEMM_STATUS_NOT_SUPPORTED); m, n arbitrary.
 *   Alignment: Ac, meta, B, C (when read), D 16-byte aligned; rows of Ac and B (lda, ldb
 *           elements) and of the metadata (ld_meta bytes) multiples of 16 bytes, ldc as for
 *           mpgemm_run.
 * Ownership, ordering and errors as for mpgemm_run; nothing is allocated. */
mpgemm_status_t mpgemm_run_sp24(mpgemm_handle_t handle, mpgemm_op_t transb, int64_t m, int64_t n,
                                int64_t k, const void *alpha, const void *Ac,
                                mpgemm_dtype_t a_type, int64_t lda, const void *meta,
                                int64_t ld_meta, const void *B, mpgemm_dtype_t b_type,
                                int64_t ldb, const void *beta, const void *C,
                                mpgemm_dtype_t c_type, int64_t ldc, void *D,
                                mpgemm_dtype_t compute_type, void *stream);

/* Host-only argument check of mpgemm_run_sp24 (as mpgemm_check is for mpgemm_run). */
mpgemm_status_t mpgemm_check_sp24(mpgemm_op_t transb, int64_t m, int64_t n, int64_t k,
                                  const void *alpha, const void *Ac, mpgemm_dtype_t a_type,
                                  int64_t lda, const void *meta, int64_t ld_meta, const void *B,
                                  mpgemm_dtype_t b_type, int64_t ldb, const void *beta,
                                  const void *C, mpgemm_dtype_t c_type, int64_t ldc,
                                  const void *D, mpgemm_dtype_t compute_type);

/* Workspace bytes mpgemm_run_bf16x3 needs for these sizes (0 when m, n or k is 0); 0 also
 * for negative sizes or flags outside MPGEMM_OP_N / MPGEMM_OP_T.  Host-only. */
uint64_t mpgemm_bf16x3_workspace_size(mpgemm_op_t transa, mpgemm_op_t transb, int64_t m,
                                      int64_t n, int64_t k);

/* Host-only argument check: returns exactly the status mpgemm_run would return for these
 * arguments before touching the device (MPGEMM_STATUS_SUCCESS if it would launch).  It needs
 * no handle and no device, and dereferences only alpha and beta. */
mpgemm_status_t mpgemm_check(mpgemm_op_t transa, mpgemm_op_t transb, int64_t m, int64_t n,
                             int64_t k, const void *alpha, const void *A, mpgemm_dtype_t a_type,
                             int64_t lda, const void *B, mpgemm_dtype_t b_type, int64_t ldb,
                             const void *beta, const void *C, mpgemm_dtype_t c_type, int64_t ldc,
                             const void *D, mpgemm_dtype_t compute_type);

/* Release a handle.  NULL or an unknown/destroyed handle returns
 * MPGEMM_STATUS_NOT_INITIALIZED.  Work already queued is not affected. */
mpgemm_status_t mpgemm_destroy(mpgemm_handle_t handle);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *mpgemm_status_string(mpgemm_status_t status);

/* Tile shape (rows x columns of D per workgroup) that mpgemm_run picks for an m x n output
 * with inputs of type a_type on a device with 256 compute units (a whole MI355X; mpgemm_run
 * uses the handle's device's count), written to *tile_m and *tile_n.  Host-only; for
 * diagnostics and benchmarks.  Returns MPGEMM_STATUS_INVALID_VALUE for negative sizes or null
 * outputs. */
mpgemm_status_t mpgemm_tile_shape(int64_t m, int64_t n, mpgemm_dtype_t a_type, int *tile_m,
                                  int *tile_n);

#ifdef __cplusplus
}
#endif

#endif /* MPGEMM_H */
