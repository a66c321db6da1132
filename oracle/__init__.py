"""CPU oracle and comparator for D = alpha * op(A) * op(B) + beta * C.

TEST INFRASTRUCTURE ONLY.  The GPU library (``mixed_precision_dense_amd``) never imports,
links or calls anything in this package, and this package imports nothing from it.  Only
``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` use it.

The arithmetic lives in ``mpgemm_oracle.c`` (plain C, fp64 / int64); this module builds it
with gcc, wraps it with ctypes, and holds the comparator that decides whether a GPU result
is acceptable.  Every stored array is a numpy array of raw storage: FP16 and BF16 as
``uint16`` bit patterns, FP32 as ``float32``, INT8 as ``int8``, INT32 as ``int32``, each
row-major with an explicit leading dimension.

Pages (cited by title and section):
  * "Programming Tensor Cores in CUDA 9" (makelele.cn/d/1827294.html) -- the GEMM call and
    its alpha/beta epilogue (sections on cuBLAS usage and "Finishing").
  * "Mixed-Precision Programming with CUDA 8" (m.ruidan.com/infomation/detail/138780) --
    number formats (Figure 1) and the DP4A integer dot product (Figure 2).
  * "NVIDIA Tensor Core mixed-precision computing: principles and applications"
    (jsqmd.com/news/1087138) -- section 2.3, rounding model and the error expression
    E = sum(a_i b_i)(1 + d_i) + c(1 + d_c), |d| <= 2^-p, which the bound below instantiates
    with FP32's p = 23; sections 2.2-2.3, 3.1 and 4.2.1, the block-FMA model of matrix-core
    accumulation (``gemm_mfma``), whose open parameters are set to gfx950's measured ones.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mpgemm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmpgemm_oracle.so")
# A differently built copy of the same source (the sanitizer build of
# tests/test_host_sanitizers.py) may be loaded in its place.
_LIB_OVERRIDE = os.environ.get("MPGEMM_ORACLE_LIB")

# Type codes private to the oracle (mirrors the enum in mpgemm_oracle.c).
_CODES = {"f16": 0, "bf16": 1, "i8": 2, "f32": 3, "i32": 4, "e4m3": 5, "e5m2": 6}
_STORAGE = {"f16": np.uint16, "bf16": np.uint16, "i8": np.int8, "f32": np.float32,
            "i32": np.int32, "e4m3": np.uint8, "e5m2": np.uint8}
FP8 = ("e4m3", "e5m2")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction) and return its path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib: Optional[ctypes.CDLL] = None


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
        i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        lib.oracle_decode.restype = dbl
        lib.oracle_decode.argtypes = [ctypes.c_uint64, i32, i32]
        lib.oracle_encode_rne.restype = ctypes.c_uint64
        lib.oracle_encode_rne.argtypes = [dbl, i32, i32]
        lib.oracle_gemm_fp_points.restype = i32
        lib.oracle_gemm_fp_points.argtypes = [i32, i32, i64, i64, i64, dbl, vp, i32, i64, vp,
                                              i32, i64, dbl, vp, i32, i64, i64, vp, vp, vp,
                                              vp, vp]
        lib.oracle_gemm_fp_full.restype = i32
        lib.oracle_gemm_fp_full.argtypes = [i32, i32, i64, i64, i64, dbl, vp, i32, i64, vp,
                                            i32, i64, dbl, vp, i32, i64, vp, vp, vp]
        lib.oracle_gemm_int_points.restype = i32
        lib.oracle_gemm_int_points.argtypes = [i32, i32, i64, i64, i64, i64, vp, i64, vp, i64,
                                               i64, vp, i64, i64, vp, vp, vp]
        lib.oracle_gemm_int_full.restype = i32
        lib.oracle_gemm_int_full.argtypes = [i32, i32, i64, i64, i64, i64, vp, i64, vp, i64,
                                             i64, vp, i64, vp]
        lib.oracle_round_array.restype = i32
        lib.oracle_round_array.argtypes = [vp, i64, i32, vp]
        flt = ctypes.c_float
        lib.oracle_gemm_mfma_points.restype = i32
        lib.oracle_gemm_mfma_points.argtypes = [i32, i32, i64, i64, i64, flt, vp, i32, i64, vp,
                                                i32, i64, flt, vp, i32, i64, i32, i32, i32,
                                                i32, i64, vp, vp, vp]
        lib.oracle_gemm_mfma_full.restype = i32
        lib.oracle_gemm_mfma_full.argtypes = [i32, i32, i64, i64, i64, flt, vp, i32, i64, vp,
                                              i32, i64, flt, vp, i32, i64, i32, i32, i32, i32,
                                              vp]
        lib.oracle_split_bf16.restype = i32
        lib.oracle_split_bf16.argtypes = [vp, i64, vp, vp]
        lib.oracle_gemm_f32_points.restype = i32
        lib.oracle_gemm_f32_points.argtypes = [i32, i32, i64, dbl, vp, i64, vp, i64, dbl, vp,
                                               i64, i64, vp, vp, vp, vp]
        lib.oracle_decode_e4m3.restype = dbl
        lib.oracle_decode_e4m3.argtypes = [ctypes.c_uint32]
        lib.oracle_gemm_fp8_points.restype = i32
        lib.oracle_gemm_fp8_points.argtypes = lib.oracle_gemm_fp_points.argtypes
        lib.oracle_gemm_fp8_full.restype = i32
        lib.oracle_gemm_fp8_full.argtypes = lib.oracle_gemm_fp_full.argtypes
        lib.oracle_gemm_sp24_points.restype = i32
        lib.oracle_gemm_sp24_points.argtypes = [i32, i64, dbl, vp, i32, i64, vp, i64, vp, i64, dbl,
                                                vp, i32, i64, i64, vp, vp, vp, vp, vp]
        lib.oracle_gemm_sp24_mfma_points.restype = i32
        lib.oracle_gemm_sp24_mfma_points.argtypes = [i32, i64, flt, vp, i32, i64, vp, i64, vp, i64,
                                                     flt, vp, i32, i64, i32, i32, i32, i32, i64,
                                                     vp, vp, vp]
        lib.oracle_gemm_sp24_int_points.restype = i32
        lib.oracle_gemm_sp24_int_points.argtypes = [i32, i64, i64, vp, i64, vp, i64, vp, i64, i64,
                                                    vp, i64, i64, vp, vp, vp]
        lib.oracle_gemm_sp24_fp8_points.restype = i32
        lib.oracle_gemm_sp24_fp8_points.argtypes = [i32, i64, dbl, vp, i32, i64, vp, i64, vp, i32,
                                                    i64, dbl, vp, i32, i64, i64, vp, vp, vp, vp,
                                                    vp]
        lib.oracle_gemm_fp8_mfma_points.restype = i32
        lib.oracle_gemm_fp8_mfma_points.argtypes = [i32, i32, i64, flt, vp, i32, i64, vp, i32, i64,
                                                    flt, vp, i32, i64, i32, i32, i32, i32, i32,
                                                    i32, i32, i64, vp, vp, vp]
        lib.oracle_gemm_sp24_fp8_mfma_points.restype = i32
        lib.oracle_gemm_sp24_fp8_mfma_points.argtypes = [i32, i64, flt, vp, i32, i64, vp, i64, vp,
                                                         i32, i64, flt, vp, i32, i64, i32, i32,
                                                         i32, i32, i32, i32, i32, i64, vp, vp, vp]
        lib.oracle_num_threads.restype = i32
        lib.oracle_num_threads.argtypes = []
        lib.oracle_set_num_threads.restype = None
        lib.oracle_set_num_threads.argtypes = [i32]
        _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle's loops run on."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Run the oracle's loops on ``n`` OpenMP threads from now on (timing runs)."""
    _load().oracle_set_num_threads(int(n))


# ----------------------------------------------------------------------------- formats
_FIELDS = {"f16": (5, 10), "bf16": (8, 7), "f32": (8, 23)}


def decode(bits: int, fmt: str) -> float:
    """Value of one bit pattern of ``fmt`` ('f16', 'bf16', 'f32', 'e4m3', 'e5m2'), from the
    field definition."""
    if fmt == "e4m3":
        return float(_load().oracle_decode_e4m3(int(bits)))
    if fmt == "e5m2":
        return float(_load().oracle_decode(int(bits), 5, 2))
    e, m = _FIELDS[fmt]
    return float(_load().oracle_decode(int(bits), e, m))


def encode_rne(value: float, fmt: str) -> int:
    """Bit pattern of ``value`` rounded to nearest-even in ``fmt``."""
    e, m = _FIELDS[fmt]
    return int(_load().oracle_encode_rne(float(value), e, m))


def round_to(v: np.ndarray, fmt: str) -> np.ndarray:
    """Round float64 values once (nearest-even) to ``fmt``; returns raw storage."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint32 if fmt == "f32" else np.uint16)
    rc = _load().oracle_round_array(v.ctypes.data, v.size, _CODES[fmt], out.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle cannot round to {fmt}")
    return out.view(np.float32) if fmt == "f32" else out


# ----------------------------------------------------------------------------- GEMM
@dataclass
class FpReference:
    """Oracle result for floating-point outputs, per output element."""
    v: np.ndarray    # alpha*s + beta*c in double, before output rounding
    S: np.ndarray    # sum_p |a(i,p) * b(p,j)|
    bc: np.ndarray   # beta * c (0 where beta == 0)


def _ptr(a: Optional[np.ndarray]) -> Optional[int]:
    return None if a is None else a.ctypes.data


def _check_storage(name: str, arr: Optional[np.ndarray], fmt: str) -> None:
    if arr is None:
        return
    if arr.dtype != _STORAGE[fmt]:
        raise TypeError(f"{name}: expected storage {np.dtype(_STORAGE[fmt])} for {fmt}, "
                        f"got {arr.dtype}")
    if not arr.flags.c_contiguous:
        raise ValueError(f"{name} must be C-contiguous raw storage")


def gemm_fp(transa: bool, transb: bool, m: int, n: int, k: int, alpha: float,
            A: np.ndarray, atype: str, lda: int, B: np.ndarray, btype: str, ldb: int,
            beta: float, C: Optional[np.ndarray], ctype: str, ldc: int,
            points: Optional[tuple] = None) -> FpReference:
    """Floating-point oracle.  With ``points=(ii, jj)`` only those elements are computed
    (each one from the definition); otherwise the full m x n output."""
    _check_storage("A", A, atype)
    _check_storage("B", B, btype)
    if beta != 0.0:
        _check_storage("C", C, ctype)
    else:
        C = None
    lib = _load()
    args = (int(bool(transa)), int(bool(transb)), m, n, k, float(alpha), _ptr(A),
            _CODES[atype], lda, _ptr(B), _CODES[btype], ldb, float(beta), _ptr(C),
            _CODES[ctype], ldc)
    if points is None:
        v = np.empty((m, n), np.float64)
        S = np.empty((m, n), np.float64)
        bc = np.empty((m, n), np.float64)
        rc = lib.oracle_gemm_fp_full(*args, v.ctypes.data, S.ctypes.data, bc.ctypes.data)
    else:
        ii = np.ascontiguousarray(points[0], dtype=np.int64)
        jj = np.ascontiguousarray(points[1], dtype=np.int64)
        v = np.empty(ii.shape, np.float64)
        S = np.empty(ii.shape, np.float64)
        bc = np.empty(ii.shape, np.float64)
        rc = lib.oracle_gemm_fp_points(*args, ii.size, ii.ctypes.data, jj.ctypes.data,
                                       v.ctypes.data, S.ctypes.data, bc.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle rejected types a={atype} b={btype} c={ctype} (rc={rc})")
    return FpReference(v, S, bc)


def gemm_fp8(transa: bool, transb: bool, m: int, n: int, k: int, alpha: float,
             A: np.ndarray, atype: str, lda: int, B: np.ndarray, btype: str, ldb: int,
             beta: float, C: Optional[np.ndarray], ctype: str, ldc: int,
             points: Optional[tuple] = None) -> FpReference:
    """FP8 (E4M3 / E5M2, A and B each) oracle: exact products, double sums, as gemm_fp."""
    _check_storage("A", A, atype)
    _check_storage("B", B, btype)
    if beta != 0.0:
        _check_storage("C", C, ctype)
    else:
        C = None
    lib = _load()
    args = (int(bool(transa)), int(bool(transb)), m, n, k, float(alpha), _ptr(A),
            _CODES[atype], lda, _ptr(B), _CODES[btype], ldb, float(beta), _ptr(C),
            _CODES[ctype], ldc)
    if points is None:
        v = np.empty((m, n), np.float64)
        S = np.empty((m, n), np.float64)
        bc = np.empty((m, n), np.float64)
        rc = lib.oracle_gemm_fp8_full(*args, v.ctypes.data, S.ctypes.data, bc.ctypes.data)
    else:
        ii = np.ascontiguousarray(points[0], dtype=np.int64)
        jj = np.ascontiguousarray(points[1], dtype=np.int64)
        v = np.empty(ii.shape, np.float64)
        S = np.empty(ii.shape, np.float64)
        bc = np.empty(ii.shape, np.float64)
        rc = lib.oracle_gemm_fp8_points(*args, ii.size, ii.ctypes.data, jj.ctypes.data,
                                        v.ctypes.data, S.ctypes.data, bc.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle rejected FP8 types a={atype} b={btype} c={ctype}")
    return FpReference(v, S, bc)


# Block-FMA parameters of gfx950's v_mfma_f32_16x16x32_{f16,bf16}: 8 products per block, 24
# fraction bits below the block's exponent (the 2+23+1 accumulator of the numerics page), and
# a block sum that keeps 32 significant bits before its rounding to FP32.
MFMA_BLOCK = 8
MFMA_FRAC = 24
MFMA_SUM_BITS = 32


def gemm_mfma(transa: bool, transb: bool, m: int, n: int, k: int, alpha: float,
              A: np.ndarray, atype: str, lda: int, B: np.ndarray, btype: str, ldb: int,
              beta: float, C: Optional[np.ndarray], ctype: str, ldc: int, out_fmt: str,
              points: Optional[tuple] = None, nblk: int = MFMA_BLOCK,
              frac: int = MFMA_FRAC, sum_bits: int = MFMA_SUM_BITS) -> np.ndarray:
    """Block-FMA model of matrix-core accumulation (mpgemm_oracle.c): the output in
    ``out_fmt`` storage, bit for bit.  alpha and beta are FP32 values (they are rounded to
    FP32 here, as the C ABI takes them).  With ``points=(ii, jj)`` only those elements."""
    _check_storage("A", A, atype)
    _check_storage("B", B, btype)
    if beta != 0.0:
        _check_storage("C", C, ctype)
    else:
        C = None
    lib = _load()
    args = (int(bool(transa)), int(bool(transb)), m, n, k, float(np.float32(alpha)), _ptr(A),
            _CODES[atype], lda, _ptr(B), _CODES[btype], ldb, float(np.float32(beta)),
            _ptr(C), _CODES[ctype], ldc, _CODES[out_fmt], int(nblk), int(frac),
            int(sum_bits))
    odt = np.uint32 if out_fmt == "f32" else np.uint16
    if points is None:
        D = np.empty((m, n), odt)
        rc = lib.oracle_gemm_mfma_full(*args, D.ctypes.data)
    else:
        ii = np.ascontiguousarray(points[0], dtype=np.int64)
        jj = np.ascontiguousarray(points[1], dtype=np.int64)
        D = np.empty(ii.shape, odt)
        rc = lib.oracle_gemm_mfma_points(*args, ii.size, ii.ctypes.data, jj.ctypes.data,
                                         D.ctypes.data)
    if rc != 0:
        raise ValueError(f"block model rejected a={atype} b={btype} c={ctype} out={out_fmt} "
                         f"nblk={nblk} frac={frac} sum_bits={sum_bits}")
    return D.view(np.float32) if out_fmt == "f32" else D


# ----------------------------------------------------------------------------- FP32 via BF16 pieces
def split_bf16(x: np.ndarray) -> tuple:
    """x_hi = RN_bf16(x), x_lo = RN_bf16(x - x_hi) (0 where x_hi is not finite), as BF16
    patterns of x's shape (mpgemm_oracle.c, oracle_split_bf16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    hi = np.empty(x.shape, np.uint16)
    lo = np.empty(x.shape, np.uint16)
    _load().oracle_split_bf16(x.ctypes.data, x.size, hi.ctypes.data, lo.ctypes.data)
    return hi, lo


def _rup8(v: int) -> int:
    return (v + 7) // 8 * 8


def bf16x3_operands(transa: bool, transb: bool, m: int, n: int, k: int, A: np.ndarray,
                    lda: int, B: np.ndarray, ldb: int) -> tuple:
    """The BF16 operands of the three-product GEMM, built from their definition: k3 = 3 kp
    (kp = k rounded up to 8); op(A3) = [A_hi | A_lo | A_hi] and op(B3) = [B_hi ; B_hi ; B_lo]
    along k, each piece zero-padded from k to kp; stored like A and B (transposed when
    transa / transb), leading dimensions k3 along k and the other size rounded up to 8.
    Returns (A3, lda3, B3, ldb3, k3)."""
    kp = _rup8(k)
    k3 = 3 * kp
    opA = (A[:k, :m].T if transa else A[:m, :k]).astype(np.float32)     # m x k
    opB = (B[:n, :k].T if transb else B[:k, :n]).astype(np.float32)     # k x n
    ah, al = split_bf16(opA)
    bh, bl = split_bf16(opB)
    a3 = np.zeros((m, k3), np.uint16)
    for piece, part in enumerate((ah, al, ah)):
        a3[:, piece * kp: piece * kp + k] = part
    b3 = np.zeros((k3, n), np.uint16)
    for piece, part in enumerate((bh, bh, bl)):
        b3[piece * kp: piece * kp + k, :] = part
    if transa:
        lda3 = _rup8(m)
        A3 = np.zeros((k3, lda3), np.uint16)
        A3[:, :m] = a3.T
    else:
        lda3 = k3
        A3 = a3
    if transb:
        ldb3 = k3
        B3 = np.ascontiguousarray(b3.T)
    else:
        ldb3 = _rup8(n)
        B3 = np.zeros((k3, ldb3), np.uint16)
        B3[:, :n] = b3
    return np.ascontiguousarray(A3), lda3, np.ascontiguousarray(B3), ldb3, k3


def gemm_bf16x3(transa: bool, transb: bool, m: int, n: int, k: int, alpha: float,
                A: np.ndarray, lda: int, B: np.ndarray, ldb: int, beta: float,
                C: Optional[np.ndarray], ldc: int, points: Optional[tuple] = None):
    """The three-product GEMM under the block-FMA model: FP32 output, bit for bit (also the
    pieces, for the caller's checks).  Returns (D, (A3, lda3, B3, ldb3, k3))."""
    ops = bf16x3_operands(transa, transb, m, n, k, A, lda, B, ldb)
    A3, lda3, B3, ldb3, k3 = ops
    D = gemm_mfma(transa, transb, m, n, k3, alpha, A3, "bf16", lda3, B3, "bf16", ldb3, beta,
                  C, "f32", ldc, "f32", points=points)
    return D, ops


def gemm_f32(transa: bool, transb: bool, m: int, n: int, k: int, alpha: float,
             A: np.ndarray, lda: int, B: np.ndarray, ldb: int, beta: float,
             C: Optional[np.ndarray], ldc: int, points: Optional[tuple] = None) -> tuple:
    """FP32 GEMM in double (exact products, double sums): (v, S) at the points (default all)."""
    if points is None:
        ii, jj = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
        ii, jj = ii.reshape(-1), jj.reshape(-1)
    else:
        ii, jj = points
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    A = np.ascontiguousarray(A, dtype=np.float32)
    B = np.ascontiguousarray(B, dtype=np.float32)
    Cp = None if beta == 0.0 else np.ascontiguousarray(C, dtype=np.float32)
    v = np.empty(ii.shape, np.float64)
    S = np.empty(ii.shape, np.float64)
    _load().oracle_gemm_f32_points(int(bool(transa)), int(bool(transb)), k, float(alpha),
                                   A.ctypes.data, lda, B.ctypes.data, ldb, float(beta),
                                   _ptr(Cp), ldc, ii.size, ii.ctypes.data, jj.ctypes.data,
                                   v.ctypes.data, S.ctypes.data)
    if points is None:
        v, S = v.reshape(m, n), S.reshape(m, n)
    return v, S


# Representation error of the three products per element: |a b - (a_hi b_hi + a_lo b_hi +
# a_hi b_lo)| <= (3 u^2 + 2 u^3 + ...) |a b| with u = 2^-8 (BF16 unit roundoff).
BF16X3_PRODUCT_ERROR = 3.0 * 2.0 ** -16 * (1.0 + 2.0 ** -6)


def bf16x3_bound(S: np.ndarray, k: int, alpha: float, bc: np.ndarray) -> np.ndarray:
    """Radius around the double FP32 GEMM within which the three-product result must lie:
    the products' representation error, FP32 accumulation of 3 kp terms (the section 2.3
    bound with p = 23, on sums of |pieces| <= (1 + 2^-7) S), one rounding of alpha * acc and
    of beta * c, and the oracle's own double error."""
    k3 = 3 * _rup8(k)
    a = abs(alpha)
    keff = k3 if _is_pow2_or_zero(alpha) else k3 + 1
    return (a * S * (BF16X3_PRODUCT_ERROR + keff * 2.0 ** -23 * (1.0 + 2.0 ** -7))
            + 2.0 ** -23 * np.abs(bc) + a * max(k - 1, 0) * 2.0 ** -53 * S + 1e-300)


def gemm_sp24(transb: bool, m: int, n: int, k: int, alpha: float, Ac: np.ndarray, atype: str,
              lda: int, meta: np.ndarray, ld_meta: int, B: np.ndarray, ldb: int, beta: float,
              C: Optional[np.ndarray], ctype: str, ldc: int,
              points: Optional[tuple] = None, btype: Optional[str] = None) -> FpReference:
    """2:4 structured-sparse A (kept values Ac, metadata meta), dense B of the same type (FP8:
    ``btype`` may be the other format): exact products, double sums, as gemm_fp
    (mpgemm_oracle.c, oracle_gemm_sp24_points / oracle_gemm_sp24_fp8_points)."""
    btype = atype if btype is None else btype
    _check_storage("A", Ac, atype)
    _check_storage("B", B, btype)
    if beta != 0.0:
        _check_storage("C", C, ctype)
    else:
        C = None
    meta = np.ascontiguousarray(meta, dtype=np.uint8)
    if points is None:
        ii, jj = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
        ii, jj = ii.reshape(-1), jj.reshape(-1)
    else:
        ii, jj = points
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    v = np.empty(ii.shape, np.float64)
    S = np.empty(ii.shape, np.float64)
    bc = np.empty(ii.shape, np.float64)
    if atype in FP8:
        rc = _load().oracle_gemm_sp24_fp8_points(
            int(bool(transb)), k, float(alpha), _ptr(Ac), _CODES[atype], lda, meta.ctypes.data,
            ld_meta, _ptr(B), _CODES[btype], ldb, float(beta), _ptr(C), _CODES[ctype], ldc,
            ii.size, ii.ctypes.data, jj.ctypes.data, v.ctypes.data, S.ctypes.data,
            bc.ctypes.data)
    else:
        rc = _load().oracle_gemm_sp24_points(int(bool(transb)), k, float(alpha), _ptr(Ac),
                                             _CODES[atype], lda, meta.ctypes.data, ld_meta,
                                             _ptr(B), ldb, float(beta), _ptr(C), _CODES[ctype],
                                             ldc, ii.size, ii.ctypes.data, jj.ctypes.data,
                                             v.ctypes.data, S.ctypes.data, bc.ctypes.data)
    if rc != 0:
        raise ValueError(f"sparse oracle rejected type {atype}")
    if points is None:
        v, S, bc = v.reshape(m, n), S.reshape(m, n), bc.reshape(m, n)
    return FpReference(v, S, bc)


def gemm_sp24_int(transb: bool, m: int, n: int, k: int, alpha: int, Ac: np.ndarray, lda: int,
                  meta: np.ndarray, ld_meta: int, B: np.ndarray, ldb: int, beta: int,
                  C: Optional[np.ndarray], ldc: int, points: Optional[tuple] = None) -> np.ndarray:
    """INT8 2:4 sparse A -> INT32, exact, wrapping modulo 2^32 (mpgemm_oracle.c,
    oracle_gemm_sp24_int_points).  Returns int32 values (m x n, or at the points)."""
    _check_storage("A", Ac, "i8")
    _check_storage("B", B, "i8")
    if beta != 0:
        _check_storage("C", C, "i32")
    else:
        C = None
    meta = np.ascontiguousarray(meta, dtype=np.uint8)
    if points is None:
        ii, jj = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
        ii, jj = ii.reshape(-1), jj.reshape(-1)
    else:
        ii, jj = points
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    d = np.empty(ii.shape, np.int32)
    _load().oracle_gemm_sp24_int_points(int(bool(transb)), k, int(alpha), _ptr(Ac), lda,
                                        meta.ctypes.data, ld_meta, _ptr(B), ldb, int(beta),
                                        _ptr(C), ldc, ii.size, ii.ctypes.data, jj.ctypes.data,
                                        d.ctypes.data)
    return d.reshape(m, n) if points is None else d


def gemm_fp8_mfma(transa: bool, transb: bool, m: int, n: int, k: int, alpha: float,
                  A: np.ndarray, atype: str, lda: int, B: np.ndarray, btype: str, ldb: int,
                  beta: float, C: Optional[np.ndarray], ctype: str, ldc: int, out_fmt: str,
                  points: Optional[tuple] = None, kinst: int = 128, nblk: int = 8,
                  sblk: int = 16, frac: int = 13, wide: int = 24, accw: int = 31) -> np.ndarray:
    """Two-level block model of the FP8 matrix-core accumulation (mpgemm_oracle.c,
    oracle_gemm_fp8_mfma_points): output patterns in ``out_fmt`` storage.  Defaults: gfx950's
    v_mfma_f32_16x16x128_f8f6f4 as measured (groups of 8 products with a 13-bit window; blocks
    of 16 k, in order, each cut to a 24-bit window, or to 31 bits below the accumulator's
    leading bit when that is coarser, added to the FP32 accumulator and rounded to FP32 to
    nearest even; kinst = 128 k per call of the block loop).  accw = 0 drops the
    accumulator's window."""
    _check_storage("A", A, atype)
    _check_storage("B", B, btype)
    if beta != 0.0:
        _check_storage("C", C, ctype)
    else:
        C = None
    if points is None:
        ii, jj = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
        ii, jj = ii.reshape(-1), jj.reshape(-1)
    else:
        ii, jj = points
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    odt = np.uint32 if out_fmt == "f32" else np.uint16
    D = np.empty(ii.shape, odt)
    rc = _load().oracle_gemm_fp8_mfma_points(
        int(bool(transa)), int(bool(transb)), k, float(np.float32(alpha)), _ptr(A), _CODES[atype],
        lda, _ptr(B), _CODES[btype], ldb, float(np.float32(beta)), _ptr(C), _CODES[ctype], ldc,
        _CODES[out_fmt], kinst, nblk, sblk, frac, wide, accw, ii.size, ii.ctypes.data, jj.ctypes.data,
        D.ctypes.data)
    if rc != 0:
        raise ValueError("FP8 block model rejected its arguments")
    if points is None:
        D = D.reshape(m, n)
    return D.view(np.float32) if out_fmt == "f32" else D


def gemm_sp24_fp8_mfma(transb: bool, m: int, n: int, k: int, alpha: float, Ac: np.ndarray,
                       atype: str, lda: int, meta: np.ndarray, ld_meta: int, B: np.ndarray,
                       btype: str, ldb: int, beta: float, C: Optional[np.ndarray], ctype: str,
                       ldc: int, out_fmt: str, points: Optional[tuple] = None, kinst: int = 64,
                       nblk: int = 8, sblk: int = 16, frac: int = 13,
                       wide: int = 24, accw: int = 31) -> np.ndarray:
    """The FP8 block model over a 2:4 sparse A's kept products, in kept order
    (mpgemm_oracle.c, oracle_gemm_sp24_fp8_mfma_points): output patterns in ``out_fmt``."""
    _check_storage("A", Ac, atype)
    _check_storage("B", B, btype)
    if beta != 0.0:
        _check_storage("C", C, ctype)
    else:
        C = None
    meta = np.ascontiguousarray(meta, dtype=np.uint8)
    if points is None:
        ii, jj = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
        ii, jj = ii.reshape(-1), jj.reshape(-1)
    else:
        ii, jj = points
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    odt = np.uint32 if out_fmt == "f32" else np.uint16
    D = np.empty(ii.shape, odt)
    rc = _load().oracle_gemm_sp24_fp8_mfma_points(
        int(bool(transb)), k, float(np.float32(alpha)), _ptr(Ac), _CODES[atype], lda,
        meta.ctypes.data, ld_meta, _ptr(B), _CODES[btype], ldb, float(np.float32(beta)), _ptr(C),
        _CODES[ctype], ldc, _CODES[out_fmt], kinst, nblk, sblk, frac, wide, accw, ii.size,
        ii.ctypes.data, jj.ctypes.data, D.ctypes.data)
    if rc != 0:
        raise ValueError("sparse FP8 block model rejected its arguments")
    if points is None:
        D = D.reshape(m, n)
    return D.view(np.float32) if out_fmt == "f32" else D


# Kept products per block of the sparse matrix cores (v_smfmac 16x16x64 FP16/BF16): eight, i.e.
# sixteen logical k, with the dense window and sum rules -- measured on gfx950.
SP24_BLOCK = 8


def gemm_sp24_mfma(transb: bool, m: int, n: int, k: int, alpha: float, Ac: np.ndarray,
                   atype: str, lda: int, meta: np.ndarray, ld_meta: int, B: np.ndarray, ldb: int,
                   beta: float, C: Optional[np.ndarray], ctype: str, ldc: int, out_fmt: str,
                   points: Optional[tuple] = None, nblk: int = SP24_BLOCK,
                   frac: int = MFMA_FRAC, sum_bits: int = MFMA_SUM_BITS) -> np.ndarray:
    """The block-FMA model applied to the 2:4 sparse GEMM's kept products in kept order
    (mpgemm_oracle.c, oracle_gemm_sp24_mfma_points): output patterns in ``out_fmt``."""
    _check_storage("A", Ac, atype)
    _check_storage("B", B, atype)
    if beta != 0.0:
        _check_storage("C", C, ctype)
    else:
        C = None
    meta = np.ascontiguousarray(meta, dtype=np.uint8)
    if points is None:
        ii, jj = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
        ii, jj = ii.reshape(-1), jj.reshape(-1)
    else:
        ii, jj = points
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    odt = np.uint32 if out_fmt == "f32" else np.uint16
    D = np.empty(ii.shape, odt)
    rc = _load().oracle_gemm_sp24_mfma_points(
        int(bool(transb)), k, float(np.float32(alpha)), _ptr(Ac), _CODES[atype], lda,
        meta.ctypes.data, ld_meta, _ptr(B), ldb, float(np.float32(beta)), _ptr(C), _CODES[ctype],
        ldc, _CODES[out_fmt], int(nblk), int(frac), int(sum_bits), ii.size, ii.ctypes.data,
        jj.ctypes.data, D.ctypes.data)
    if rc != 0:
        raise ValueError(f"sparse block model rejected a={atype} c={ctype} out={out_fmt}")
    if points is None:
        D = D.reshape(m, n)
    return D.view(np.float32) if out_fmt == "f32" else D


def gemm_int(transa: bool, transb: bool, m: int, n: int, k: int, alpha: int,
             A: np.ndarray, lda: int, B: np.ndarray, ldb: int, beta: int,
             C: Optional[np.ndarray], ldc: int, points: Optional[tuple] = None) -> np.ndarray:
    """INT8 x INT8 -> INT32 oracle (exact, wraps modulo 2^32).  Returns int32 values."""
    _check_storage("A", A, "i8")
    _check_storage("B", B, "i8")
    if beta != 0:
        _check_storage("C", C, "i32")
    else:
        C = None
    lib = _load()
    args = (int(bool(transa)), int(bool(transb)), m, n, k, int(alpha), _ptr(A), lda, _ptr(B),
            ldb, int(beta), _ptr(C), ldc)
    if points is None:
        d = np.empty((m, n), np.int32)
        lib.oracle_gemm_int_full(*args, d.ctypes.data)
    else:
        ii = np.ascontiguousarray(points[0], dtype=np.int64)
        jj = np.ascontiguousarray(points[1], dtype=np.int64)
        d = np.empty(ii.shape, np.int32)
        lib.oracle_gemm_int_points(*args, ii.size, ii.ctypes.data, jj.ctypes.data,
                                   d.ctypes.data)
    return d


# ----------------------------------------------------------------------------- comparator
_OUT_ROUNDING = {
    # unit roundoff of the output format and half its smallest subnormal spacing
    "f16": (2.0 ** -11, 2.0 ** -25),
    "bf16": (2.0 ** -8, 2.0 ** -134),
}


def output_to_f64(D: np.ndarray, fmt: str) -> np.ndarray:
    """Widen raw output storage to float64 (exact conversions)."""
    if fmt == "f32":
        return np.asarray(D).view(np.float32).astype(np.float64)
    if fmt == "f16":
        return np.asarray(D).view(np.float16).astype(np.float64)
    if fmt == "bf16":
        return (np.asarray(D).view(np.uint16).astype(np.uint32) << 16).view(
            np.float32).astype(np.float64)
    raise ValueError(fmt)


def _is_pow2_or_zero(x: float) -> bool:
    if x == 0.0:
        return True
    mant, _ = np.frexp(abs(x))
    return mant == 0.5


@dataclass
class CheckReport:
    ok: bool
    n: int
    n_bad: int
    worst_ratio: float          # max |D - v| / bound over finite elements (0 for exact mode)
    first_bad: Optional[int]    # flat index of the first failing element
    detail: str = ""

    def __bool__(self) -> bool:
        return self.ok


def fp_bound(ref: FpReference, k: int, alpha: float, out_fmt: str,
             underflow_floor: bool = False) -> np.ndarray:
    """Per-element acceptance radius around the oracle's v.

    FP32 accumulation (the Tensor Core numerics page, section 2.3, with p = 23):
        E = |alpha| * K * 2^-23 * S + 2^-23 * |beta * c|
    K becomes K + 1 when alpha is not 0 or a power of two (one more rounding in alpha*acc).
    The oracle's own double summation error, (K-1) * 2^-53 * |alpha| * S, is added.
    FP16/BF16 outputs add the final rounding: u * (|v| + E) + eta.
    ``underflow_floor`` adds (K+1) * 2^-126 * max(|alpha|, 1) for directed subnormal-scale
    cases, where flush-to-zero of FP32 intermediates is allowed.
    """
    keff = k if _is_pow2_or_zero(alpha) else k + 1
    a = abs(alpha)
    E = a * keff * 2.0 ** -23 * ref.S + 2.0 ** -23 * np.abs(ref.bc)
    E = E + a * max(k - 1, 0) * 2.0 ** -53 * ref.S
    if underflow_floor:
        E = E + (k + 1) * 2.0 ** -126 * max(a, 1.0)
    if out_fmt in _OUT_ROUNDING:
        u, eta = _OUT_ROUNDING[out_fmt]
        E = E + u * (np.abs(ref.v) + E) + eta
    return E


# FP8 accumulation on gfx950 (v_mfma_f32_16x16x128_f8f6f4, measured): blocks of 16 products,
# 13 fraction bits kept below each group's exponent (so at most 16 truncated terms of less
# than 2^(emax - 13) each, emax <= log2 of the block's largest |a b|), the accumulator cut
# (or dropped, when below half a unit) at the block's 24-bit window, and the sum rounded to
# FP32 after every block of 16 k.
FP8_TRUNCATION = 17.0 * 2.0 ** -13


def fp8_bound(ref: FpReference, k: int, alpha: float, out_fmt: str) -> np.ndarray:
    """Acceptance radius for FP8 inputs: the truncation term FP8_TRUNCATION * S, one FP32
    rounding per block of 16 k (and for alpha when it is not a power of two), beta * c's
    rounding, the oracle's own double error, and the output rounding for 16-bit outputs."""
    steps = max(1, -(-k // 16))
    a = abs(alpha)
    keff = steps if _is_pow2_or_zero(alpha) else steps + 1
    E = a * ref.S * (FP8_TRUNCATION + keff * 2.0 ** -23) + 2.0 ** -23 * np.abs(ref.bc)
    E = E + a * max(k - 1, 0) * 2.0 ** -53 * ref.S
    if out_fmt in _OUT_ROUNDING:
        u, eta = _OUT_ROUNDING[out_fmt]
        E = E + u * (np.abs(ref.v) + E) + eta
    return E


def check_fp(D: np.ndarray, out_fmt: str, ref: FpReference, k: int, alpha: float,
             exact: bool = False, underflow_floor: bool = False,
             fp8: bool = False) -> CheckReport:
    """Accept or reject a floating-point GPU result against the oracle.

    exact=True: bitwise equality with the oracle's once-rounded value (+0 == -0, any NaN ==
    any NaN).  Otherwise: NaN where v is NaN, the same infinity where v is infinite, and
    |D - v| <= bound elsewhere (an output that the oracle rounds to infinity may also be
    that infinity)."""
    Dv = output_to_f64(D, out_fmt).reshape(-1)
    v = ref.v.reshape(-1)
    n = v.size
    ref_rounded = output_to_f64(round_to(v, out_fmt), out_fmt)
    if exact:
        same = (Dv == ref_rounded) | (np.isnan(Dv) & np.isnan(ref_rounded))
        bad = ~same
        worst = 0.0
    else:
        E = (fp8_bound(ref, k, alpha, out_fmt) if fp8
             else fp_bound(ref, k, alpha, out_fmt, underflow_floor)).reshape(-1)
        nan_v = np.isnan(v)
        inf_v = np.isinf(v)
        fin_v = ~(nan_v | inf_v)
        bad = np.zeros(n, dtype=bool)
        bad |= nan_v & ~np.isnan(Dv)
        bad |= inf_v & ~(Dv == v)
        with np.errstate(invalid="ignore", over="ignore"):
            err = np.abs(Dv - v)
            within = np.isfinite(Dv) & (err <= E)
            overflow_ok = np.isinf(ref_rounded) & (Dv == ref_rounded)
            bad |= fin_v & ~(within | overflow_ok)
            ratio = np.where(fin_v & np.isfinite(Dv) & (E > 0), err / np.where(E > 0, E, 1),
                             0.0)
        worst = float(ratio.max()) if n else 0.0
    idx = np.flatnonzero(bad)
    first = int(idx[0]) if idx.size else None
    detail = ""
    if first is not None:
        detail = (f"first bad flat index {first}: D={Dv[first]!r} v={v[first]!r} "
                  f"ref_rounded={ref_rounded[first]!r}")
    return CheckReport(ok=idx.size == 0, n=n, n_bad=int(idx.size), worst_ratio=worst,
                       first_bad=first, detail=detail)


def check_bits(D: np.ndarray, out_fmt: str, ref: np.ndarray) -> CheckReport:
    """Bitwise equality of two floating outputs in ``out_fmt`` storage, except that +0 equals
    -0 and any NaN equals any NaN."""
    d = output_to_f64(D, out_fmt).reshape(-1)
    r = output_to_f64(ref, out_fmt).reshape(-1)
    bad = ~((d == r) | (np.isnan(d) & np.isnan(r)))
    idx = np.flatnonzero(bad)
    first = int(idx[0]) if idx.size else None
    detail = "" if first is None else f"first bad flat index {first}: D={d[first]!r} model={r[first]!r}"
    return CheckReport(ok=idx.size == 0, n=d.size, n_bad=int(idx.size), worst_ratio=0.0,
                       first_bad=first, detail=detail)


def check_int(D: np.ndarray, ref: np.ndarray) -> CheckReport:
    """INT32 outputs must equal the oracle bit for bit."""
    d = np.asarray(D).view(np.int32).reshape(-1)
    r = np.asarray(ref).view(np.int32).reshape(-1)
    bad = d != r
    idx = np.flatnonzero(bad)
    first = int(idx[0]) if idx.size else None
    detail = "" if first is None else f"first bad flat index {first}: D={d[first]} ref={r[first]}"
    return CheckReport(ok=idx.size == 0, n=d.size, n_bad=int(idx.size), worst_ratio=0.0,
                       first_bad=first, detail=detail)
