"""Pins of the oracle's three-product BF16 emulation of an FP32 GEMM (multiword splitting,
"NVIDIA Tensor Core mixed-precision computing: principles and applications", section 5.1).

  * the split x_hi = RN_bf16(x), x_lo = RN_bf16(x - x_hi) against torch's float32 -> bfloat16
    conversion (an independent round-to-nearest-even implementation), on random values,
    ties, subnormals, values near BF16's overflow threshold, Inf and NaN;
  * the split's error bound |x - x_hi - x_lo| <= 2^-16 |x| (two roundings with u = 2^-8);
  * the operand layout: every element of op(A3) and op(B3) checked against its definition
    by index (pieces hi, lo, hi along k for A and hi, hi, lo for B, zero padding to kp);
  * the method's accuracy: on random inputs the block model of the three products lies
    within BF16X3_PRODUCT_ERROR * S + FP32 accumulation of the double FP32 GEMM, and well
    inside what TF32-rounded inputs would give; with BF16-representable inputs x_lo = 0 and
    the result is that of the one-product BF16 GEMM.
"""
import numpy as np
import pytest
import torch

import oracle
from gemm_inputs import Workload, generate


def _torch_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bf16_value(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _special_values():
    rng = np.random.default_rng(8)
    v = [0.0, -0.0, 1.0, -1.0, 1 + 2 ** -8, 1 + 2 ** -8 + 2 ** -16, 1 + 3 * 2 ** -8,
         1 - 2 ** -9, 2 ** -126, 2 ** -127, 2 ** -133, 2 ** -140, 1e-40, -3e-42, 2 ** -149,
         3.3895313892515355e38, 3.3961e38, 3.4028234663852886e38, -3.39e38, np.inf, -np.inf,
         np.nan, 65504.0, 1e30, -7.5e-20]
    v += list(rng.normal(size=2000) * np.exp2(rng.integers(-140, 120, size=2000)))
    v += list(np.float32(rng.uniform(-1, 1, size=500)))
    x = np.array(v, dtype=np.float64).astype(np.float32)
    return x[np.isnan(x) | (np.abs(x) <= np.finfo(np.float32).max)]


def test_split_matches_torch_rounding():
    x = _special_values()
    hi, lo = oracle.split_bf16(x)
    want_hi = _torch_bf16_bits(x)
    nan = np.isnan(x)
    assert np.array_equal(hi[~nan], want_hi[~nan])
    assert np.all(np.isnan(_bf16_value(hi[nan])))
    hv = _bf16_value(hi)
    fin = np.isfinite(hv)
    resid = (x.astype(np.float64) - hv)[fin]                      # exact in double
    assert np.all(resid.astype(np.float32).astype(np.float64) == resid)   # and in FP32
    assert np.array_equal(lo[fin], _torch_bf16_bits(resid.astype(np.float32)))
    assert np.all(lo[~fin] == 0)                                   # Inf, NaN, overflow


def test_split_error_bound():
    x = _special_values()
    x = x[np.isfinite(x) & (np.abs(x) >= 2.0 ** -110) & (np.abs(x) < 3.38e38)]
    hi, lo = oracle.split_bf16(x)
    err = np.abs(x.astype(np.float64) - _bf16_value(hi) - _bf16_value(lo))
    assert np.all(err <= 2.0 ** -16 * np.abs(x.astype(np.float64)))


def test_split_worked_examples():
    # 1 + 2^-8 + 2^-16 lies above the midpoint 1 + 2^-8: x_hi = 1 + 2^-7, and
    # x - x_hi = -(2^-8 - 2^-16) has 8 significant bits: x_lo takes it exactly.
    # 1 + 2^-8 is the midpoint itself: to even, x_hi = 1, x_lo = 2^-8.
    # 3.4e38 rounds past BF16's largest value: x_hi = Inf, x_lo = 0.
    x = np.array([1 + 2 ** -8 + 2 ** -16, 1 + 2 ** -8, 3.4e38], dtype=np.float32)
    hi, lo = oracle.split_bf16(x)
    assert list(_bf16_value(hi)[:2]) == [1 + 2 ** -7, 1.0]
    assert list(_bf16_value(lo)[:2]) == [-(2 ** -8 - 2 ** -16), 2 ** -8]
    assert np.isinf(_bf16_value(hi)[2]) and lo[2] == 0


@pytest.mark.parametrize("transa,transb", [(False, False), (False, True), (True, False), (True, True)])
@pytest.mark.parametrize("m,n,k", [(5, 3, 7), (9, 17, 16), (1, 1, 1), (12, 4, 21)])
def test_operand_layout(transa, transb, m, n, k):
    rng = np.random.default_rng(m * 100 + k)
    opA = rng.normal(size=(m, k)).astype(np.float32)
    opB = rng.normal(size=(k, n)).astype(np.float32)
    lda = m + 4 if transa else k + 4
    ldb = k + 8 if transb else n + 8
    A = np.zeros((k, lda) if transa else (m, lda), np.float32)
    B = np.zeros((n, ldb) if transb else (k, ldb), np.float32)
    if transa:
        A[:, :m] = opA.T
    else:
        A[:, :k] = opA
    if transb:
        B[:, :k] = opB.T
    else:
        B[:, :n] = opB
    A3, lda3, B3, ldb3, k3 = oracle.bf16x3_operands(transa, transb, m, n, k, A, lda, B, ldb)
    kp = (k + 7) // 8 * 8
    assert k3 == 3 * kp
    assert lda3 == ((m + 7) // 8 * 8 if transa else k3)
    assert ldb3 == (k3 if transb else (n + 7) // 8 * 8)
    # pieces element by element from the definition
    def a_at(i, p):
        return int(A3[p, i] if transa else A3[i, p])

    def b_at(p, j):
        return int(B3[j, p] if transb else B3[p, j])

    for i in range(m):
        for p in range(k3):
            piece, q = divmod(p, kp)
            if q >= k:
                assert a_at(i, p) == 0
                continue
            x = opA[i, q]
            h = _torch_bf16_bits(np.array([x]))[0]
            l = _torch_bf16_bits(np.array([x - _bf16_value(np.array([h]))[0]], np.float32))[0]
            assert a_at(i, p) == (l if piece == 1 else h)
    for p in range(k3):
        piece, q = divmod(p, kp)
        for j in range(n):
            if q >= k:
                assert b_at(p, j) == 0
                continue
            x = opB[q, j]
            h = _torch_bf16_bits(np.array([x]))[0]
            l = _torch_bf16_bits(np.array([x - _bf16_value(np.array([h]))[0]], np.float32))[0]
            assert b_at(p, j) == (l if piece == 2 else h)


@pytest.mark.parametrize("k", [40, 333])
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (0.3, -0.7)])
def test_accuracy_against_the_fp32_gemm(k, alpha, beta):
    w = Workload("bf16x3_acc", "f32", "f32", 23, 19, k, alpha=alpha, beta=beta,
                 a_dist="normal(0,1)", b_dist="normal(0,1)", c_dist="normal(0,1)", seed=k)
    inp = generate(w)
    D, _ = oracle.gemm_bf16x3(False, False, w.m, w.n, w.k, alpha, inp.A, w.lda, inp.B, w.ldb,
                              beta, inp.C, w.ldc)
    v, S = oracle.gemm_f32(False, False, w.m, w.n, w.k, alpha, inp.A, w.lda, inp.B, w.ldb, beta,
                           inp.C, w.ldc)
    bc = beta * inp.C[:, : w.n].astype(np.float64) if beta else np.zeros_like(v)
    err = np.abs(D.astype(np.float64) - v)
    bound = oracle.bf16x3_bound(S, w.k, alpha, bc)
    assert np.all(err <= bound)
    # TF32 (10-bit fraction, the handbook's FP32-on-Tensor-Core format) would allow about
    # 2^-10 S; the three products stay far inside it
    assert np.max(err / (S * abs(alpha))) < 2.0 ** -14


def test_bf16_inputs_reduce_to_one_product():
    """Inputs representable in BF16 have x_lo = 0: the three-product result equals the BF16
    GEMM of the inputs (the extra pieces add exact zeros)."""
    w = Workload("bf16x3_exact", "bf16", "f32", 17, 9, 50, a_dist="normal(0,1)",
                 b_dist="normal(0,1)", seed=4)
    inp = generate(w)
    A32 = (inp.A.astype(np.uint32) << 16).view(np.float32)
    B32 = (inp.B.astype(np.uint32) << 16).view(np.float32)
    D, ops = oracle.gemm_bf16x3(False, False, w.m, w.n, w.k, 1.0, A32, w.lda, B32, w.ldb, 0.0,
                                None, w.ldc)
    one = oracle.gemm_mfma(False, False, w.m, w.n, w.k, 1.0, inp.A, "bf16", w.lda, inp.B, "bf16",
                           w.ldb, 0.0, None, "f32", w.ldc, "f32")
    assert np.array_equal(D.view(np.uint32), one.view(np.uint32))
