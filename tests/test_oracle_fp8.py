"""Pins of the oracle's FP8 arithmetic (E4M3 / E5M2, "NVIDIA Tensor Core mixed-precision
computing: principles and applications", section 4.3.1; fields read as the OCP definitions).

  * both decoders, all 256 patterns each, against torch's float8_e4m3fn / float8_e5m2
    (an independent implementation of the same formats);
  * the FP8 GEMM against exact rational brute force on tiny mixed-format shapes (every
    layout), and against integer matrix products on integer-valued inputs;
  * the acceptance radius covers the truncation the accumulation structure allows.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from gemm_inputs import Workload, f64_to_fp8_bits, generate


@pytest.mark.parametrize("fmt,tdt", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_decoders_match_torch(fmt, tdt):
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(tdt).to(torch.float64).numpy()
    got = np.array([oracle.decode(int(c), fmt) for c in codes])
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all(), codes[~same]
    assert oracle.decode(0x7E, "e4m3") == 448.0 and oracle.decode(0x7B, "e5m2") == 57344.0
    assert oracle.decode(0x01, "e4m3") == 2.0 ** -9 and oracle.decode(0x01, "e5m2") == 2.0 ** -16


@pytest.mark.parametrize("fmt,tdt", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_input_rounding_matches_torch(fmt, tdt):
    rng = np.random.default_rng(3)
    mx = 448.0 if fmt == "e4m3" else 57344.0
    x = np.clip((rng.normal(size=50000) * np.exp2(rng.integers(-20, 16, size=50000))).astype(np.float32),
                -mx, mx)
    vals = torch.arange(0, 127, dtype=torch.uint8).view(tdt).to(torch.float64).numpy()
    v = vals[np.isfinite(vals)]
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)               # exact ties
    x = np.concatenate([x, mids, -mids])
    want = torch.from_numpy(x).to(tdt).view(torch.uint8).numpy()
    assert np.array_equal(f64_to_fp8_bits(x.astype(np.float64), fmt), want)


@pytest.mark.parametrize("transa,transb", [(False, False), (False, True), (True, False), (True, True)])
@pytest.mark.parametrize("a_t,b_t", [("e4m3", "e5m2"), ("e5m2", "e4m3")])
def test_gemm_fp8_brute_force(transa, transb, a_t, b_t):
    w = Workload("fp8_bf", a_t, "f32", 3, 4, 5, b_type=b_t, transa=transa, transb=transb,
                 alpha=1.5, beta=-0.5, a_dist="normal(0,2)", b_dist="normal(0,2)",
                 c_dist="normal(0,1)", seed=17)
    inp = generate(w)
    ref = oracle.gemm_fp8(transa, transb, w.m, w.n, w.k, w.alpha, inp.A, a_t, w.lda, inp.B, b_t,
                          w.ldb, w.beta, inp.C, "f32", w.ldc)
    def a(i, p):
        return Fraction(oracle.decode(int(inp.A[p, i] if transa else inp.A[i, p]), a_t))

    def b(p, j):
        return Fraction(oracle.decode(int(inp.B[j, p] if transb else inp.B[p, j]), b_t))
    for i in range(w.m):
        for j in range(w.n):
            s = sum(a(i, p) * b(p, j) for p in range(w.k))
            exact = Fraction(w.alpha) * s + Fraction(w.beta) * Fraction(float(inp.C[i, j]))
            assert ref.v[i, j] == float(exact)
            assert ref.S[i, j] == float(sum(abs(a(i, p) * b(p, j)) for p in range(w.k)))


def test_gemm_fp8_integer_inputs():
    w = Workload("fp8_int", "e4m3", "f32", 20, 30, 300, b_type="e5m2", a_dist="int_uniform(-4,4)",
                 b_dist="int_uniform(-4,4)", seed=2)
    inp = generate(w)
    A = np.array([[oracle.decode(int(c), "e4m3") for c in row] for row in inp.A[:, : w.k]])
    B = np.array([[oracle.decode(int(c), "e5m2") for c in row] for row in inp.B[:, : w.n]])
    assert np.all(A == np.round(A)) and np.all(np.abs(A) <= 4)
    ref = oracle.gemm_fp8(False, False, w.m, w.n, w.k, 1.0, inp.A, "e4m3", w.lda, inp.B, "e5m2",
                          w.ldb, 0.0, None, "f32", w.ldc)
    assert np.array_equal(ref.v, (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float64))


def test_fp8_bound_covers_block_truncation():
    """A worst case of the measured structure: per 16-product block, a product at the block's
    exponent plus 15 products just under 2^(emax - 13), all cut away: the radius holds it."""
    S = np.array([[1.0 + 15 * 2.0 ** -13]])
    ref = oracle.FpReference(v=np.array([[1.0]]), S=S, bc=np.zeros((1, 1)))
    E = oracle.fp8_bound(ref, 16, 1.0, "f32")
    assert E[0, 0] >= 15 * 2.0 ** -13
