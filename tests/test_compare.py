"""Sensitivity of the comparator: correct FP32 accumulations in several orders pass; results
with a plausible mistake (a dropped term, FP16 accumulation, a transposed or sign-flipped
operand, a skipped beta*C) fail.  CPU only."""
import numpy as np
import pytest

import oracle
from gemm_inputs import Workload, generate, WORKLOADS


def _decoded(inp):
    """op(A), op(B), C as float64 from raw storage (numpy conversions, exact)."""
    w = inp.w
    if w.transa:
        a = oracle.output_to_f64(np.ascontiguousarray(inp.A[:, :w.m]), w.in_type).T
    else:
        a = oracle.output_to_f64(np.ascontiguousarray(inp.A[:, :w.k]), w.in_type)
    if w.transb:
        b = oracle.output_to_f64(np.ascontiguousarray(inp.B[:, :w.k]), w.in_type).T
    else:
        b = oracle.output_to_f64(np.ascontiguousarray(inp.B[:, :w.n]), w.in_type)
    c = None if inp.C is None else oracle.output_to_f64(np.ascontiguousarray(inp.C[:, :w.n]), w.out_type)
    return a, b, c


def _f32_accumulate(a, b, order):
    """FP32 accumulation of exact products in a given order; returns float32 m x n."""
    prods = a[:, :, None] * b[None, :, :]            # m x k x n, exact in double
    m, k, n = prods.shape
    if order == "forward":
        idx = range(k)
    elif order == "reverse":
        idx = range(k - 1, -1, -1)
    if order in ("forward", "reverse"):
        acc = np.zeros((m, n), np.float32)
        for p in idx:
            acc = (acc + prods[:, p, :].astype(np.float32)).astype(np.float32)
        return acc
    if order == "pairwise":
        parts = [prods[:, p, :].astype(np.float32) for p in range(k)]
        while len(parts) > 1:
            nxt = [(parts[t] + parts[t + 1]).astype(np.float32) for t in range(0, len(parts) - 1, 2)]
            if len(parts) % 2:
                nxt.append(parts[-1])
            parts = nxt
        return parts[0]
    if order == "block16_truncate":
        # exact 16-term block sums added into an FP32 accumulator that truncates toward zero
        acc = np.zeros((m, n), np.float64)
        for p0 in range(0, k, 16):
            s = acc + prods[:, p0:p0 + 16, :].sum(axis=1)
            r = s.astype(np.float32).astype(np.float64)
            too_far = np.abs(r) > np.abs(s)
            r = np.where(too_far, np.nextafter(r.astype(np.float32), np.float32(0)).astype(np.float64), r)
            acc = r
        return acc.astype(np.float32)
    if order == "fp16":
        acc = np.zeros((m, n), np.float16)
        for p in range(k):
            acc = (acc + prods[:, p, :].astype(np.float16)).astype(np.float16)
        return acc.astype(np.float32)
    raise ValueError(order)


@pytest.fixture(scope="module")
def problem():
    w = Workload("cmp", "f16", "f32", 24, 20, 512, transb=True, alpha=1.0, beta=0.5,
                 a_dist="normal(0,1)", b_dist="normal(0,1)", c_dist="normal(0,1)", seed=21)
    inp = generate(w)
    ref = oracle.gemm_fp(w.transa, w.transb, w.m, w.n, w.k, w.alpha, inp.A, "f16", w.lda, inp.B,
                         "f16", w.ldb, w.beta, inp.C, "f32", w.ldc)
    a, b, c = _decoded(inp)
    return w, inp, ref, a, b, c


def _epilogue(acc, w, c):
    out = (np.float32(w.alpha) * acc).astype(np.float32)
    if w.beta:
        out = (out + (np.float32(w.beta) * c.astype(np.float32)).astype(np.float32)).astype(np.float32)
    return out


@pytest.mark.parametrize("order", ["forward", "reverse", "pairwise", "block16_truncate"])
def test_correct_fp32_orders_pass(problem, order):
    w, inp, ref, a, b, c = problem
    D = _epilogue(_f32_accumulate(a, b, order), w, c)
    rep = oracle.check_fp(D, "f32", ref, w.k, w.alpha)
    assert rep.ok, rep.detail
    assert rep.worst_ratio < 0.5


def test_fp16_accumulation_fails(problem):
    w, inp, ref, a, b, c = problem
    D = _epilogue(_f32_accumulate(a, b, "fp16"), w, c)
    assert not oracle.check_fp(D, "f32", ref, w.k, w.alpha).ok


def test_dropped_term_fails(problem):
    w, inp, ref, a, b, c = problem
    for drop in (0, w.k // 2, w.k - 1):
        keep = [p for p in range(w.k) if p != drop]
        D = _epilogue(_f32_accumulate(a[:, keep], b[keep, :], "forward"), w, c)
        assert not oracle.check_fp(D, "f32", ref, w.k, w.alpha).ok


def test_wrong_operand_fails(problem):
    w, inp, ref, a, b, c = problem
    D = _epilogue(_f32_accumulate(-a, b, "forward"), w, c)                  # sign
    assert not oracle.check_fp(D, "f32", ref, w.k, w.alpha).ok
    D = _epilogue(_f32_accumulate(a, b[::-1, :], "forward"), w, c)          # k reversed in B only
    assert not oracle.check_fp(D, "f32", ref, w.k, w.alpha).ok
    D = _epilogue(_f32_accumulate(a, b, "forward"), w, np.zeros_like(c))    # beta*C skipped
    assert not oracle.check_fp(D, "f32", ref, w.k, w.alpha).ok
    D = _epilogue(_f32_accumulate(a, b, "forward"), w, c)
    E = oracle.fp_bound(ref, w.k, w.alpha, "f32")
    D[3, 4] = np.float32(ref.v[3, 4] + 1.5 * E[3, 4])                      # one element off
    assert not oracle.check_fp(D, "f32", ref, w.k, w.alpha).ok


def test_square_transpose_fails():
    w = Workload("cmp_sq", "bf16", "f32", 16, 16, 64, a_dist="normal(0,1)", b_dist="normal(0,1)",
                 seed=22)
    inp = generate(w)
    ref = oracle.gemm_fp(False, False, 16, 16, 64, 1.0, inp.A, "bf16", 64, inp.B, "bf16", 16, 0.0,
                         None, "f32", 16)
    a, b, _ = _decoded(inp)
    good = _f32_accumulate(a, b, "forward")
    assert oracle.check_fp(good, "f32", ref, 64, 1.0).ok
    assert not oracle.check_fp(np.ascontiguousarray(good.T), "f32", ref, 64, 1.0).ok


def test_half_output_bound_and_exact_mode():
    w = Workload("cmp_h", "f16", "f16", 8, 8, 2049, a_dist="ones", b_dist="ones", seed=23)
    inp = generate(w)
    ref = oracle.gemm_fp(False, False, 8, 8, 2049, 1.0, inp.A, "f16", w.lda, inp.B, "f16", w.ldb,
                         0.0, None, "f16", w.ldc)
    exact = oracle.round_to(ref.v, "f16")
    assert oracle.check_fp(exact, "f16", ref, w.k, 1.0, exact=True).ok
    wrong = exact.copy()
    wrong[0, 0] += 1                                       # 2050 instead of 2048
    assert not oracle.check_fp(wrong, "f16", ref, w.k, 1.0, exact=True).ok



def test_beta_c_rounded_to_fp32_passes():
    """beta * c rounded to FP32 before the add: with products near 2^-21 beside |beta c| near
    0.1, that rounding is the error, and the bound's 2^-23 |beta c| term must admit it."""
    w = Workload("cmp_bc", "f16", "f32", 16, 16, 1, beta=float(np.float32(0.1)),
                 a_dist="log_uniform(-12,-10)", b_dist="log_uniform(-12,-10)",
                 c_dist="normal(0,1)", seed=24)
    inp = generate(w)
    ref = oracle.gemm_fp(False, False, w.m, w.n, w.k, w.alpha, inp.A, "f16", w.lda, inp.B, "f16",
                         w.ldb, w.beta, inp.C, "f32", w.ldc)
    a, b, c = _decoded(inp)
    D = _epilogue(_f32_accumulate(a, b, "forward"), w, c)
    assert not np.array_equal(D.astype(np.float64), ref.v)   # the rounding is there to admit
    rep = oracle.check_fp(D, "f32", ref, w.k, w.alpha)
    assert rep.ok, rep.detail


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_16bit_outputs_rounded_once_pass(fmt):
    """An FP32 accumulation rounded once to FP16 or BF16 output passes the bound check (the
    output rounding, 2^-11 or 2^-8 of |v|, dwarfs the short sum's K 2^-23 S)."""
    w = Workload(f"cmp_o_{fmt}", fmt, fmt, 16, 16, 4, a_dist="normal(0,1)", b_dist="normal(0,1)",
                 seed=25)
    inp = generate(w)
    ref = oracle.gemm_fp(False, False, w.m, w.n, w.k, 1.0, inp.A, fmt, w.lda, inp.B, fmt, w.ldb,
                         0.0, None, fmt, w.ldc)
    a, b, _ = _decoded(inp)
    D = oracle.round_to(_f32_accumulate(a, b, "forward").astype(np.float64), fmt)
    rep = oracle.check_fp(D, fmt, ref, w.k, 1.0)
    assert rep.ok, rep.detail
    assert rep.worst_ratio > 0.01                  # the output rounding carries real weight


def test_exact_mode_takes_nan_as_equal_to_nan():
    ref = oracle.FpReference(v=np.array([np.nan, 1.0]), S=np.ones(2), bc=np.zeros(2))
    assert oracle.check_fp(np.array([np.nan, 1.0], np.float32), "f32", ref, 1, 1.0, exact=True).ok
    assert not oracle.check_fp(np.array([1.0, 1.0], np.float32), "f32", ref, 1, 1.0, exact=True).ok


def test_nonfinite_rules():
    ref = oracle.FpReference(v=np.array([np.nan, np.inf, -np.inf, 1.0]), S=np.array([1.0] * 4),
                             bc=np.zeros(4))
    good = np.array([np.nan, np.inf, -np.inf, 1.0], np.float32)
    assert oracle.check_fp(good, "f32", ref, 1, 1.0).ok
    for bad in ([1.0, np.inf, -np.inf, 1.0], [np.nan, -np.inf, -np.inf, 1.0],
                [np.nan, np.inf, -np.inf, np.nan]):
        assert not oracle.check_fp(np.array(bad, np.float32), "f32", ref, 1, 1.0).ok


def test_int_check():
    r = np.array([1, -2, 3], np.int32)
    assert oracle.check_int(r.copy(), r).ok
    assert not oracle.check_int(np.array([1, -2, 4], np.int32), r).ok


def test_workload_table_matches_recipe():
    w = WORKLOADS["f16_4096_nt"]
    assert (w.m, w.n, w.k, w.transa, w.transb, w.beta) == (4096, 4096, 4096, False, True, 0.0)
    w = WORKLOADS["f16_5000x3000x1000_f16out_padded"]
    assert (w.lda, w.ldb, w.ldc) == (1008, 3008, 3008)
