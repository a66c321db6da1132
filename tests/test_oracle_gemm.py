"""Pins for the oracle's GEMM: closed forms, exact brute force with rationals, the worked
vectors printed on the Tensor Core numerics page, the DP4A definition, the INT8 product
table, epilogue special cases and NaN/Inf propagation.  CPU only."""
import ast
import operator
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from gemm_inputs import f64_to_bf16_bits, f64_to_f16_bits, place, stored_shape

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]


def to_bits(x, fmt):
    return f64_to_f16_bits(x) if fmt == "f16" else f64_to_bf16_bits(x)


def make_operand(vals_op, trans, fmt, pad=0):
    """Stored buffer for op(X) = vals_op (logical rows x cols), optionally padded."""
    stored = vals_op.T if trans else vals_op
    stored = np.ascontiguousarray(stored)
    ld = stored.shape[1] + pad
    if fmt == "i8":
        return place(stored.astype(np.int8), ld, "i8"), ld
    return place(to_bits(stored, fmt), ld, fmt), ld


def run_fp(a_op, b_op, fmt, ta, tb, alpha=1.0, beta=0.0, c=None, cfmt="f32", pad=0):
    m, k = a_op.shape
    n = b_op.shape[1]
    A, lda = make_operand(a_op, ta, fmt, pad)
    B, ldb = make_operand(b_op, tb, fmt, pad)
    C, ldc = None, n
    if c is not None:
        if cfmt == "f32":
            C = place(c.astype(np.float32), n + pad, "f32")
        else:
            C = place(to_bits(c, cfmt), n + pad, cfmt)
        ldc = n + pad
    return oracle.gemm_fp(ta, tb, m, n, k, alpha, A, fmt, lda, B, fmt, ldb, beta, C, cfmt, ldc)


# ----------------------------------------------------------------------------- closed forms
@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_identity_gives_other_operand(ta, tb, fmt):
    rng = np.random.default_rng(1)
    n = 9
    b = rng.uniform(-3, 3, (7, n))
    b = oracle_exact_values(b, fmt)
    r = run_fp(np.eye(7), b, fmt, ta, tb, pad=3)
    assert np.array_equal(r.v, b)
    a = oracle_exact_values(rng.uniform(-3, 3, (5, 7)), fmt)
    r = run_fp(a, np.eye(7), fmt, ta, tb, pad=1)
    assert np.array_equal(r.v, a)


def oracle_exact_values(x, fmt):
    """The values that ``x`` takes after rounding to ``fmt`` (widened with numpy/torch-free
    bit arithmetic through the oracle's decoder)."""
    bits = to_bits(x, fmt)
    return np.array([oracle.decode(int(b), fmt) for b in bits.ravel()]).reshape(x.shape)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_permutation_permutes_rows(ta, tb):
    rng = np.random.default_rng(2)
    perm = rng.permutation(8)
    P = np.eye(8)[perm]
    b = oracle_exact_values(rng.uniform(-1, 1, (8, 5)), "f16")
    r = run_fp(P, b, "f16", ta, tb)
    assert np.array_equal(r.v, b[perm])
    r = run_fp(b.T.copy(), P.T.copy(), "f16", ta, tb)       # columns permuted
    assert np.array_equal(r.v, b.T[:, perm])


@pytest.mark.parametrize("k", [1, 3, 1000, 4096])
def test_all_ones_gives_k(k):
    r = run_fp(np.ones((3, k)), np.ones((k, 4)), "f16", False, True)
    assert np.all(r.v == k) and np.all(r.S == k)


def test_rank_one_outer_product():
    rng = np.random.default_rng(4)
    a = oracle_exact_values(rng.uniform(-2, 2, (6, 1)), "bf16")
    b = oracle_exact_values(rng.uniform(-2, 2, (1, 5)), "bf16")
    for ta, tb in LAYOUTS:
        r = run_fp(a, b, "bf16", ta, tb)
        assert np.array_equal(r.v, a[:, 0][:, None] * b[0][None, :])


# ----------------------------------------------------------------------------- brute force
def _frac_matrix(vals):
    return [[Fraction(float(x)) for x in row] for row in vals]


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 3, 4), (5, 4, 6), (6, 6, 3), (3, 5, 0)])
def test_brute_force_exact_dyadic(ta, tb, fmt, shape):
    """Dyadic inputs (multiples of 1/8, |x| <= 4): every partial sum is exact in double, so
    v must equal the rational value exactly, in every layout, with alpha/beta epilogue."""
    m, n, k = shape
    rng = np.random.default_rng(100 + m * 31 + n * 7 + k)
    a = rng.integers(-32, 33, (m, k)) / 8.0
    b = rng.integers(-32, 33, (k, n)) / 8.0
    c = rng.integers(-32, 33, (m, n)) / 4.0
    for alpha, beta in [(1.0, 0.0), (0.5, 2.0), (-3.0, 1.0)]:
        r = run_fp(a, b, fmt, ta, tb, alpha=alpha, beta=beta, c=c, pad=2)
        A, B, C = _frac_matrix(a), _frac_matrix(b), _frac_matrix(c)
        for i in range(m):
            for j in range(n):
                s = sum((A[i][p] * B[p][j] for p in range(k)), Fraction(0))
                sa = sum((abs(A[i][p] * B[p][j]) for p in range(k)), Fraction(0))
                want = Fraction(alpha) * s + (Fraction(beta) * C[i][j] if beta else 0)
                assert Fraction(r.v[i, j]) == want
                assert Fraction(r.S[i, j]) == sa


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_brute_force_random_within_double_error(ta, tb):
    """General FP16 inputs: v is within (k-1) 2^-53 S of the exact rational sum."""
    rng = np.random.default_rng(5)
    m, n, k = 4, 5, 6
    a = oracle_exact_values(rng.normal(0, 1, (m, k)), "f16")
    b = oracle_exact_values(rng.normal(0, 1, (k, n)), "f16")
    r = run_fp(a, b, "f16", ta, tb)
    for i in range(m):
        for j in range(n):
            s = sum(Fraction(float(a[i, p])) * Fraction(float(b[p, j])) for p in range(k))
            assert abs(Fraction(r.v[i, j]) - s) <= Fraction((k - 1) * 2.0 ** -53) * Fraction(r.S[i, j])


def test_matches_float64_matmul_on_dyadic_inputs():
    """Special case reducing to a library routine: integer-valued inputs, so numpy's float64
    matmul is exact and must agree bit for bit."""
    rng = np.random.default_rng(6)
    m, n, k = 37, 29, 70
    a = rng.integers(-8, 9, (m, k)).astype(np.float64)
    b = rng.integers(-8, 9, (k, n)).astype(np.float64)
    for ta, tb in LAYOUTS:
        for fmt in ("f16", "bf16"):
            r = run_fp(a, b, fmt, ta, tb)
            assert np.array_equal(r.v, a @ b)


def test_points_agree_with_full():
    rng = np.random.default_rng(8)
    m, n, k = 20, 30, 40
    a = rng.normal(0, 1, (m, k))
    b = rng.normal(0, 1, (k, n))
    c = rng.normal(0, 1, (m, n))
    A, lda = make_operand(a, False, "f16")
    B, ldb = make_operand(b, True, "f16")
    C = c.astype(np.float32)
    full = oracle.gemm_fp(False, True, m, n, k, 1.0, A, "f16", lda, B, "f16", ldb, 0.5, C, "f32", n)
    ii = rng.integers(0, m, 50)
    jj = rng.integers(0, n, 50)
    pts = oracle.gemm_fp(False, True, m, n, k, 1.0, A, "f16", lda, B, "f16", ldb, 0.5, C, "f32", n,
                         points=(ii, jj))
    assert np.array_equal(pts.v, full.v[ii, jj])
    assert np.array_equal(pts.S, full.S[ii, jj])
    assert np.array_equal(pts.bc, full.bc[ii, jj])


# ----------------------------------------------------------------------------- page vectors
_OPS = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul,
        ast.Pow: operator.pow}


def _eval_exact(expr):
    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.Constant):
            return Fraction(str(node.value))
        if isinstance(node, ast.UnaryOp) and isinstance(node.op, ast.USub):
            return -ev(node.operand)
        if isinstance(node, ast.BinOp) and type(node.op) in _OPS:
            left, right = ev(node.left), ev(node.right)
            if isinstance(node.op, ast.Pow):
                return left ** int(right)
            return _OPS[type(node.op)](left, right)
        raise ValueError(expr)
    return ev(ast.parse(expr.strip(), mode="eval"))


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([p.strip() for p in line.split(";")])
    return rows


@pytest.mark.parametrize("row", _golden_rows("tc_numerics_vectors.txt"),
                         ids=lambda r: f"{r[0]}-{r[1]}")
def test_tensor_core_numerics_page_vectors(row):
    name, fmt, a_s, b_s, c_s, exact_s, bits_s = row
    a = [_eval_exact(x) for x in a_s.split(",")]
    b = [_eval_exact(x) for x in b_s.split(",")]
    exact = _eval_exact(exact_s)
    k = len(a)
    av = np.array([[float(x) for x in a]])
    bv = np.array([[float(x)] for x in b])
    assert [Fraction(float(x)) for x in a] == a          # inputs representable as given
    A, lda = make_operand(av, False, fmt)
    B, ldb = make_operand(bv, False, fmt)
    for t in range(k):                                     # and in the input format
        assert Fraction(oracle.decode(int(A[0, t]), fmt)) == a[t]
        assert Fraction(oracle.decode(int(B[t, 0]), fmt)) == b[t]
    r = oracle.gemm_fp(False, False, 1, 1, k, 1.0, A, fmt, lda, B, fmt, ldb, float(_eval_exact(c_s)),
                       None, "f32", 1)
    assert Fraction(r.v[0, 0]) == exact                    # the sum is exact in double
    got = oracle.round_to(r.v, "f32").view(np.uint32)[0, 0]
    assert int(got) == int(bits_s, 16)


# ----------------------------------------------------------------------------- INT8
def _dp4a(a_word, b_word, c):
    """DP4A as defined on the CUDA 8 mixed-precision page (section on low-precision
    integers, Figure 2): four signed bytes packed in each 32-bit word, multiplied pairwise,
    summed and added to the 32-bit c."""
    tot = c
    for t in range(4):
        x = (a_word >> (8 * t)) & 0xFF
        y = (b_word >> (8 * t)) & 0xFF
        x = x - 256 if x >= 128 else x
        y = y - 256 if y >= 128 else y
        tot += x * y
    return tot


def test_int8_k4_is_one_dp4a():
    rng = np.random.default_rng(9)
    for _ in range(200):
        a = rng.integers(-128, 128, 4).astype(np.int8)
        b = rng.integers(-128, 128, 4).astype(np.int8)
        c = int(rng.integers(-2 ** 31, 2 ** 31))
        a_word = int(a.view(np.uint8).astype(np.uint32) @ (256 ** np.arange(4, dtype=np.uint32)))
        b_word = int(b.view(np.uint8).astype(np.uint32) @ (256 ** np.arange(4, dtype=np.uint32)))
        want = _dp4a(a_word, b_word, c)
        want = (want + 2 ** 31) % 2 ** 32 - 2 ** 31
        d = oracle.gemm_int(False, False, 1, 1, 4, 1, a.reshape(1, 4), 4, b.reshape(4, 1), 1, 1,
                            np.array([[c]], np.int32), 1)
        assert int(d[0, 0]) == want


def test_int8_exhaustive_product_table():
    vals = np.arange(-128, 128, dtype=np.int8)
    A = vals.reshape(256, 1).copy()
    B = vals.reshape(1, 256).copy()
    d = oracle.gemm_int(False, False, 256, 256, 1, 1, A, 1, B, 256, 0, None, 256)
    assert np.array_equal(d, np.outer(vals.astype(np.int64), vals.astype(np.int64)))


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_int8_brute_force_with_wrap(ta, tb):
    rng = np.random.default_rng(10)
    m, n, k = 5, 7, 33
    a = rng.integers(-128, 128, (m, k))
    b = rng.integers(-128, 128, (k, n))
    c = rng.integers(-2 ** 31, 2 ** 31, (m, n))
    A, lda = make_operand(a, ta, "i8", pad=16)
    B, ldb = make_operand(b, tb, "i8", pad=3)
    C = c.astype(np.int32)
    for alpha, beta in [(1, 0), (1, 1), (3, -2), (2 ** 20, 7)]:
        d = oracle.gemm_int(ta, tb, m, n, k, alpha, A, lda, B, ldb, beta,
                            C if beta else None, n)
        for i in range(m):
            for j in range(n):
                s = sum(int(a[i, p]) * int(b[p, j]) for p in range(k))
                want = alpha * s + (beta * int(c[i, j]) if beta else 0)
                want = (want + 2 ** 31) % 2 ** 32 - 2 ** 31
                assert int(d[i, j]) == want


def test_int8_extremes():
    k = 4096
    A = np.full((2, k), -128, np.int8)
    B = np.full((k, 2), -128, np.int8)
    B[:, 1] = 127
    d = oracle.gemm_int(False, False, 2, 2, k, 1, A, k, B, 2, 0, None, 2)
    assert np.all(d[:, 0] == 16384 * k) and np.all(d[:, 1] == -16256 * k)


# ----------------------------------------------------------------------------- epilogue
def test_k_zero_gives_beta_c():
    c = np.array([[1.5, -2.0], [0.25, 8.0]])
    r = run_fp(np.zeros((2, 0)), np.zeros((0, 2)), "f16", False, False, alpha=1.0, beta=0.5, c=c)
    assert np.array_equal(r.v, 0.5 * c)
    r = run_fp(np.zeros((2, 0)), np.zeros((0, 2)), "f16", False, False, alpha=1.0, beta=0.0)
    assert np.array_equal(r.v, np.zeros((2, 2)))


def test_beta_zero_never_reads_c():
    a = np.ones((2, 3))
    b = np.ones((3, 2))
    A, lda = make_operand(a, False, "f16")
    B, ldb = make_operand(b, False, "f16")
    C = np.full((2, 2), np.nan, np.float32)
    r = oracle.gemm_fp(False, False, 2, 2, 3, 1.0, A, "f16", lda, B, "f16", ldb, 0.0, C, "f32", 2)
    assert np.all(r.v == 3.0)


def test_nan_and_inf_propagation():
    a = np.array([[np.nan, 1.0], [np.inf, 1.0], [np.inf, 1.0], [1.0, 1.0]])
    b = np.array([[1.0, 0.0], [1.0, 1.0]])
    A, lda = make_operand(a, False, "f16")
    A[2, 1] = 0xFC00                                        # -inf
    B, ldb = make_operand(b, False, "f16")
    r = oracle.gemm_fp(False, False, 4, 2, 2, 1.0, A, "f16", lda, B, "f16", ldb, 0.0, None, "f32", 2)
    assert np.isnan(r.v[0, 0]) and np.isnan(r.v[0, 1])      # NaN spreads along its row
    assert r.v[1, 0] == np.inf                              # inf * 1 + 1
    assert np.isnan(r.v[1, 1])                              # inf * 0
    assert np.isnan(r.v[2, 0])                              # inf - inf
    assert r.v[3, 0] == 2.0
    # alpha = 0 does not short-circuit: NaN still propagates
    r0 = oracle.gemm_fp(False, False, 4, 2, 2, 0.0, A, "f16", lda, B, "f16", ldb, 0.0, None, "f32", 2)
    assert np.isnan(r0.v[0, 0]) and r0.v[3, 0] == 0.0


def test_half_output_rounding_ties():
    """All-ones with K = 2049 and 2051: FP16 output must round the exact K to even."""
    for k, want in [(2049, 2048.0), (2051, 2052.0)]:
        r = run_fp(np.ones((1, k)), np.ones((k, 1)), "f16", False, False)
        assert oracle.decode(int(oracle.round_to(r.v, "f16")[0, 0]), "f16") == want


def test_thread_count_does_not_change_results():
    """The oracle's thread count (set to 1 for the single-thread timing of the smallest
    configuration) changes only the schedule: each output's sum is computed by one thread in
    the same order, so results are identical."""
    rng = np.random.default_rng(11)
    a = rng.integers(-3, 4, size=(70, 90)).astype(np.float64) * 0.37
    b = rng.integers(-3, 4, size=(90, 50)).astype(np.float64) * 1.3
    threads = oracle.num_threads()
    try:
        oracle.set_num_threads(1)
        assert oracle.num_threads() == 1
        r1 = run_fp(a, b, "f16", False, False)
    finally:
        oracle.set_num_threads(threads)
    assert oracle.num_threads() == threads
    rn = run_fp(a, b, "f16", False, False)
    assert np.array_equal(r1.v, rn.v) and np.array_equal(r1.S, rn.S)
