"""Pins of the oracle's 2:4 structured-sparse GEMM (sparse tensor cores on the page
"稀疏张量核心加速模板计算的技术解析",
sections 1.2.1 and 1.3.2: at most two nonzeros in every group of four consecutive k, held as
the kept values plus a 2-bit position each).

  * the metadata packing against hand-worked bytes (position j of a row in bits 2 (j % 4) of
    byte j / 4, little-endian order);
  * the generator: every group of four keeps two distinct positions, all six pairs occur about
    equally often, padding bytes are 0xFF;
  * the sparse reference against the dense reference of the decompressed A (each kept value
    placed at column 4 q + idx), which is an independent code path: equal bit for bit when
    the positions increase, since the nonzero products are then summed in the same order;
  * brute force with exact rational sums on tiny inputs, including repeated and decreasing
    positions, which the definition allows;
  * the sparse block model with blocks of four kept products equals the dense block model
    (blocks of eight k) of the decompressed A: a dense block of eight k holds exactly the four
    kept products of its two groups, and zero products take no part in a block.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from gemm_inputs import SP24_PAIRS, Workload, generate, pack_sp24_meta


def _unpack(meta, m, k):
    kh = k // 2
    j = np.arange(kh)
    return (meta[:, j // 4] >> (2 * (j % 4))) & 3


def _decompress(inp):
    """Dense m x k A (storage format, padded with zeros to lda = k) from the kept values."""
    w = inp.w
    idx = _unpack(inp.meta, w.m, w.k)
    A = np.zeros((w.m, w.k), np.uint16)
    j = np.arange(w.k // 2)
    cols = 4 * (j // 2) + idx
    rows = np.repeat(np.arange(w.m)[:, None], w.k // 2, axis=1)
    A[rows, cols] = inp.A[:, : w.k // 2]
    return A


def _value16(bits, t):
    bits = np.asarray(bits)
    if t == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


def test_meta_packing_worked_example():
    # positions (0,1) (2,3) (1,3) (0,2) | (0,3) (1,2) (2,3) (0,1)
    idx = np.array([[0, 1, 2, 3, 1, 3, 0, 2, 0, 3, 1, 2, 2, 3, 0, 1]], np.uint8)
    meta = pack_sp24_meta(idx, 16)
    # byte 0: 0 | 1 << 2 | 2 << 4 | 3 << 6 = 0xE4;  byte 1: 1 | 3 << 2 | 0 << 4 | 2 << 6 = 0x8D
    # byte 2: 0 | 3 << 2 | 1 << 4 | 2 << 6 = 0x9C;  byte 3: 2 | 3 << 2 | 0 << 4 | 1 << 6 = 0x4E
    assert list(meta[0, :4]) == [0xE4, 0x8D, 0x9C, 0x4E]
    assert np.all(meta[0, 4:] == 0xFF)


@pytest.mark.parametrize("k", [128, 384])
def test_generator_structure(k):
    w = Workload("sp_gen", "f16", "f32", 300, 8, k, sparse24=True, a_dist="normal(0,1)", seed=k)
    inp = generate(w)
    assert inp.A.shape == (w.m, w.lda) and w.lda >= k // 2
    assert inp.meta.shape == (w.m, w.ld_meta) and w.ld_meta % 16 == 0 and w.ld_meta >= k // 8
    assert np.all(inp.meta[:, k // 8:] == 0xFF)
    idx = _unpack(inp.meta, w.m, k).reshape(w.m, k // 4, 2)
    assert np.all(idx[..., 0] < idx[..., 1])            # two distinct positions, increasing
    code = {p: c for c, p in enumerate(SP24_PAIRS)}
    counts = np.bincount([code[(a, b)] for a, b in idx.reshape(-1, 2)], minlength=6)
    expect = idx.shape[0] * idx.shape[1] / 6
    assert np.all(np.abs(counts - expect) < 5 * np.sqrt(expect))


@pytest.mark.parametrize("atype", ["f16", "bf16"])
@pytest.mark.parametrize("transb", [False, True])
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (0.5, -1.25)])
def test_matches_dense_reference_of_decompressed_a(atype, transb, alpha, beta):
    w = Workload("sp_dense", atype, "f32", 37, 29, 256, transb=transb, alpha=alpha, beta=beta,
                 sparse24=True, a_dist="normal(0,1)", b_dist="normal(0,1)",
                 c_dist="normal(0,1)", seed=3)
    inp = generate(w)
    ref = oracle.gemm_sp24(transb, w.m, w.n, w.k, alpha, inp.A, atype, w.lda, inp.meta,
                           w.ld_meta, inp.B, w.ldb, beta, inp.C, "f32", w.ldc)
    Ad = _decompress(inp)
    dense = oracle.gemm_fp(False, transb, w.m, w.n, w.k, alpha, Ad, atype, w.k, inp.B, atype,
                           w.ldb, beta, inp.C, "f32", w.ldc)
    assert np.array_equal(ref.v, dense.v)
    assert np.array_equal(ref.S, dense.S)
    # the kept values really are only half of the work: a dense A with the other half nonzero
    # gives a different result
    Ad2 = Ad.copy()
    Ad2[Ad2 == 0] = 0x3C00 if atype == "f16" else 0x3F80
    other = oracle.gemm_fp(False, transb, w.m, w.n, w.k, alpha, Ad2, atype, w.k, inp.B, atype,
                           w.ldb, beta, inp.C, "f32", w.ldc)
    assert not np.allclose(other.v, ref.v)


@pytest.mark.parametrize("transb", [False, True])
def test_brute_force_any_positions(transb):
    """Tiny case, positions drawn freely (repeated and decreasing ones too), exact sums."""
    rng = np.random.default_rng(11)
    m, n, k = 3, 4, 16
    kh = k // 2
    idx = rng.integers(0, 4, size=(m, kh)).astype(np.uint8)
    idx[0, :2] = (3, 3)
    idx[1, 2:4] = (2, 0)
    meta = pack_sp24_meta(idx, 16)
    Ac = np.float16(rng.normal(size=(m, 8))).view(np.uint16)
    Bop = np.float16(rng.normal(size=(k, n))).view(np.uint16)
    B = np.ascontiguousarray(Bop.T) if transb else Bop
    C = np.float32(rng.normal(size=(m, n)))
    ldb = B.shape[1]
    alpha, beta = 0.75, 1.5
    ref = oracle.gemm_sp24(transb, m, n, k, alpha, Ac, "f16", 8, meta, 16, B, ldb, beta, C,
                           "f32", n)
    for i in range(m):
        for c in range(n):
            s = Fraction(0)
            sa = Fraction(0)
            for j in range(kh):
                r = 4 * (j // 2) + int(idx[i, j])
                prod = Fraction(float(_value16(Ac[i, j], "f16"))) * Fraction(
                    float(_value16(Bop[r, c], "f16")))
                s += prod
                sa += abs(prod)
            want = Fraction(alpha) * s + Fraction(beta) * Fraction(float(C[i, c]))
            assert abs(Fraction(ref.v[i, c]) - want) <= Fraction(2) ** -50 * (
                abs(Fraction(alpha)) * sa + abs(Fraction(beta) * Fraction(float(C[i, c]))))
            assert ref.S[i, c] == pytest.approx(float(sa), rel=1e-15)


@pytest.mark.parametrize("atype,dist", [("f16", "normal(0,1)"), ("bf16", "normal(0,1)"),
                                        ("bf16", "log_uniform(-60,40)"),
                                        ("f16", "log_uniform(-20,8)")])
@pytest.mark.parametrize("out", ["f32", "same"])
def test_block_model_of_four_kept_equals_dense_model(atype, dist, out):
    otype = atype if out == "same" else "f32"
    w = Workload("sp_model", atype, otype, 21, 19, 384, transb=True, alpha=1.0, beta=0.5,
                 sparse24=True, a_dist=dist, b_dist=dist, c_dist="normal(0,1)", seed=9)
    inp = generate(w)
    sp = oracle.gemm_sp24_mfma(True, w.m, w.n, w.k, 0.3, inp.A, atype, w.lda, inp.meta,
                               w.ld_meta, inp.B, w.ldb, -0.7, inp.C, otype, w.ldc, otype, nblk=4)
    dn = oracle.gemm_mfma(False, True, w.m, w.n, w.k, 0.3, _decompress(inp), atype, w.k, inp.B,
                          atype, w.ldb, -0.7, inp.C, otype, w.ldc, otype, nblk=8)
    assert np.array_equal(sp.view(np.uint32 if otype == "f32" else np.uint16),
                          dn.view(np.uint32 if otype == "f32" else np.uint16))
    # blocks of eight kept products are a different partition: not the same bits everywhere
    # for wide-range data
    if dist.startswith("log") and otype == "f32":
        sp8 = oracle.gemm_sp24_mfma(True, w.m, w.n, w.k, 0.3, inp.A, atype, w.lda, inp.meta,
                                    w.ld_meta, inp.B, w.ldb, -0.7, inp.C, otype, w.ldc, otype,
                                    nblk=8)
        assert not np.array_equal(sp8.view(np.uint8), sp.view(np.uint8))


def test_points_equal_full():
    w = Workload("sp_pts", "bf16", "f32", 40, 33, 128, sparse24=True, a_dist="normal(0,1)",
                 b_dist="normal(0,1)", seed=5)
    inp = generate(w)
    full = oracle.gemm_sp24(False, w.m, w.n, w.k, 1.0, inp.A, "bf16", w.lda, inp.meta,
                            w.ld_meta, inp.B, w.ldb, 0.0, None, "f32", w.ldc)
    ii = np.array([0, 39, 17, 5]); jj = np.array([0, 32, 1, 30])
    pts = oracle.gemm_sp24(False, w.m, w.n, w.k, 1.0, inp.A, "bf16", w.lda, inp.meta,
                           w.ld_meta, inp.B, w.ldb, 0.0, None, "f32", w.ldc, points=(ii, jj))
    assert np.array_equal(pts.v, full.v[ii, jj])


@pytest.mark.parametrize("transb", [False, True])
@pytest.mark.parametrize("alpha,beta", [(1, 0), (3, -2)])
def test_int8_matches_dense_int_reference_of_decompressed_a(transb, alpha, beta):
    """INT8: the sparse reference equals the dense INT8 reference of the decompressed A exactly
    (integers: no ordering question), including INT32 wrap-around with large alpha."""
    w = Workload("sp_int", "i8", "i32", 33, 27, 256, transb=transb, alpha=alpha, beta=beta,
                 sparse24=True, a_dist="int_uniform(-128,127)", b_dist="int_uniform(-128,127)",
                 c_dist="int_uniform(-1000,1000)", seed=13)
    inp = generate(w)
    ref = oracle.gemm_sp24_int(transb, w.m, w.n, w.k, alpha, inp.A, w.lda, inp.meta, w.ld_meta,
                               inp.B, w.ldb, beta, inp.C, w.ldc)
    idx = _unpack(inp.meta, w.m, w.k)
    Ad = np.zeros((w.m, w.k), np.int8)
    j = np.arange(w.k // 2)
    Ad[np.repeat(np.arange(w.m)[:, None], w.k // 2, 1), 4 * (j // 2) + idx] = inp.A[:, : w.k // 2]
    dense = oracle.gemm_int(False, transb, w.m, w.n, w.k, alpha, Ad, w.k, inp.B, w.ldb, beta,
                            inp.C, w.ldc)
    assert np.array_equal(ref, dense)
    big = oracle.gemm_sp24_int(transb, w.m, w.n, w.k, 1 << 20, inp.A, w.lda, inp.meta,
                               w.ld_meta, inp.B, w.ldb, 0, None, w.ldc)
    plain = oracle.gemm_int(False, transb, w.m, w.n, w.k, 1, Ad, w.k, inp.B, w.ldb, 0, None,
                            w.ldc).astype(np.int64)        # |sum| < 2^22: no wrap
    exact = plain * (1 << 20)
    assert np.array_equal(big, ((exact + (1 << 31)) % (1 << 32) - (1 << 31)).astype(np.int32))
    assert np.any(np.abs(exact) >= 1 << 31)                 # the wrap is exercised


def test_int8_brute_force_any_positions():
    rng = np.random.default_rng(17)
    m, n, k = 3, 5, 16
    idx = rng.integers(0, 4, size=(m, k // 2)).astype(np.uint8)
    idx[0, :2] = (2, 2)
    meta = pack_sp24_meta(idx, 16)
    Ac = rng.integers(-128, 128, size=(m, 16)).astype(np.int8)
    B = rng.integers(-128, 128, size=(k, 16)).astype(np.int8)
    C = rng.integers(-50, 50, size=(m, 8)).astype(np.int32)
    ref = oracle.gemm_sp24_int(False, m, n, k, -2, Ac, 16, meta, 16, B, 16, 5, C, 8)
    for i in range(m):
        for c in range(n):
            s = sum(int(Ac[i, j]) * int(B[4 * (j // 2) + int(idx[i, j]), c]) for j in range(k // 2))
            assert ref[i, c] == -2 * s + 5 * int(C[i, c])


@pytest.mark.parametrize("atype,btype", [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e4m3"),
                                         ("e5m2", "e5m2")])
@pytest.mark.parametrize("transb", [False, True])
def test_fp8_matches_dense_fp8_reference_of_decompressed_a(atype, btype, transb):
    w = Workload("sp_fp8", atype, "f32", 29, 23, 256, transb=transb, alpha=0.5, beta=-1.5,
                 sparse24=True, a_dist="normal(0,1)", b_dist="normal(0,1)",
                 c_dist="normal(0,1)", seed=15, b_type=btype)
    inp = generate(w)
    ref = oracle.gemm_sp24(transb, w.m, w.n, w.k, w.alpha, inp.A, atype, w.lda, inp.meta,
                           w.ld_meta, inp.B, w.ldb, w.beta, inp.C, "f32", w.ldc, btype=btype)
    idx = _unpack(inp.meta, w.m, w.k)
    Ad = np.zeros((w.m, w.k), np.uint8)
    j = np.arange(w.k // 2)
    Ad[np.repeat(np.arange(w.m)[:, None], w.k // 2, 1), 4 * (j // 2) + idx] = inp.A[:, : w.k // 2]
    dense = oracle.gemm_fp8(False, transb, w.m, w.n, w.k, w.alpha, Ad, atype, w.k, inp.B, btype,
                            w.ldb, w.beta, inp.C, "f32", w.ldc)
    assert np.array_equal(ref.v, dense.v) and np.array_equal(ref.S, dense.S)


@pytest.mark.parametrize("atype,btype", [("e4m3", "e4m3"), ("e5m2", "e4m3")])
@pytest.mark.parametrize("dist", ["normal(0,1)", "log_uniform(-9,8)"])
def test_fp8_sparse_model_of_four_kept_equals_dense_fp8_model(atype, btype, dist):
    """The FP8 block model over kept products with groups of 4 kept, blocks of 8 and 64 kept per
    instruction equals the dense FP8 model (groups of 8 k, blocks of 16, 128 k) of the
    decompressed A: each dense group holds exactly its 4 kept products, zeros take no part."""
    w = Workload("sp_f8m", atype, "f32", 19, 17, 512, transb=True, alpha=0.3, beta=-0.7,
                 sparse24=True, a_dist=dist, b_dist=dist, c_dist="normal(0,1)", seed=21,
                 b_type=btype)
    inp = generate(w)
    sp = oracle.gemm_sp24_fp8_mfma(True, w.m, w.n, w.k, w.alpha, inp.A, atype, w.lda, inp.meta,
                                   w.ld_meta, inp.B, btype, w.ldb, w.beta, inp.C, "f32", w.ldc,
                                   "f32", kinst=64, nblk=4, sblk=8)
    idx = _unpack(inp.meta, w.m, w.k)
    Ad = np.zeros((w.m, w.k), np.uint8)
    j = np.arange(w.k // 2)
    Ad[np.repeat(np.arange(w.m)[:, None], w.k // 2, 1), 4 * (j // 2) + idx] = inp.A[:, : w.k // 2]
    dn = oracle.gemm_fp8_mfma(False, True, w.m, w.n, w.k, w.alpha, Ad, atype, w.k, inp.B, btype,
                              w.ldb, w.beta, inp.C, "f32", w.ldc, "f32")
    assert np.array_equal(sp.view(np.uint32), dn.view(np.uint32))
