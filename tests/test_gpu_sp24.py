"""GPU parity of the 2:4 structured-sparse GEMM (mpgemm_run_sp24) against the oracle.

The oracle (``oracle.gemm_sp24``) sums the kept products Ac(i, j) * op(B)(4 (j / 2) +
idx(i, j), c) exactly in double (2:4 sparsity as the page "稀疏张量核心加速模板计算的技术解析" describes it, sections 1.2.1 and
1.3.2).  Integer-valued inputs whose sums are exact in FP32 must match bit for bit; real-valued
inputs must lie within the FP16/BF16 GEMM bound over the k/2 kept products.  Shapes span several
256 x 128 tiles with ragged m and n (k is a multiple of 128 by contract), both layouts of B,
FP32 and 16-bit outputs, free position patterns (repeated and decreasing positions included),
k = 0, D aliasing C, and the 4096^3 workloads (every output; the block-model checks at sampled
points).
"""
import numpy as np
import pytest

import mixed_precision_dense_amd as mp
from gemm_inputs import NEXT_WORKLOADS, Workload, generate, pack_sp24_meta, sample_points
from tests.gpu_harness import (compare_sp24, compare_sp24_fp8_model, compare_sp24_model,
                                run_sp24, say)

pytestmark = pytest.mark.gpu

TYPES = [("f16", "f32"), ("f16", "f16"), ("bf16", "f32"), ("bf16", "bf16")]


def _run(w, inp=None, exact=False, points=None, in_place=False):
    say(f"[gpu sp24] {w.name} {w.in_type}->{w.out_type} m={w.m} n={w.n} k={w.k} tb={w.transb} "
        f"lda={w.lda} ld_meta={w.ld_meta} ldb={w.ldb} ldc={w.ldc} alpha={w.alpha} "
        f"beta={w.beta} exact={exact} points={'all' if points is None else len(points[0])}")
    inp = inp if inp is not None else generate(w)
    res, st = run_sp24(inp, in_place=in_place)
    assert st == mp.SUCCESS
    rep = compare_sp24(inp, res, exact=exact, points=points)
    assert rep.ok, f"{rep.n_bad}/{rep.n} outside; {rep.detail}"
    assert res.guard_ok
    return inp, res


@pytest.mark.parametrize("in_type,out_type", TYPES)
@pytest.mark.parametrize("tb", [False, True])
def test_sp24_exact_integers(in_type, out_type, tb):
    """Small integers: every sum is exact in FP32, so D equals the oracle bit for bit."""
    for t, (m, n, k) in enumerate([(300, 200, 384), (256, 128, 128), (1, 1, 128),
                                   (513, 257, 1024), (255, 129, 256)]):
        _run(Workload(f"sp_int_{in_type}", in_type, out_type, m, n, k, transb=tb,
                      sparse24=True, a_dist="int_uniform(-3,3)", b_dist="int_uniform(-3,3)",
                      seed=100 + t), exact=True)


@pytest.mark.parametrize("in_type,out_type", TYPES)
@pytest.mark.parametrize("tb", [False, True])
def test_sp24_random_within_bound(in_type, out_type, tb):
    for t, (m, n, k) in enumerate([(300, 200, 384), (257, 263, 1024), (64, 64, 4096)]):
        _run(Workload(f"sp_rand_{in_type}", in_type, out_type, m, n, k, transb=tb, alpha=1.0,
                      beta=0.5, sparse24=True, a_dist="normal(0,1)", b_dist="normal(0,1)",
                      c_dist="normal(0,1)", seed=200 + t))


@pytest.mark.parametrize("in_type", ["f16", "bf16"])
@pytest.mark.parametrize("tb", [False, True])
def test_sp24_free_positions(in_type, tb):
    """Positions drawn freely from 0..3 for every kept value (repeated and decreasing pairs
    too): each kept value multiplies the row of op(B) its own position names."""
    w = Workload(f"sp_pos_{in_type}", in_type, "f32", 260, 140, 512, transb=tb, sparse24=True,
                 a_dist="int_uniform(-3,3)", b_dist="int_uniform(-3,3)", seed=301)
    inp = generate(w)
    rng = np.random.default_rng(301)
    idx = rng.integers(0, 4, size=(w.m, w.k // 2)).astype(np.uint8)
    inp.meta = pack_sp24_meta(idx, w.ld_meta)
    _run(w, inp=inp, exact=True)
    # every one of the 16 (first, second) position pairs in its own column of groups
    idx = np.zeros((w.m, w.k // 2), np.uint8)
    for q in range(w.k // 4):
        idx[:, 2 * q], idx[:, 2 * q + 1] = (q % 16) // 4, q % 4
    inp.meta = pack_sp24_meta(idx, w.ld_meta)
    _run(w, inp=inp, exact=True)


@pytest.mark.parametrize("in_type,out_type", TYPES)
def test_sp24_epilogue_scalars(in_type, out_type):
    for alpha, beta in ((0.3, -0.7), (-1.7, 0.0), (0.3, 1.0)):
        _run(Workload(f"sp_epi_{in_type}", in_type, out_type, 257, 129, 256, alpha=alpha,
                      beta=beta, sparse24=True, a_dist="normal(0,1)", b_dist="normal(0,1)",
                      c_dist="normal(0,4)", seed=23))


@pytest.mark.parametrize("in_type", ["f16", "bf16"])
def test_sp24_k_zero_and_in_place(in_type):
    """k = 0 gives D = beta * C; D may alias C."""
    _run(Workload(f"sp_k0_{in_type}", in_type, "f32", 300, 130, 0, beta=0.5, sparse24=True,
                  c_dist="normal(0,1)", seed=7))
    _run(Workload(f"sp_alias_{in_type}", in_type, "f32", 300, 130, 256, beta=1.0,
                  sparse24=True, a_dist="normal(0,1)", b_dist="normal(0,1)",
                  c_dist="normal(0,1)", seed=8), in_place=True)


@pytest.mark.parametrize("in_type", ["f16", "bf16"])
@pytest.mark.parametrize("tb", [False, True])
def test_sp24_padded_strides_and_edges(in_type, tb):
    """Leading dimensions beyond the row length, and a large ragged output (every element)."""
    m, n, k = 256 * 5 + 37, 128 * 7 + 5, 640
    w = Workload(f"sp_pad_{in_type}", in_type, "f32", m, n, k, transb=tb, sparse24=True,
                 lda=k // 2 + 24, ldb=(k if tb else 904) + 40, ldc=904 + 12, ld_meta=k // 8 + 48,
                 a_dist="normal(0,1)", b_dist="normal(0,1)", seed=9)
    _run(w)


@pytest.mark.parametrize("in_type", ["f16", "bf16"])
def test_sp24_special_values(in_type):
    """Inf and NaN kept values and B entries propagate; zeros are ordinary values."""
    w = Workload(f"sp_special_{in_type}", in_type, "f32", 70, 90, 256, sparse24=True,
                 a_dist="normal(0,1)", b_dist="normal(0,1)", seed=41)
    inp = generate(w)
    rng = np.random.default_rng(41)
    inf, ninf, nan = (0x7C00, 0xFC00, 0x7E00) if in_type == "f16" else (0x7F80, 0xFF80, 0x7FC0)
    for arr, rows, cols in ((inp.A, w.m, w.k // 2), (inp.B, w.k, w.n)):
        for val, count in ((inf, 4), (ninf, 4), (nan, 2), (0, 20)):
            arr[rng.integers(0, rows, count), rng.integers(0, cols, count)] = val
    _run(w, inp=inp)


def test_sp24_workload():
    w = NEXT_WORKLOADS["f16_sp24_4096_nt"]
    _run(w)


def test_sp24_rejections_launch_nothing():
    """Arguments outside the contract return the check's status and leave D untouched."""
    w = Workload("sp_rej", "f16", "f32", 64, 64, 256, sparse24=True, a_dist="normal(0,1)",
                 b_dist="normal(0,1)", seed=1)
    inp = generate(w)
    bad = Workload("sp_rej", "f16", "f32", 64, 64, 200, sparse24=True, a_dist="normal(0,1)",
                   b_dist="normal(0,1)", seed=1)      # k not a multiple of 128
    res, st = run_sp24(generate(bad), check=False)
    assert mp.STATUS[st] == "NOT_SUPPORTED" and res.guard_ok
    assert np.all(res.D.view(np.uint8) == 0x5A)
    w.ld_meta = 40                                     # not a multiple of 16
    inp.meta = np.zeros((w.m, 40), np.uint8)
    res, st = run_sp24(inp, check=False)
    assert mp.STATUS[st] == "NOT_SUPPORTED" and np.all(res.D.view(np.uint8) == 0x5A)


# --------------------------------------------------------------------------------------------
# Bit-exact: the sparse matrix cores accumulate the kept products in blocks of eight (sixteen
# logical k) under the dense block rules (oracle.gemm_sp24_mfma, pinned on the CPU against the
# dense model of the decompressed A).
def _bitexact(w, inp=None, points=None, in_place=False):
    say(f"[gpu sp24 bitexact] {w.name} {w.in_type}->{w.out_type} m={w.m} n={w.n} k={w.k} "
        f"tb={w.transb} alpha={w.alpha} beta={w.beta} a={w.a_dist} "
        f"points={'all' if points is None else len(points[0])}")
    inp = inp if inp is not None else generate(w)
    res, st = run_sp24(inp, in_place=in_place)
    assert st == mp.SUCCESS
    rep = compare_sp24_model(inp, res, points=points)
    assert rep.ok, f"{rep.n_bad}/{rep.n} differ from the model; {rep.detail}"
    assert res.guard_ok


@pytest.mark.parametrize("in_type,out_type", TYPES)
@pytest.mark.parametrize("tb", [False, True])
def test_sp24_bitexact_random(in_type, out_type, tb):
    for t, (m, n, k) in enumerate([(300, 200, 384), (257, 263, 1024), (64, 64, 4096)]):
        _bitexact(Workload(f"spx_rand_{in_type}", in_type, out_type, m, n, k, transb=tb,
                           alpha=0.3, beta=-0.7, sparse24=True, a_dist="normal(0,1)",
                           b_dist="normal(0,1)", c_dist="normal(0,1)", seed=400 + t))


@pytest.mark.parametrize("in_type,dist", [("f16", "log_uniform(-14,6)"),
                                          ("f16", "log_uniform(-24,15)"),
                                          ("f16", "log_uniform(-25,-12)"),
                                          ("bf16", "log_uniform(-40,30)"),
                                          ("bf16", "log_uniform(-120,60)"),
                                          ("bf16", "log_uniform(-126,-60)")])
@pytest.mark.parametrize("tb", [False, True])
def test_sp24_bitexact_wide_and_tiny(in_type, dist, tb):
    """Wide exponent ranges (window cuts, the 32-bit block sum), subnormal FP16 inputs and
    FP32-subnormal BF16 products."""
    _bitexact(Workload(f"spx_wide_{in_type}", in_type, "f32", 96, 96, 2048, transb=tb,
                       sparse24=True, a_dist=dist, b_dist=dist, seed=500))


@pytest.mark.parametrize("in_type", ["f16", "bf16"])
def test_sp24_bitexact_free_positions_and_specials(in_type):
    w = Workload(f"spx_pos_{in_type}", in_type, "f32", 260, 140, 512, sparse24=True,
                 a_dist="normal(0,1)", b_dist="normal(0,1)", seed=501)
    inp = generate(w)
    rng = np.random.default_rng(501)
    inp.meta = pack_sp24_meta(rng.integers(0, 4, size=(w.m, w.k // 2)).astype(np.uint8),
                              w.ld_meta)
    _bitexact(w, inp=inp)
    inf, ninf, nan = (0x7C00, 0xFC00, 0x7E00) if in_type == "f16" else (0x7F80, 0xFF80, 0x7FC0)
    for arr, rows, cols in ((inp.A, w.m, w.k // 2), (inp.B, w.k, w.n)):
        for val, count in ((inf, 4), (ninf, 4), (nan, 2), (0, 20)):
            arr[rng.integers(0, rows, count), rng.integers(0, cols, count)] = val
    _bitexact(w, inp=inp)


def test_sp24_bitexact_workload():
    w = NEXT_WORKLOADS["f16_sp24_4096_nt"]
    _bitexact(w, points=sample_points(w.m, w.n, 3000))


# --------------------------------------------------------------------------------------------
# INT8 inputs (v_smfmac_i32_16x16x128_i8): exact INT32 results, wrapping like the dense path.
@pytest.mark.parametrize("tb", [False, True])
@pytest.mark.parametrize("alpha,beta", [(1, 0), (3, -2)])
def test_sp24_int8_exact(tb, alpha, beta):
    """Shapes with odd and even counts of 128-deep INT8 stages (k = 128, 384, 640: a zero stage
    pads the last pair), ragged m and n, full-range values, C read when beta != 0."""
    for t, (m, n, k) in enumerate([(300, 200, 384), (256, 256, 256), (1, 1, 128),
                                   (513, 257, 1024), (255, 129, 640)]):
        _run(Workload(f"sp_i8_{alpha}_{beta}", "i8", "i32", m, n, k, transb=tb, alpha=alpha,
                      beta=beta, sparse24=True, a_dist="int_uniform(-128,127)",
                      b_dist="int_uniform(-128,127)", c_dist="int_uniform(-100000,100000)",
                      seed=600 + t))


@pytest.mark.parametrize("tb", [False, True])
def test_sp24_int8_free_positions_wrap_and_k0(tb):
    w = Workload("sp_i8_pos", "i8", "i32", 260, 140, 512, transb=tb, alpha=1 << 20, beta=0,
                 sparse24=True, a_dist="int_uniform(-128,127)", b_dist="int_uniform(-128,127)",
                 seed=601)
    inp = generate(w)
    rng = np.random.default_rng(601)
    inp.meta = pack_sp24_meta(rng.integers(0, 4, size=(w.m, w.k // 2)).astype(np.uint8),
                              w.ld_meta)
    _run(w, inp=inp)                     # alpha = 2^20: the INT32 epilogue wraps
    _run(Workload("sp_i8_k0", "i8", "i32", 300, 130, 0, alpha=1, beta=-3, sparse24=True,
                  c_dist="int_uniform(-1000,1000)", seed=602))
    _run(Workload("sp_i8_alias", "i8", "i32", 300, 130, 256, alpha=2, beta=1, sparse24=True,
                  a_dist="int_uniform(-128,127)", b_dist="int_uniform(-128,127)",
                  c_dist="int_uniform(-1000,1000)", seed=603), in_place=True)


@pytest.mark.parametrize("tb", [False, True])
def test_sp24_int8_padded_strides_and_edges(tb):
    m, n, k = 256 * 5 + 37, 256 * 3 + 5, 768
    w = Workload("sp_i8_pad", "i8", "i32", m, n, k, transb=tb, sparse24=True,
                 lda=k // 2 + 48, ldb=(k if tb else 784) + 32, ldc=776, ld_meta=k // 8 + 32,
                 a_dist="int_uniform(-128,127)", b_dist="int_uniform(-128,127)", seed=604)
    _run(w)


def test_sp24_int8_workload():
    w = NEXT_WORKLOADS["i8_sp24_4096_nn"]
    _run(w)


# --------------------------------------------------------------------------------------------
# FP8 inputs (v_smfmac_f32_16x16x128_{fp8,bf8}_{fp8,bf8}, OCP E4M3 / E5M2, either pairing).
FP8_PAIRS = [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")]


@pytest.mark.parametrize("a_t,b_t", FP8_PAIRS)
@pytest.mark.parametrize("out_type", ["f32", "bf16"])
@pytest.mark.parametrize("tb", [False, True])
def test_sp24_fp8_exact_integers(a_t, b_t, out_type, tb):
    """Integers -7..7 are exact in both formats; every sum here is exact in FP32 and in the
    matrix cores' 13-bit block window, so D is the oracle's once-rounded value."""
    for t, (m, n, k) in enumerate([(300, 200, 384), (1, 1, 128), (513, 257, 1024)]):
        _run(Workload(f"sp_f8int_{a_t}_{b_t}", a_t, out_type, m, n, k, transb=tb, b_type=b_t,
                      sparse24=True, a_dist="int_uniform(-7,7)", b_dist="int_uniform(-7,7)",
                      seed=700 + t), exact=True)


@pytest.mark.parametrize("a_t,b_t", FP8_PAIRS)
@pytest.mark.parametrize("tb", [False, True])
def test_sp24_fp8_random_within_bound(a_t, b_t, tb):
    for t, (m, n, k) in enumerate([(300, 200, 384), (257, 263, 1024), (64, 64, 4096)]):
        _run(Workload(f"sp_f8_{a_t}_{b_t}", a_t, "f32", m, n, k, transb=tb, b_type=b_t,
                      alpha=0.5, beta=0.5, sparse24=True, a_dist="normal(0,1)",
                      b_dist="normal(0,1)", c_dist="normal(0,1)", seed=710 + t))


def test_sp24_fp8_edges_and_workload():
    m, n, k = 256 * 5 + 37, 256 * 3 + 5, 640
    w = Workload("sp_f8_pad", "e4m3", "bf16", m, n, k, sparse24=True, lda=k // 2 + 48,
                 ldb=784 + 32, ldc=776 + 8, ld_meta=k // 8 + 32, a_dist="normal(0,1)",
                 b_dist="normal(0,1)", seed=720)
    _run(w)
    _run(Workload("sp_f8_k0", "e5m2", "f32", 300, 130, 0, beta=0.5, sparse24=True,
                  c_dist="normal(0,1)", seed=721))
    w = NEXT_WORKLOADS["e4m3_sp24_4096_nt"]
    _run(w)


@pytest.mark.parametrize("a_t,b_t", FP8_PAIRS)
@pytest.mark.parametrize("tb", [False, True])
def test_sp24_fp8_bitexact(a_t, b_t, tb):
    """The sparse FP8 instructions follow the FP8 block model over the kept products in kept
    order (groups of 8 kept products; 64 kept per instruction)."""
    for t, (m, n, k, out, alpha, beta) in enumerate([(300, 200, 384, "f32", 1.0, 0.0),
                                                     (257, 129, 1024, "bf16", 0.3, -0.7)]):
        w = Workload(f"spx_f8_{a_t}_{b_t}", a_t, out, m, n, k, transb=tb, b_type=b_t,
                     alpha=alpha, beta=beta, sparse24=True, a_dist="normal(0,1)",
                     b_dist="normal(0,1)", c_dist="normal(0,1)", seed=730 + t)
        say(f"[gpu sp24 fp8 bitexact] {w.name} {out} m={m} n={n} k={k} tb={tb}")
        inp = generate(w)
        res, st = run_sp24(inp)
        assert st == mp.SUCCESS
        rep = compare_sp24_fp8_model(inp, res)
        assert rep.ok, f"{rep.n_bad}/{rep.n} differ from the model; {rep.detail}"


@pytest.mark.parametrize("a_t,b_t,tb,k,dists", [
    ("e4m3", "e4m3", True, 512, ("log_uniform(-6,6)", "log_uniform(-6,6)")),
    ("e5m2", "e5m2", False, 1024, ("log_uniform(-12,12)", "log_uniform(-12,12)")),
    ("e4m3", "e5m2", True, 384, ("log_uniform(-6,6)", "log_uniform(-12,12)"))])
def test_sp24_fp8_bitexact_wide_range(a_t, b_t, tb, k, dists):
    """Kept values and B spread over many binades: blocks of 16 kept products meet the
    accumulator far above and below them, and the model's rules for that hold too."""
    w = Workload(f"spx_f8w_{a_t}_{b_t}", a_t, "f32", 256, 256, k, transb=tb, b_type=b_t,
                 sparse24=True, a_dist=dists[0], b_dist=dists[1], seed=740 + k)
    say(f"[gpu sp24 fp8 wide] {w.name} k={k} tb={tb} a={dists[0]} b={dists[1]}")
    inp = generate(w)
    res, st = run_sp24(inp)
    assert st == mp.SUCCESS
    rep = compare_sp24_fp8_model(inp, res)
    assert rep.ok, f"{rep.n_bad}/{rep.n} differ from the model; {rep.detail}"


def test_sp24_fp8_bitexact_workload():
    w = NEXT_WORKLOADS["e4m3_sp24_4096_nt"]
    inp = generate(w)
    res, st = run_sp24(inp)
    pts = sample_points(w.m, w.n, 3000)
    rep = compare_sp24_fp8_model(inp, res, points=pts)
    assert rep.ok, f"{rep.n_bad}/{rep.n} differ from the model; {rep.detail}"


@pytest.mark.parametrize("which", ["lda", "ld_meta", "ldc"])
def test_sp24_largest_accepted_strides(which):
    """Kept values, metadata or D at the largest leading dimension the argument check accepts
    (256 rows just under 2 GiB): the second tile row starts that far on and every in-tile
    offset of the 32-bit buffer addressing stays in range.  Bit-exact against the sparse
    block model."""
    limit = (1 << 31) - 4096
    big = {"lda": limit // (256 * 2), "ld_meta": limit // 256, "ldc": limit // (256 * 4)}
    w = Workload(f"sp_maxld_{which}", "f16", "f32", 300, 72, 256, transb=True, sparse24=True,
                 a_dist="normal(0,1)", b_dist="normal(0,1)", seed=58, **{which: big[which]})
    inp, res = _run(w)
    rep = compare_sp24_model(inp, res)
    assert rep.ok, f"{rep.n_bad}/{rep.n} differ from the model; {rep.detail}"
