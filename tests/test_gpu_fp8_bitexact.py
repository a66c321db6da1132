"""FP8 GEMM outputs equal the oracle's two-level FP8 block model bit for bit.

The model (``oracle.gemm_fp8_mfma``, pinned by tests/test_oracle_fp8_model.py): groups of 8
products cut toward zero 13 bits below the group's largest exponent sum; blocks of 16 k, in k
order, each meeting the FP32 accumulator in a 24-bit window below the block's largest exponent
sum (and no finer than 31 bits below the accumulator's leading bit; an accumulator two or more
places below the window is dropped), the sum rounded to FP32 to nearest even after every block (the numerics page, "NVIDIA Tensor Core mixed-precision
computing: principles and applications", sections 2.2-2.3 and 4.2.1, with gfx950's parameters).
It reproduces gfx950 on narrow and on wide operand ranges (log-uniform over 24 binades of
products and more), every pairing and layout, and the probe vectors below, which decided the
rules.
"""
import numpy as np
import pytest

from gemm_inputs import NEXT_WORKLOADS, Workload, generate, sample_points
from tests.gpu_harness import compare, compare_fp8_model, run_gpu, say

pytestmark = pytest.mark.gpu

PAIRS = [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")]
LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]


def _check(w, points=None, inp=None):
    say(f"[gpu fp8 bitexact] {w.name} {w.in_type}x{w.b_type}->{w.out_type} m={w.m} n={w.n} "
        f"k={w.k} ta={w.transa} tb={w.transb} alpha={w.alpha} beta={w.beta} a={w.a_dist} "
        f"points={'all' if points is None else len(points[0])}")
    inp = inp if inp is not None else generate(w)
    res = run_gpu(inp)
    rep = compare_fp8_model(inp, res, points=points)
    assert rep.ok, f"{rep.n_bad}/{rep.n} differ from the model; {rep.detail}"
    assert res.guard_ok


@pytest.mark.parametrize("a_t,b_t", PAIRS)
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_fp8_bitexact_layouts(a_t, b_t, ta, tb):
    """Every pairing and layout, k = 1000 (a partial last instruction), ragged tiles."""
    _check(Workload(f"f8x_{a_t}_{b_t}", a_t, "f32", 200, 136, 1000, transa=ta, transb=tb,
                    b_type=b_t, a_dist="normal(0,1)", b_dist="normal(0,1)", seed=31))


@pytest.mark.parametrize("dist", ["normal(0,1)", "uniform(-1,1)", "log_uniform(-3,3)"])
def test_fp8_bitexact_distributions_and_epilogue(dist):
    _check(Workload("f8x_dist", "e4m3", "bf16", 257, 129, 4096, b_type="e4m3", alpha=0.3,
                    beta=-0.7, a_dist=dist, b_dist=dist, c_dist="normal(0,1)", seed=32))
    _check(Workload("f8x_dist5", "e5m2", "f32", 96, 96, 1024, b_type="e5m2", a_dist=dist,
                    b_dist=dist, seed=33))


def test_fp8_bitexact_tile_edges_and_specials():
    for t, (m, n, k) in enumerate([(513, 257, 1000), (1, 1, 1), (5, 3, 200), (300, 9, 136),
                                   (17, 260, 4100)]):
        _check(Workload("f8x_edge", "e4m3", "f32", m, n, k, b_type="e5m2", a_dist="normal(0,1)",
                        b_dist="normal(0,1)", seed=40 + t))
    w = Workload("f8x_special", "e5m2", "f32", 70, 90, 300, b_type="e5m2", a_dist="normal(0,1)",
                 b_dist="normal(0,1)", seed=41)
    inp = generate(w)
    rng = np.random.default_rng(41)
    for arr, rows, cols in ((inp.A, w.m, w.k), (inp.B, w.k, w.n)):
        for val, count in ((0x7C, 4), (0xFC, 4), (0x7E, 2), (0, 20)):   # +Inf, -Inf, NaN, 0
            arr[rng.integers(0, rows, count), rng.integers(0, cols, count)] = val
    _check(w, inp=inp)


def test_fp8_bitexact_workload():
    w = NEXT_WORKLOADS["e4m3_4096_nt"]
    _check(w, points=sample_points(w.m, w.n, 3000))


# Operands spread over many binades (log-uniform magnitudes): products of one output span 24
# binades (E4M3 over 2^-6 .. 2^6) or 48 (E5M2 over 2^-12 .. 2^12), so blocks meet accumulators
# far above or below them and every rule of the block model is exercised.
W6, W12 = "log_uniform(-6,6)", "log_uniform(-12,12)"
WIDE_CASES = [
    Workload("f8x_wide", "e4m3", "f32", 256, 256, 128, b_type="e4m3", a_dist=W6, b_dist=W6,
             seed=35),
    Workload("f8x_wide_k1000", "e4m3", "f32", 256, 256, 1000, b_type="e4m3", a_dist=W6,
             b_dist=W6, seed=201),
    Workload("f8x_wide_e5", "e5m2", "f32", 256, 256, 512, b_type="e5m2", a_dist=W12,
             b_dist=W12, seed=202),
    Workload("f8x_wide_mixed", "e4m3", "bf16", 200, 136, 333, b_type="e5m2", transa=True,
             alpha=0.3, beta=-0.7, a_dist=W6, b_dist=W12, c_dist="normal(0,1)", seed=203),
    Workload("f8x_wide_long", "e5m2", "f32", 256, 256, 4096, b_type="e4m3", transb=True,
             a_dist=W12, b_dist=W6, seed=204),
]


@pytest.mark.parametrize("w", WIDE_CASES, ids=[w.name for w in WIDE_CASES])
def test_fp8_bitexact_wide_range(w):
    say(f"[gpu fp8 wide] {w.name} {w.in_type}x{w.b_type}->{w.out_type} m={w.m} n={w.n} k={w.k} "
        f"a={w.a_dist} b={w.b_dist}")
    inp = generate(w)
    res = run_gpu(inp)
    rep = compare(inp, res)
    assert rep.ok, f"{rep.n_bad}/{rep.n} outside the FP8 bound; {rep.detail}"
    assert res.guard_ok
    model = compare_fp8_model(inp, res)
    assert model.ok, f"{model.n_bad}/{model.n} differ from the model; {model.detail}"


def _sweep_case(t):
    """Random configuration t of the sweep: pairing, layout, k, shape, output type, alpha,
    beta and operand distributions (normal, uniform, log-uniform over up to 31 binades,
    E5M2 subnormals included), dense or (every fourth) 2:4 sparse."""
    rng = np.random.default_rng(2024 + t)
    dists = {"e4m3": ["normal(0,1)", "log_uniform(-6,6)", "log_uniform(-9,8)", "uniform(-1,1)"],
             "e5m2": ["normal(0,1)", "log_uniform(-12,12)", "log_uniform(-16,15)",
                      "log_uniform(-6,6)"]}
    fa, fb = ("e4m3", "e5m2")[rng.integers(2)], ("e4m3", "e5m2")[rng.integers(2)]
    sparse = t % 4 == 3
    k = int(rng.choice([16, 48, 128, 200, 384, 640, 1000, 2048]))
    if sparse:
        k = max(128, k // 128 * 128)
    return Workload(f"f8sweep{t}", fa, ("f32", "bf16")[rng.integers(2)], int(rng.integers(40, 300)),
                    int(rng.integers(40, 300)), k, transa=bool(rng.integers(2)) and not sparse,
                    transb=bool(rng.integers(2)), b_type=fb,
                    alpha=float(rng.choice([1.0, 0.3, -2.0])),
                    beta=float(rng.choice([0.0, 0.5, -1.25])), a_dist=dists[fa][rng.integers(4)],
                    b_dist=dists[fb][rng.integers(4)], c_dist="normal(0,1)", seed=900 + t,
                    sparse24=sparse)


@pytest.mark.parametrize("t", range(16))
def test_fp8_bitexact_random_sweep(t):
    from tests.gpu_harness import compare_sp24_fp8_model, run_sp24
    w = _sweep_case(t)
    say(f"[gpu fp8 sweep] {w.name} {'sparse ' if w.sparse24 else ''}{w.in_type}x{w.b_type}->"
        f"{w.out_type} m={w.m} n={w.n} k={w.k} ta={w.transa} tb={w.transb} a={w.a_dist} "
        f"b={w.b_dist} alpha={w.alpha} beta={w.beta}")
    inp = generate(w)
    if w.sparse24:
        res, _ = run_sp24(inp)
        rep = compare_sp24_fp8_model(inp, res)
    else:
        res = run_gpu(inp)
        rep = compare_fp8_model(inp, res)
    assert rep.ok, f"{rep.n_bad}/{rep.n} differ from the model; {rep.detail}"


# GNFT-style feature-detection vectors of the FP8 instruction (the numerics page, section 3.1),
# which fixed the model's rules: each probe is one diagonal output of a small E5M2 GEMM whose
# A row and B column hold a few chosen power-of-two products at chosen k.  The whole output
# must equal the FP8 block model bit for bit, and the facts the rules rest on are asserted.
def _probe_case(probes, K=256, fmt="e5m2"):
    import torch
    from gemm_inputs import f64_to_fp8_bits
    T = len(probes)
    w = Workload("fp8_probe", fmt, "f32", T, T, K, b_type=fmt, a_dist="zeros", b_dist="zeros",
                 seed=0)
    inp = generate(w)
    a = np.zeros((T, K))
    b = np.zeros((K, T))
    for t, pr in enumerate(probes):
        for k, av, bv in pr:
            a[t, k] = av
            b[k, t] = bv
    for x in (a, b):      # every probe value is exact in the format
        back = torch.from_numpy(f64_to_fp8_bits(x, fmt)).view(torch.float8_e5m2).double().numpy()
        assert np.array_equal(back, x)
    inp.A[:, :K] = f64_to_fp8_bits(a, fmt)
    inp.B[:K, :T] = f64_to_fp8_bits(b, fmt)
    res = run_gpu(inp)
    rep = compare_fp8_model(inp, res)
    assert rep.ok, f"{rep.n_bad}/{rep.n} differ from the model; {rep.detail}"
    return np.diag(res.D[:, :T]).astype(np.float64)


def test_fp8_gnft_blocks_of_16_in_order():
    """+1 and -1 at k = p, p + 1 beside 2^-30 at k = q: the tiny product is lost exactly when q
    lies in the pair's block of 16 or in an earlier block of the same 128-deep instruction."""
    tiny = 2.0 ** -15
    for p in (0, 16, 112):
        qs = [q for q in range(128) if q not in (p, p + 1)]
        say(f"[gpu fp8 gnft] blocks: pair at k = {p}, {p + 1}")
        d = _probe_case([[(p, 1.0, 1.0), (p + 1, 1.0, -1.0), (q, tiny, tiny)] for q in qs])
        lost = {q for q, v in zip(qs, d) if v == 0.0}
        assert lost == {q for q in qs if q < (p // 16 + 1) * 16}
        assert all(v == tiny * tiny for q, v in zip(qs, d) if q not in lost)


def test_fp8_gnft_window_13_bits():
    """1 + 2^-x in one group of 8: 2^-13 is kept, 2^-14 and below are cut."""
    xs = list(range(10, 20))
    say("[gpu fp8 gnft] window: 1 + 2^-x")
    d = _probe_case([[(0, 1.0, 1.0), (1, 2.0 ** -(x // 2), 2.0 ** -(x - x // 2))] for x in xs])
    for x, v in zip(xs, d):
        assert v == (1.0 + 2.0 ** -x if x <= 13 else 1.0), (x, v)


def test_fp8_gnft_accumulator_carried_across_instructions():
    """2^s from the first 128-deep instruction, then 1 + 2^-x from the second: the carried FP32
    accumulator is not cut, so the result is the FP32 rounding of the exact sum whenever the
    second instruction keeps its 2^-x (x <= 13)."""
    probes, tags = [], []
    for sa in (4, 8, 12):
        for x in (8, 10, 12):
            probes.append([(0, 2.0 ** (sa // 2), 2.0 ** (sa - sa // 2)), (128, 1.0, 1.0),
                           (129, 2.0 ** -(x // 2), 2.0 ** -(x - x // 2))])
            tags.append((sa, x))
    say("[gpu fp8 gnft] accumulator: 2^s, then 1 + 2^-x")
    d = _probe_case(probes)
    for (sa, x), v in zip(tags, d):
        assert v == float(np.float32(2.0 ** sa + 1.0 + 2.0 ** -x)), (sa, x, v)


def test_fp8_gnft_rounded_after_each_block():
    """2^11 plus a 2^-12 / 2^-13 pattern in block 0, -2^10 (or -(2^11 + 2^10)) in block 1: the
    accumulator is rounded to FP32 after block 0 (ties to even, down and up, and a nearest
    case), which the finer spacing after block 1 shows; in one block the groups meet exactly."""
    big, down = (0, 2.0 ** 6, 2.0 ** 5), (16, -(2.0 ** 5), 2.0 ** 5)
    probes = [
        [big, (8, 2.0 ** -6, 2.0 ** -7), down],
        [big, (8, 2.0 ** -6, 2.0 ** -6), (9, 2.0 ** -6, 2.0 ** -7), down],
        [big, (1, 2.0 ** 6, 2.0 ** 5), (8, 2.0 ** -6, 2.0 ** -6), (9, 2.0 ** -6, 2.0 ** -7),
         (16, -(2.0 ** 6), 2.0 ** 5), (17, -(2.0 ** 5), 2.0 ** 5)],
        [big, (8, 2.0 ** -6, 2.0 ** -7), (1, -(2.0 ** 5), 2.0 ** 5)],
    ]
    say("[gpu fp8 gnft] rounding after each block")
    d = _probe_case(probes)
    assert list(d) == [2.0 ** 10, 2.0 ** 10 + 2.0 ** -11, 2.0 ** 10 + 2.0 ** -11,
                       2.0 ** 10 + 2.0 ** -13]


def test_fp8_gnft_accumulator_window():
    """Accumulator 2^20 from block 0; block 1 brings 2^-4 (half of FP32's spacing there) and
    2^t: kept for t >= 20 - 31 (the sum passes the tie and rounds up), cut below (the tie rounds
    to even); two groups of 2^-5 + 2^-12 are cut once as a total, not group by group; and a
    carried -2^-30, far below the next instruction's +1, -1 block (grid 2^-24), is dropped."""
    acc = (0, 2.0 ** 10, 2.0 ** 10)
    ts = [-10, -11, -12, -13]
    probes = [[acc, (16, 2.0 ** -2, 2.0 ** -2), (24, 2.0 ** (t // 2), 2.0 ** (t - t // 2))]
              for t in ts]
    probes.append([acc, (16, 2.0 ** -2, 2.0 ** -3), (17, 2.0 ** -6, 2.0 ** -6),
                   (24, 2.0 ** -2, 2.0 ** -3), (25, 2.0 ** -6, 2.0 ** -6)])
    probes.append([(0, -(2.0 ** -15), 2.0 ** -15), (128, 1.0, 1.0), (129, 1.0, -1.0)])
    say("[gpu fp8 gnft] accumulator window and cut")
    d = _probe_case(probes)
    up = 2.0 ** 20 + 2.0 ** -3
    assert list(d) == [up, up, 2.0 ** 20, 2.0 ** 20, up, 0.0]


def test_fp8_gnft_accumulator_cut_or_dropped():
    """A running sum meets a block of +1 (grid 2^-24), within an instruction and across one:
    cut toward -infinity (-2^-25 and -(2^-24 + 2^-25) lose to -2^-24 and -2^-23, +(2^-24 +
    2^-25) to 2^-24), kept on the grid, and dropped when its leading bit lies two or more places
    below the grid (-2^-26; -2^-25 beside a block of 2^4, grid 2^-20)."""
    p = lambda e: 2.0 ** e
    probes = [
        [(0, -p(-12), p(-13)), (16, 1.0, 1.0)],
        [(0, -p(-12), p(-13)), (128, 1.0, 1.0)],
        [(0, -p(-13), p(-13)), (16, 1.0, 1.0)],
        [(0, -p(-12), p(-12)), (1, -p(-12), p(-13)), (16, 1.0, 1.0)],
        [(0, -p(-12), p(-12)), (1, -p(-12), p(-13)), (128, 1.0, 1.0)],
        [(0, -p(-12), p(-12)), (16, 1.0, 1.0)],
        [(0, -p(-11), p(-12)), (1, -p(-12), p(-13)), (16, 1.0, 1.0)],
        [(0, p(-12), p(-12)), (1, p(-12), p(-13)), (16, -1.0, 1.0)],
        [(0, p(-12), p(-13)), (16, -1.0, 1.0)],
        [(0, -p(-12), p(-13)), (16, 2.0, 2.0)],
    ]
    say("[gpu fp8 gnft] accumulator cut or dropped")
    d = _probe_case(probes)
    one_down = float(np.float32(1.0 - p(-24)))
    assert list(d) == [one_down, one_down, 1.0, float(np.float32(1.0 - p(-23))),
                       float(np.float32(1.0 - p(-23))), one_down,
                       float(np.float32(1.0 - p(-23) - p(-24))), -one_down, -1.0, 4.0]
