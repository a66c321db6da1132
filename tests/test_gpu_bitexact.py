"""GPU results equal the oracle's block-FMA model bit for bit (FP16/BF16 inputs).

The model (``oracle.gemm_mfma``) is the block-FMA accumulation of "NVIDIA Tensor Core
mixed-precision computing: principles and applications" (jsqmd.com/news/1087138), sections
2.2-2.3 and 4.2.1, with gfx950's parameters, pinned on the CPU by test_oracle_mfma_model.py.
Here whole outputs (sampled points for the largest shapes) are compared with it bitwise
(+0 equals -0, any NaN equals any NaN), on inputs chosen to reach every rule: typical data,
wide exponent ranges (the window cuts and the 32-bit block sum), tiny values (subnormal
inputs, FP32 subnormal results), ragged tile edges and K tails (blocks of zeros), the
epilogue with inexact alpha and beta, and Inf/NaN inputs.
"""
import numpy as np
import pytest

from gemm_inputs import WORKLOADS, Workload, generate, sample_points
from tests.gpu_harness import compare_model, run_gpu, say

pytestmark = pytest.mark.gpu

LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]


def _check(w: Workload, points=None, inp=None):
    say(f"[gpu bitexact] {w.name} {w.in_type}->{w.out_type} m={w.m} n={w.n} k={w.k} "
        f"ta={w.transa} tb={w.transb} alpha={w.alpha} beta={w.beta} a={w.a_dist} "
        f"points={'all' if points is None else len(points[0])}")
    inp = inp if inp is not None else generate(w)
    res = run_gpu(inp)
    rep = compare_model(inp, res, points=points)
    assert rep.ok, f"{rep.n_bad}/{rep.n} differ from the model; {rep.detail}"
    assert res.guard_ok
    return inp, res


def _edge_points(m, n, count, seed=1):
    """The last three rows and columns in full, the first row and column, and random points."""
    ii, jj = sample_points(m, n, count, seed=seed)
    rows = [r for r in (0, m - 3, m - 2, m - 1) if 0 <= r < m]
    cols = [c for c in (0, n - 3, n - 2, n - 1) if 0 <= c < n]
    extra_i = np.concatenate([np.repeat(rows, n), np.tile(np.arange(m), len(cols))])
    extra_j = np.concatenate([np.tile(np.arange(n), len(rows)), np.repeat(cols, m)])
    return (np.concatenate([ii, extra_i]).astype(np.int64),
            np.concatenate([jj, extra_j]).astype(np.int64))


@pytest.mark.parametrize("in_type,out_type", [("f16", "f32"), ("f16", "f16"), ("bf16", "f32"),
                                              ("bf16", "bf16")])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_random_bitexact(in_type, out_type, ta, tb):
    """Normal inputs over shapes spanning several tiles with ragged tails, beta = 0.5."""
    for (m, n, k) in [(300, 200, 333), (257, 263, 1000), (64, 64, 4095)]:
        _check(Workload(f"bx_rand_{in_type}_{out_type}", in_type, out_type, m, n, k, transa=ta,
                        transb=tb, alpha=1.0, beta=0.5, a_dist="normal(0,1)",
                        b_dist="normal(0,1)", c_dist="normal(0,1)", seed=17 + m))


@pytest.mark.parametrize("in_type,out_type", [("f16", "f32"), ("f16", "f16"), ("bf16", "f32"),
                                              ("bf16", "bf16")])
def test_epilogue_inexact_scalars_bitexact(in_type, out_type):
    """alpha = 0.3 and beta = -0.7 (not powers of two): the epilogue's single fused rounding."""
    for alpha, beta in ((0.3, -0.7), (-1.7, 0.0), (0.3, 1.0)):
        _check(Workload(f"bx_epi_{in_type}_{out_type}", in_type, out_type, 257, 129, 100,
                        alpha=alpha, beta=beta, a_dist="normal(0,1)", b_dist="normal(0,1)",
                        c_dist="normal(0,4)", seed=23))


@pytest.mark.parametrize("in_type,dist", [("f16", "log_uniform(-14,6)"), ("f16", "log_uniform(-24,15)"),
                                          ("bf16", "log_uniform(-40,30)"), ("bf16", "log_uniform(-120,60)")])
@pytest.mark.parametrize("k", [1000, 4096])
def test_wide_exponent_range_bitexact(in_type, dist, k):
    """Magnitudes spread over many binades: products far below the block's largest are cut,
    running sums far above the block's products keep 32 bits; FP16 draws below 2^-14 are
    subnormal inputs."""
    _check(Workload(f"bx_wide_{in_type}", in_type, "f32", 96, 96, k, a_dist=dist, b_dist=dist,
                    seed=k))


@pytest.mark.parametrize("in_type,dist", [("f16", "log_uniform(-25,-12)"), ("bf16", "log_uniform(-126,-60)"),
                                          ("bf16", "log_uniform(-90,-40)")])
def test_tiny_values_bitexact(in_type, dist):
    """Subnormal FP16 inputs, and BF16 products in and below FP32's subnormal range."""
    _check(Workload(f"bx_tiny_{in_type}", in_type, "f32", 128, 128, 520, a_dist=dist,
                    b_dist=dist, seed=31))


@pytest.mark.parametrize("in_type", ["f16", "bf16"])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_tile_edges_bitexact(in_type, ta, tb):
    """The tile-edge shapes (ragged 256 x 256 tiles, partial and odd K stages, K tails of
    zero blocks, ld equal to the row length) with real-valued data."""
    shapes = [(256 * 14 + 37, 256 * 14 + 5, 200), (256 * 15 + 255, 256 * 13 + 1, 136),
              (5, 3, 200), (300, 9, 136), (17, 260, 320), (1, 1, 1), (2, 513, 48), (257, 1, 4112)]
    for t, (m, n, k) in enumerate(shapes):
        w = Workload(f"bx_edge_{in_type}", in_type, "f32", m, n, k, transa=ta, transb=tb,
                     a_dist="normal(0,1)", b_dist="normal(0,1)", seed=5000 + t)
        _check(w, points=_edge_points(m, n, 4000) if m * n > 200_000 else None)


def test_workloads_bitexact():
    """The five workloads' FP cases at full size (sampled where the output is large)."""
    _check(WORKLOADS["f16_256_nn_beta1"])
    w = WORKLOADS["f16_4096_nt"]
    _check(w, points=sample_points(w.m, w.n, 3000))
    w = WORKLOADS["bf16_8192_nn"]
    _check(w, points=sample_points(w.m, w.n, 1500))
    for name in ("f16_5000x3000x1000_f16out", "f16_5000x3000x1000_f16out_padded"):
        w = WORKLOADS[name]
        _check(w, points=_edge_points(w.m, w.n, 4000))


@pytest.mark.parametrize("in_type", ["f16", "bf16"])
def test_special_values_bitexact(in_type):
    """Inf and NaN operands scattered over normal data: Inf x 0 and opposite infinities give
    NaN, other infinities propagate through their rows and columns."""
    w = Workload(f"bx_special_{in_type}", in_type, "f32", 70, 90, 300, a_dist="normal(0,1)",
                 b_dist="normal(0,1)", seed=41)
    inp = generate(w)
    rng = np.random.default_rng(41)
    inf, ninf, nan = (0x7C00, 0xFC00, 0x7E00) if in_type == "f16" else (0x7F80, 0xFF80, 0x7FC0)
    for arr, rows, cols in ((inp.A, w.m, w.k), (inp.B, w.k, w.n)):
        for val, count in ((inf, 6), (ninf, 6), (nan, 3), (0, 20)):
            arr[rng.integers(0, rows, count), rng.integers(0, cols, count)] = val
    _check(w, inp=inp)
