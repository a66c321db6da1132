"""GPU parity of mpgemm_run_bf16x3, the FP32 GEMM computed from BF16 pieces (multiword
emulation, "NVIDIA Tensor Core mixed-precision computing: principles and applications",
section 5.1).

  * the split kernel's output (the workspace) equals the oracle's pieces bit for bit,
    padding included, for every layout;
  * D equals the oracle's block model of the three-product GEMM bit for bit, and lies within
    the method's bound of the double-precision FP32 GEMM;
  * ragged k (pieces padded to multiples of 8), tile edges, the benchmark workload (the model
    at sampled points, the bound at every output),
    Inf/NaN/overflowing/subnormal inputs, k = 0, D == C, and the workspace contract.
"""
import numpy as np
import pytest

import mixed_precision_dense_amd as mp
import oracle
from gemm_inputs import Workload, generate, sample_points
from tests.gpu_harness import run_bf16x3, say

pytestmark = pytest.mark.gpu

LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]
ST = {v: k for k, v in mp.STATUS.items()}


def _check(w: Workload, points=None, inp=None, pieces=True, accuracy=True):
    say(f"[gpu bf16x3] {w.name} m={w.m} n={w.n} k={w.k} ta={w.transa} tb={w.transb} "
        f"alpha={w.alpha} beta={w.beta} a={w.a_dist} points={'all' if points is None else len(points[0])}")
    inp = inp if inp is not None else generate(w)
    res, ws, _ = run_bf16x3(inp)
    assert res.guard_ok
    model, (A3, lda3, B3, ldb3, k3) = oracle.gemm_bf16x3(
        w.transa, w.transb, w.m, w.n, w.k, w.alpha, inp.A, w.lda, inp.B, w.ldb, w.beta, inp.C,
        w.ldc, points=points)
    if pieces and w.k > 0:
        off_b = (A3.nbytes + 255) // 256 * 256
        got_a = ws[: A3.nbytes].view(np.uint16).reshape(A3.shape)
        got_b = ws[off_b: off_b + B3.nbytes].view(np.uint16).reshape(B3.shape)
        assert np.array_equal(got_a, A3), "A pieces differ"
        assert np.array_equal(got_b, B3), "B pieces differ"
    D = res.D[:, : w.n]
    if points is not None:
        D = D[points[0], points[1]]
    rep = oracle.check_bits(np.ascontiguousarray(D), "f32", model)
    assert rep.ok, f"{rep.n_bad}/{rep.n} differ from the model; {rep.detail}"
    if accuracy:
        v, S = oracle.gemm_f32(w.transa, w.transb, w.m, w.n, w.k, w.alpha, inp.A, w.lda, inp.B,
                               w.ldb, w.beta, inp.C, w.ldc, points=points)
        if w.beta:
            c = inp.C[:, : w.n].astype(np.float64)
            bc = w.beta * (c if points is None else c[points[0], points[1]])
        else:
            bc = np.zeros_like(v)
        err = np.abs(np.asarray(D, np.float64) - v)
        bound = oracle.bf16x3_bound(S, w.k, w.alpha, bc)
        fin = np.isfinite(v)
        assert np.all(err[fin] <= bound[fin]), f"max err/bound {np.max(err[fin] / bound[fin]):.3g}"
    return inp, res


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_bf16x3_bitexact_and_accurate(ta, tb):
    for (m, n, k) in [(300, 200, 333), (257, 263, 1000), (64, 64, 4095), (5, 3, 7), (1, 1, 1)]:
        _check(Workload("bx3_rand", "f32", "f32", m, n, k, transa=ta, transb=tb, alpha=1.0,
                        beta=0.5, a_dist="normal(0,1)", b_dist="normal(0,1)",
                        c_dist="normal(0,1)", seed=61 + k))


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_bf16x3_tile_edges_and_scalars(ta, tb):
    shapes = [(256 * 14 + 37, 256 * 14 + 5, 200), (17, 260, 320), (2, 513, 48), (257, 1, 4112)]
    for t, (m, n, k) in enumerate(shapes):
        w = Workload("bx3_edge", "f32", "f32", m, n, k, transa=ta, transb=tb, alpha=0.3, beta=-0.7,
                     a_dist="uniform(-1,1)", b_dist="normal(0,2)", c_dist="normal(0,1)", seed=70 + t)
        big = m * n > 200_000
        _check(w, points=sample_points(m, n, 3000) if big else None)


def test_bf16x3_workload_sampled():
    w = Workload("f32_4096_nt_bf16x3", "f32", "f32", 4096, 4096, 4096, transb=True,
                 a_dist="normal(0,1)", b_dist="normal(0,1)", seed=6)
    _check(w, points=sample_points(w.m, w.n, 2000))


def test_bf16x3_workload_every_output_within_bound():
    """Every output of the 4096^3 workload against the double-precision FP32 GEMM, within the
    three-product bound (the block model is compared at sampled points above: over all 16.7 M
    outputs its 12288-term sums would keep the oracle busy for minutes)."""
    w = Workload("f32_4096_nt_bf16x3", "f32", "f32", 4096, 4096, 4096, transb=True,
                 a_dist="normal(0,1)", b_dist="normal(0,1)", seed=6)
    say(f"[gpu bf16x3] {w.name} every output against the FP32 GEMM in double")
    inp = generate(w)
    res, _, _ = run_bf16x3(inp)
    assert res.guard_ok
    v, S = oracle.gemm_f32(w.transa, w.transb, w.m, w.n, w.k, w.alpha, inp.A, w.lda, inp.B,
                           w.ldb, w.beta, inp.C, w.ldc)
    bc = w.beta * inp.C[:, : w.n].astype(np.float64) if w.beta else np.zeros_like(v)
    D = np.asarray(res.D[:, : w.n], np.float64)
    assert np.all(np.isfinite(D)) and np.all(np.isfinite(v))
    ratio = np.abs(D - v) / oracle.bf16x3_bound(S, w.k, w.alpha, bc)
    say(f"[gpu bf16x3] worst error / bound over {ratio.size} outputs: {ratio.max():.3g}")
    assert ratio.max() <= 1.0


@pytest.mark.parametrize("dist", ["log_uniform(-60,60)", "log_uniform(-140,-100)"])
def test_bf16x3_wide_and_subnormal_inputs(dist):
    """Magnitudes over many binades, and FP32-subnormal inputs (whose pieces are BF16
    subnormals); accuracy is only checked where the products stay in the normal range."""
    w = Workload("bx3_range", "f32", "f32", 80, 72, 300, a_dist=dist, b_dist=dist, seed=81)
    _check(w, accuracy=dist.startswith("log_uniform(-60"))


def test_bf16x3_special_values():
    w = Workload("bx3_special", "f32", "f32", 70, 90, 300, a_dist="normal(0,1)",
                 b_dist="normal(0,1)", seed=91)
    inp = generate(w)
    rng = np.random.default_rng(91)
    for arr, rows, cols in ((inp.A, w.m, w.k), (inp.B, w.k, w.n)):
        for val, count in ((np.inf, 5), (-np.inf, 5), (np.nan, 3), (3.4e38, 4), (-3.39e38, 4),
                           (1e-41, 6), (0.0, 20)):
            arr[rng.integers(0, rows, count), rng.integers(0, cols, count)] = val
    _check(w, inp=inp, accuracy=False)


def test_bf16x3_k_zero_and_in_place():
    w = Workload("bx3_k0", "f32", "f32", 33, 20, 0, alpha=1.0, beta=-2.0, c_dist="normal(0,1)",
                 lda=4, ldb=20, seed=5)
    inp = generate(w)
    res, _, st = run_bf16x3(inp)
    assert st == ST["SUCCESS"] and res.guard_ok
    want = (np.float32(-2.0) * inp.C[:, : w.n]).astype(np.float32)
    assert np.array_equal(res.D[:, : w.n], want)
    w = Workload("bx3_inplace", "f32", "f32", 130, 70, 90, alpha=1.0, beta=1.0,
                 a_dist="normal(0,1)", b_dist="normal(0,1)", c_dist="normal(0,1)", seed=6)
    inp = generate(w)
    res, _, st = run_bf16x3(inp, in_place=True)
    model, _ = oracle.gemm_bf16x3(False, False, w.m, w.n, w.k, w.alpha, inp.A, w.lda, inp.B,
                                  w.ldb, w.beta, inp.C, w.ldc)
    assert oracle.check_bits(np.ascontiguousarray(res.D[:, : w.n]), "f32", model).ok
    assert res.guard_ok


def test_bf16x3_workspace_contract():
    w = Workload("bx3_ws", "f32", "f32", 40, 24, 56, a_dist="normal(0,1)", b_dist="normal(0,1)",
                 seed=7)
    inp = generate(w)
    need = mp.mpgemm_bf16x3_workspace_size(False, False, w.m, w.n, w.k)
    assert need == 40 * 168 * 2 + 168 * 24 * 2 + (256 - (40 * 168 * 2) % 256) % 256
    _, _, st = run_bf16x3(inp, workspace_bytes=need - 1, check=False)
    assert st == ST["INVALID_VALUE"]
    _, _, st = run_bf16x3(inp, workspace_bytes=0, check=False)
    assert st == ST["INVALID_VALUE"]
    _, _, st = run_bf16x3(inp, ws_offset=16, check=False)
    assert st == ST["NOT_SUPPORTED"]
    res, _, st = run_bf16x3(inp, workspace_bytes=need + 1000)
    assert st == ST["SUCCESS"] and res.guard_ok
