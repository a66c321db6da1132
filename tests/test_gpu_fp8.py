"""GPU parity of FP8 inputs (E4M3 / E5M2 for A and B each, FP32 accumulation), the two formats
of "NVIDIA Tensor Core mixed-precision computing: principles and applications", section 4.3.1.

  * integer-valued inputs in [-4, 4]: every product and partial sum lies on the grid that
    gfx950's FP8 accumulation keeps, so results are exact and compared bit for bit (every
    layout and format pair, ragged tile edges and K tails, both output types);
  * random inputs within the bound of the measured accumulation (oracle.fp8_bound);
  * the FP8 benchmark workload (every output); NaN and Inf inputs; k = 0.
"""
import numpy as np
import pytest

import mixed_precision_dense_amd as mp
from gemm_inputs import Workload, generate, sample_points
from tests.gpu_harness import check_case, compare, run_gpu, say

pytestmark = pytest.mark.gpu

LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]
PAIRS = [("e4m3", "e4m3"), ("e4m3", "e5m2"), ("e5m2", "e4m3"), ("e5m2", "e5m2")]
ST = {v: k for k, v in mp.STATUS.items()}


def _assert(rep, res):
    assert rep.ok, f"{rep.n_bad}/{rep.n} bad, worst ratio {rep.worst_ratio:.3g}: {rep.detail}"
    assert res.guard_ok


@pytest.mark.parametrize("a_t,b_t", PAIRS)
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_fp8_integer_exact(a_t, b_t, ta, tb):
    shapes = [(256 * 14 + 37, 256 * 14 + 5, 208), (300, 200, 333), (5, 3, 272), (17, 260, 320),
              (1, 1, 1), (257, 1, 4112), (513, 771, 1000)]
    for t, (m, n, k) in enumerate(shapes):
        out = "bf16" if t % 3 == 2 else "f32"
        w = Workload(f"fp8_int_{a_t}_{b_t}", a_t, out, m, n, k, b_type=b_t, transa=ta, transb=tb,
                     alpha=1.0, beta=0.0 if t % 2 else 1.0, a_dist="int_uniform(-4,4)",
                     b_dist="int_uniform(-4,4)", c_dist="int_uniform(-50,50)", seed=400 + t)
        rep, res = check_case(w, exact=True)
        _assert(rep, res)


@pytest.mark.parametrize("a_t,b_t", PAIRS)
@pytest.mark.parametrize("ta,tb", [(False, False), (False, True), (True, True)])
def test_fp8_random_within_bound(a_t, b_t, ta, tb):
    for (m, n, k), out, alpha, beta in [((300, 200, 333), "f32", 1.0, 0.5),
                                         ((257, 263, 1000), "bf16", 0.3, 0.0),
                                         ((64, 64, 4095), "f32", 1.0, -1.0)]:
        w = Workload(f"fp8_rand_{a_t}_{b_t}", a_t, out, m, n, k, b_type=b_t, transa=ta, transb=tb,
                     alpha=alpha, beta=beta, a_dist="normal(0,1)", b_dist="normal(0,2)",
                     c_dist="normal(0,1)", seed=500 + m)
        rep, res = check_case(w)
        _assert(rep, res)
        say(f"  worst error / bound = {rep.worst_ratio:.4f}")


def test_fp8_workload_full():
    w = Workload("e4m3_4096_nt", "e4m3", "f32", 4096, 4096, 4096, transb=True,
                 a_dist="normal(0,1)", b_dist="normal(0,1)", seed=8)
    rep, res = check_case(w)
    _assert(rep, res)
    say(f"  worst error / bound = {rep.worst_ratio:.4f}")


def test_fp8_specials():
    for a_t, b_t in (("e4m3", "e4m3"), ("e5m2", "e5m2"), ("e4m3", "e5m2")):
        w = Workload(f"fp8_special_{a_t}_{b_t}", a_t, "f32", 70, 90, 300, b_type=b_t,
                     a_dist="normal(0,1)", b_dist="normal(0,1)", seed=44)
        inp = generate(w)
        rng = np.random.default_rng(44)
        for arr, fmt, rows, cols in ((inp.A, a_t, w.m, w.k), (inp.B, b_t, w.k, w.n)):
            specials = [0x7F, 0xFF] if fmt == "e4m3" else [0x7C, 0xFC, 0x7E]
            for val in specials:
                arr[rng.integers(0, rows, 3), rng.integers(0, cols, 3)] = val
        res = run_gpu(inp)
        rep = compare(inp, res)
        _assert(rep, res)


def test_fp8_k_zero_and_contract():
    w = Workload("fp8_k0", "e4m3", "f32", 33, 40, 0, b_type="e5m2", alpha=1.0, beta=2.0,
                 c_dist="uniform(-1,1)", lda=16, ldb=48, seed=9)
    rep, res = check_case(w, exact=True)
    _assert(rep, res)
    P = 1 << 20
    assert mp.mpgemm_check(False, False, 64, 64, 64, 1.0, P, "e4m3", 64, P, "e5m2", 64, 0.0, None,
                           "f16", 64, P, "f32") == ST["NOT_SUPPORTED"]          # FP16 out
    assert mp.mpgemm_check(False, False, 64, 64, 64, 1.0, P, "e4m3", 72, P, "e4m3", 64, 0.0, None,
                           "f32", 64, P, "f32") == ST["NOT_SUPPORTED"]          # 72 B rows
    assert mp.mpgemm_check(False, False, 64, 64, 64, 1.0, P, "e4m3", 64, P, "e4m3", 64, 0.0, None,
                           "f32", 64, P, "i32") == ST["NOT_SUPPORTED"]
