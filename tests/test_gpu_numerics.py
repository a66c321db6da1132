"""GPU parity on adversarial accumulation vectors.

The vectors follow the test-vector method of "NVIDIA Tensor Core mixed-precision computing:
principles and applications" (jsqmd.com/news/1087138), section 3.1 (GNFT: inputs built to
expose accumulator width, block size, alignment and rounding), applied to this library: a
dominant product plus tiny ones in the same and in later k positions, cancellation inside a
k block and across blocks, ties at the FP32 rounding boundary, and products in the FP32
subnormal range.  These are the inputs on which a block-wise, truncating accumulation
differs most from the exact sum, so they probe the bound of the comparator rather than its
typical slack.  Expected values come from the oracle only; the comparator's bound (and the
bit-exact rule for exactly representable cases) decides.
"""
import numpy as np
import pytest

from gemm_inputs import Workload, generate, to_storage
from tests.gpu_harness import compare, compare_model, run_gpu, say

pytestmark = pytest.mark.gpu

T12 = 2.0 ** -12


def _vectors(K):
    """(name, [(k, a, b), ...]) probes; products a*b at position k, everything else zero."""
    v = []
    for e in (24, 25, 26):
        for n in (1, 3, 4, 7):
            v.append((f"same block 1 + {n} x 2^-{e}", [(0, 1.0, 1.0)] + [(q, T12, 2.0 ** -(e - 12)) for q in range(1, n + 1)]))
            v.append((f"same block 1 - {n} x 2^-{e}", [(0, 1.0, 1.0)] + [(q, T12, -(2.0 ** -(e - 12))) for q in range(1, n + 1)]))
            v.append((f"next block 1 + {n} x 2^-{e}", [(0, 1.0, 1.0)] + [(8 + q, T12, 2.0 ** -(e - 12)) for q in range(n)]))
    for j in (1, 7, 8, 9, 15, 16, 31):
        v.append((f"ties 1 + 2^-24 at 1 and {j + 1}", [(0, 1.0, 1.0), (1, T12, T12), (j + 1, T12, T12)]))
    v += [
        ("accumulator low bits vs large block", [(0, 1.0, 1.0), (1, T12, 2.0 ** -9), (2, T12, 2.0 ** -11), (8, 2.0, 4.0)]),
        ("large term in the same block", [(0, 1.0, 1.0), (1, T12, 2.0 ** -9), (2, T12, 2.0 ** -11), (3, 2.0, 4.0)]),
        ("cancellation in a block", [(0, 1.0, 1.0), (1, 1.0, -1.0), (2, T12, 2.0 ** -18)]),
        ("cancellation across blocks", [(0, 1.0, 1.0), (8, 1.0, -1.0), (9, T12, 2.0 ** -18)]),
        ("cancellation to a tiny remainder", [(0, 3.0, 5.0), (1, -2.0, 7.5), (2, T12, 2.0 ** -14), (3, T12, -(2.0 ** -13))]),
    ]
    return [(n, p) for n, p in v if all(k < K for k, _, _ in p)]


def _run(fmt, K, vectors, extra=()):
    vecs = list(vectors) + list(extra)
    T = len(vecs)
    w = Workload(f"gnft_{fmt}_k{K}", fmt, "f32", T, T, K, a_dist="zeros", b_dist="zeros", seed=90)
    inp = generate(w)
    a = np.zeros((T, K))
    b = np.zeros((K, T))
    for t, (_, probe) in enumerate(vecs):
        for k, av, bv in probe:
            a[t, k] = av
            b[k, t] = bv
    inp.A[:, :K] = to_storage(a, fmt)
    inp.B[:K, :T] = to_storage(b, fmt)
    res = run_gpu(inp)
    return inp, res, vecs


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("K", [32, 64])
def test_gnft_vectors_within_bound(fmt, K):
    vecs = _vectors(K)
    extra = []
    if fmt == "bf16":
        # products in FP32's subnormal range (BF16 reaches 2^-133): single, and split over blocks
        extra = [("product 2^-149", [(0, 2.0 ** -74, 2.0 ** -75)]),
                 ("product 2^-140", [(0, 2.0 ** -70, 2.0 ** -70)]),
                 ("4 x 2^-150 in one block", [(q, 2.0 ** -75, 2.0 ** -75) for q in range(4)]),
                 ("4 x 2^-150 in 4 blocks", [(8 * q, 2.0 ** -75, 2.0 ** -75) for q in range(4) if 8 * q < K]),
                 ("subnormal sum, last bit 2^-158", [(0, 2.0 ** -70, 2.0 ** -70), (1, 2.0 ** -75, 2.0 ** -75), (2, 2.0 ** -79, 2.0 ** -79)]),
                 ("subnormal sum, last bit 2^-157", [(0, 2.0 ** -70, 2.0 ** -70), (1, 2.0 ** -75, 2.0 ** -75), (2, 2.0 ** -78, 2.0 ** -79)])]
    inp, res, vecs = _run(fmt, K, vecs, extra)
    say(f"  {fmt} K={K}: {len(vecs)} vectors")
    # the input values must be exactly those requested (every probe value is representable)
    rep = compare(inp, res, underflow_floor=(fmt == "bf16"))
    assert rep.ok, f"{rep.n_bad}/{rep.n} outside the bound; worst ratio {rep.worst_ratio:.3g}; {rep.detail}"
    # and bit for bit the block-FMA model of the matrix cores
    bits = compare_model(inp, res)
    assert bits.ok, f"{bits.n_bad}/{bits.n} differ from the model; {bits.detail}"
    assert res.guard_ok
