"""The shared input generator: rounding of draws, layout, padding sentinels and seeding.
CPU only."""
import hashlib
import os

import numpy as np
import pytest

import oracle
from gemm_inputs import (NEXT_WORKLOADS, WORKLOADS, Workload, f64_to_bf16_bits,
                         f64_to_f16_bits, generate, sample_points)

DIGESTS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "input_digests.txt")


def _recorded_digests():
    rows = {}
    with open(DIGESTS) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, label, dtype, shape, digest = line.split()
            rows.setdefault(name, []).append((label, dtype, shape, digest))
    return rows


def test_bf16_rounding_agrees_with_oracle_encoder():
    # two independent implementations of round-to-nearest-even (integer bit arithmetic here,
    # field-by-field quantisation in the oracle)
    rng = np.random.default_rng(31)
    x = rng.normal(0, 0.5, 20000)
    x[:4] = [0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)]   # ties
    ours = f64_to_bf16_bits(x)
    assert [int(b) for b in ours] == [oracle.encode_rne(v, "bf16") for v in x]
    assert ours[1] == 0x3F80 and ours[2] == 0x3F82 and ours[3] == 0xBF80


def test_f16_rounding_agrees_with_oracle_encoder():
    rng = np.random.default_rng(32)
    x = np.concatenate([rng.normal(0, 1, 20000), rng.uniform(-2, 2, 1000) * 2.0 ** -16])
    assert [int(b) for b in f64_to_f16_bits(x)] == [oracle.encode_rne(v, "f16") for v in x]


def test_layout_padding_and_seed():
    w = Workload("t", "f16", "f16", 5, 7, 9, transa=True, lda=16, ldb=8, ldc=8, beta=1.0,
                 c_dist="uniform(-1,1)", seed=5)
    a = generate(w)
    assert a.A.shape == (9, 16) and a.B.shape == (9, 8) and a.C.shape == (5, 8)
    assert np.all(a.A[:, 5:] == 0x7E00) and np.all(a.B[:, 7:] == 0x7E00)
    b = generate(w)
    assert np.array_equal(a.A, b.A) and np.array_equal(a.C, b.C)
    c = generate(w, seed=6)
    assert not np.array_equal(a.A, c.A)


def test_int8_draws_cover_range():
    w = Workload("i", "i8", "i32", 64, 64, 256, a_dist="int_uniform(-128,127)",
                 b_dist="int_uniform(-128,127)", seed=3)
    g = generate(w)
    assert g.A.min() == -128 and g.A.max() == 127 and g.C is None


def test_sample_points_in_range():
    ii, jj = sample_points(5000, 3000, 1000)
    assert ii.min() >= 0 and ii.max() == 4999 and jj.min() >= 0 and jj.max() == 2999


def test_named_workloads():
    assert set(WORKLOADS) >= {"f16_256_nn_beta1", "f16_4096_nt", "bf16_8192_nn", "i8_4096_nn",
                              "f16_5000x3000x1000_f16out"}


def test_log_uniform_spreads_over_binades():
    """'log_uniform(e0,e1)': both signs, magnitudes 2^u with u uniform in [e0, e1) (before the
    one rounding to the storage format), deterministic for a seed."""
    from gemm_inputs import draw
    rng = np.random.Generator(np.random.PCG64(3))
    x = draw(rng, (200, 300), "log_uniform(-20,10)", "f16").view(np.float16).astype(np.float64)
    e = np.floor(np.log2(np.abs(x[x != 0])))
    assert e.min() >= -21 and e.max() <= 10
    counts = np.bincount((e + 21).astype(int), minlength=32)[1:31]
    assert counts.min() > 0.7 * counts.mean()          # every binade about equally often
    assert 0.45 < np.mean(x > 0) < 0.55
    y = draw(np.random.Generator(np.random.PCG64(3)), (200, 300), "log_uniform(-20,10)", "f16")
    assert np.array_equal(y.view(np.uint16), x.astype(np.float16).view(np.uint16))


def test_every_workload_has_recorded_digests():
    assert set(_recorded_digests()) == set(WORKLOADS) | set(NEXT_WORKLOADS)


@pytest.mark.parametrize("name", sorted(set(WORKLOADS) | set(NEXT_WORKLOADS)))
def test_input_buffers_match_their_recorded_digests(name):
    """Each named workload's seeded buffers hash to the SHA-256 recorded when the workloads
    were fixed (golden/input_digests.txt, written by golden/make_input_digests.py from the
    generator alone): the same inputs on every machine and run."""
    w = WORKLOADS.get(name) or NEXT_WORKLOADS[name]
    inp = generate(w)
    for label, dtype, shape, digest in _recorded_digests()[name]:
        arr = getattr(inp, label)
        assert str(arr.dtype) == dtype and "x".join(map(str, arr.shape)) == shape, (name, label)
        assert hashlib.sha256(arr.tobytes()).hexdigest() == digest, (name, label)
