"""Pins for the oracle's number-format code: exhaustive decodes checked against numpy and
torch, and round-to-nearest-even encoders checked against library conversions and against
a brute-force nearest-value search.  CPU only."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _decode_all(fmt):
    return np.array([oracle.decode(b, fmt) for b in range(65536)])


def _same(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return both_nan | eq


def test_decode_f16_exhaustive_vs_numpy():
    ours = _decode_all("f16")
    ref = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    assert np.all(_same(ours, ref))
    # spot values from the binary16 definition (1 sign, 5 exponent, 10 fraction bits)
    assert oracle.decode(0x3C00, "f16") == 1.0
    assert oracle.decode(0x7BFF, "f16") == 65504.0
    assert oracle.decode(0x0001, "f16") == 2.0 ** -24
    assert oracle.decode(0x0400, "f16") == 2.0 ** -14
    assert oracle.decode(0xFC00, "f16") == -np.inf


def test_decode_bf16_exhaustive_vs_numpy_and_torch():
    ours = _decode_all("bf16")
    via_f32 = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(_same(ours, via_f32))
    t = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    via_torch = t.to(torch.float64).numpy()
    assert np.all(_same(ours, via_torch))


def test_decode_f32_sample_vs_numpy():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    bits[:6] = [0, 0x80000000, 1, 0x007FFFFF, 0x7F800000, 0x7FC00000]
    ours = np.array([oracle.decode(int(b), "f32") for b in bits])
    assert np.all(_same(ours, bits.view(np.float32).astype(np.float64)))


def _interesting_doubles(rng, lo_exp, hi_exp, count):
    mant = rng.uniform(1.0, 2.0, count)
    exps = rng.integers(lo_exp, hi_exp, count)
    signs = rng.choice([-1.0, 1.0], count)
    return signs * np.ldexp(mant, exps)


def test_encode_f16_vs_numpy():
    rng = np.random.default_rng(11)
    vals = np.concatenate([
        _interesting_doubles(rng, -30, 17, 40000),          # subnormal .. overflow
        np.arange(2049, 4097, dtype=np.float64),              # ties at spacing 2
        (np.arange(1, 2048) + 0.5) * 2.0 ** -24,              # subnormal ties
        [65504.0, 65519.0, 65519.999, 65520.0, 65536.0, 1e9, -65520.0, 2.0 ** -25,
         2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 0.0, -0.0, np.inf, -np.inf],
    ])
    ours = np.array([oracle.encode_rne(v, "f16") for v in vals], dtype=np.uint16)
    ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_encode_f16_tie_table():
    # odd integers in [2049, 4095] sit halfway between two FP16 neighbours (spacing 2);
    # ties go to the even significand
    for n in range(2049, 4096, 2):
        got = oracle.decode(oracle.encode_rne(float(n), "f16"), "f16")
        lo, hi = n - 1, n + 1
        expect = lo if (lo // 2) % 2 == 0 else hi
        assert got == expect, n
    assert oracle.decode(oracle.encode_rne(2049.0, "f16"), "f16") == 2048.0
    assert oracle.decode(oracle.encode_rne(2051.0, "f16"), "f16") == 2052.0
    assert oracle.encode_rne(65520.0, "f16") == 0x7C00
    assert oracle.encode_rne(65519.99, "f16") == 0x7BFF
    assert oracle.encode_rne(float("nan"), "f16") & 0x7C00 == 0x7C00


def test_encode_nan_is_the_quiet_nan_with_its_sign():
    """A NaN encodes as the exponent field all ones with only the leading fraction bit set (the
    quiet NaN of IEEE 754, section 6.2.1), keeping the sign: not as an infinity."""
    for fmt, (e, m) in {"f16": (5, 10), "bf16": (8, 7), "f32": (8, 23)}.items():
        quiet = (((1 << e) - 1) << m) | (1 << (m - 1))
        assert oracle.encode_rne(float("nan"), fmt) == quiet, fmt
        assert oracle.encode_rne(-float("nan"), fmt) == quiet | (1 << (e + m)), fmt
    assert oracle.encode_rne(float("nan"), "f16") == int(np.array(np.nan, np.float16).view(np.uint16))
    assert oracle.encode_rne(float("nan"), "f32") == int(np.array(np.nan, np.float32).view(np.uint32))


def test_encode_f32_vs_numpy():
    rng = np.random.default_rng(12)
    vals = np.concatenate([
        _interesting_doubles(rng, -160, 130, 40000),
        (np.arange(1, 1000) + 0.5) * 2.0 ** -149,
        [2.25 + 3 * 2.0 ** -24, 255 * 2.0 ** -157, 3.4028235677973366e38, 3.5e38],
    ])
    ours = np.array([oracle.encode_rne(v, "f32") for v in vals], dtype=np.uint64).astype(np.uint32)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float32).view(np.uint32)
    assert np.array_equal(ours, ref)


def _all_finite_bf16():
    bits = np.arange(0, 0x7F80, dtype=np.uint32)          # +0 .. largest finite
    vals = (bits << 16).view(np.float32).astype(np.float64)
    return bits, vals


def test_encode_bf16_brute_force_nearest():
    """Nearest-value search over every positive finite BF16 value, ties to even pattern."""
    bits, vals = _all_finite_bf16()
    rng = np.random.default_rng(13)
    probes = np.concatenate([
        np.abs(_interesting_doubles(rng, -135, 128, 3000)),
        (vals[1:200] + vals[2:201]) / 2,                     # exact midpoints (ties)
        (vals[30000:30100] + vals[30001:30101]) / 2,
    ])
    for x in probes:
        i = np.searchsorted(vals, x)
        cands = [j for j in (i - 1, i) if 0 <= j < len(vals)]
        if i >= len(vals):
            continue
        d = [abs(Fraction(float(vals[j])) - Fraction(float(x))) for j in cands]
        best = min(d)
        winners = [cands[t] for t in range(len(cands)) if d[t] == best]
        expect = winners[0] if len(winners) == 1 else [w for w in winners if w % 2 == 0][0]
        assert oracle.encode_rne(float(x), "bf16") == int(bits[expect]), x
        assert oracle.encode_rne(-float(x), "bf16") == int(bits[expect]) | 0x8000


def test_round_array_matches_scalar_encoder():
    rng = np.random.default_rng(3)
    v = rng.normal(0, 100, 1000)
    for fmt in ("f16", "bf16"):
        arr = oracle.round_to(v, fmt)
        assert [int(x) for x in arr] == [oracle.encode_rne(x, fmt) for x in v]
    f = oracle.round_to(v, "f32")
    assert np.array_equal(f, v.astype(np.float32))
