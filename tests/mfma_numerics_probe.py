"""Characterise how the GPU path accumulates FP16/BF16 products (not a test; needs a GPU).

    python tests/mfma_numerics_probe.py

Follows the test-vector method of "NVIDIA Tensor Core mixed-precision computing: principles
and applications" (jsqmd.com/news/1087138), section 3.1 (GNFT), through the library's C ABI:
each probe is one output element D[t][t] of a small GEMM whose A row t and B column t hold a
few chosen products at chosen k positions.  It prints, per probe family, what the GPU
returns next to the exact value (in units of 2^-23), and asserts nothing.  Families:

  blocks    1 at k = 0 plus 2^-24 at positions j < j2: the result is 1 + 2^-23 exactly when
            j and j2 are summed before the running sum is rounded to FP32 (same block).
  window    1 plus n products of 2^-e in the same block: how far below the largest product a
            term still counts.
  negative  the same with negative small terms (truncation toward zero or toward -inf).
  acc       a later block's alignment against the running sum (1 + 2^-21 + 2^-23, then 8).
  subnorm   BF16 products in FP32's subnormal range.
  subin     subnormal inputs as the largest product of a block: does the alignment take the
            exponent of the leading bit or the format's minimum exponent?
  floor     a negative running sum with bits below the next block's window.
  special   FP32 overflow inside and across blocks, Inf and NaN inputs.
  zero      a zero operand times a large one beside small products: does a zero's exponent
            take part in the alignment?
  subexp    which exponent a subnormal input stands for (the minimum normal one, or one below).
  width     a running value 2^s, then a block (0.25 - 0.25 + half of 2^s's spacing + 2^x):
            whether the last bit 2^x still breaks the tie, i.e. how many bits below the
            running value's leading bit the block's sum keeps.
  sumref    ties next to a binade edge, with a last bit of either sign: is that limit set by
            the running value's leading bit or by the sum's, and does the block's product sum
            lose its low bits toward minus infinity or each product toward zero?

FP8 (E5M2 x E5M2, v_mfma_f32_16x16x128_f8f6f4), in the same way:
  fp8blocks +1 and -1 at k = b, b + 1 beside 2^-30 at k = q: the 2^-30 vanishes when q shares
            the pair's block, or comes before it in the same 128-deep instruction (the
            instruction's running sum is cut at the next block's window).
  fp8window 1 + 2^-x in one block: the block's window width.
  fp8acc    2^s accumulated over the first 128 k, then 1 + 2^-x: the accumulator's precision.
"""
import itertools
import os
import sys
from fractions import Fraction

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from gemm_inputs import Workload, f64_to_fp8_bits, generate  # noqa: E402
from tests.gpu_harness import run_gpu  # noqa: E402

T12 = 2.0 ** -12
INF = float("inf")


def storage(x, fmt):
    """Exact bit patterns of values representable in fmt (Inf and NaN included)."""
    if fmt == "e5m2":
        import torch
        bits = f64_to_fp8_bits(x, "e5m2")
        back = torch.from_numpy(bits).view(torch.float8_e5m2).to(torch.float64).numpy()
        assert np.all((back == x) | np.isnan(x)), "value not representable in e5m2"
        return bits
    if fmt == "f16":
        h = x.astype(np.float16)
        ok = np.isnan(x) | (h.astype(np.float64) == x)
        assert ok.all(), "value not representable in f16"
        return h.view(np.uint16)
    f = x.astype(np.float32)
    u = f.view(np.uint32)
    ok = np.isnan(x) | ((f.astype(np.float64) == x) & ((u & 0xFFFF) == 0))
    assert ok.all(), "value not representable in bf16"
    return (u >> 16).astype(np.uint16)


def split(v):
    """Two FP16/BF16-representable factors of the power of two v (their product is v)."""
    e = int(np.log2(v))
    return 2.0 ** (e // 2), 2.0 ** (e - e // 2)


def width_probes():
    """Running value +-2^s (block 0), then a block with the pair c - c (c = 1 or 0.25, which
    sets the block exponent), half of 2^s's FP32 spacing and one more bit 2^x, for every x
    from just below the half down to the block's window."""
    out = []
    for c, emax in ((1.0, 0), (0.25, -2)):
        for sa in range(3, 14):
            for sign in (1.0, -1.0):
                if sign < 0 and sa not in (6, 8):
                    continue
                half = 2.0 ** (sa - 24)
                for x in range(sa - 25, emax - 25, -1):
                    a0, b0 = split(2.0 ** sa)
                    ah, bh = split(half)
                    out.append([(0, a0, sign * b0), (8, c ** 0.5, c ** 0.5), (9, c ** 0.5, -(c ** 0.5)),
                                (10, ah, sign * bh), (11, 2.0 ** -13, sign * 2.0 ** (x + 13))])
    return out


def run(fmt, K, probes):
    T = len(probes)
    w = Workload("probe", fmt, "f32", T, T, K, a_dist="zeros", b_dist="zeros", seed=0)
    inp = generate(w)
    a = np.zeros((T, K))
    b = np.zeros((K, T))
    for t, pr in enumerate(probes):
        for k, av, bv in pr:
            a[t, k] = av
            b[k, t] = bv
    inp.A[:, :K] = storage(a, fmt)
    inp.B[:K, :T] = storage(b, fmt)
    D = run_gpu(inp).D
    return [float(D[t, t]) for t in range(T)]


def fp8_main():
    print("=== e5m2 x e5m2")
    K = 256
    tiny = 2.0 ** -15
    for b in (0, 16, 32, 112):
        probes = [[(b, 1.0, 1.0), (b + 1, 1.0, -1.0), (q, tiny, tiny)] for q in range(128) if q not in (b, b + 1)]
        qs = [q for q in range(128) if q not in (b, b + 1)]
        res = run("e5m2", K, probes)
        gone = [q for q, v in zip(qs, res) if v == 0.0]
        print(f"fp8blocks: pair at k = {b}, {b + 1}: 2^-30 vanished at k in [{min(gone)}, {max(gone)}] "
              f"({len(gone)} positions)" if gone else f"fp8blocks: pair at {b}: none vanished")
    probes = [[(0, 1.0, 1.0), (1, 2.0 ** -(x // 2), 2.0 ** -(x - x // 2))] for x in range(10, 20)]
    res = run("e5m2", K, probes)
    print("fp8window: 1 + 2^-x, gpu - 1:", [(x, v - 1.0) for x, v in zip(range(10, 20), res)])
    probes, tags = [], []
    for sa in (4, 8, 12):
        for x in (8, 10, 12, 14, 16, 18, 20):
            probes.append([(0, 2.0 ** (sa // 2), 2.0 ** (sa - sa // 2)), (128, 1.0, 1.0),
                           (129, 2.0 ** -(x // 2), 2.0 ** -(x - x // 2))])
            tags.append((sa, x))
    res = run("e5m2", K, probes)
    for (sa, x), v in zip(tags, res):
        print(f"fp8acc: 2^{sa} then 1 + 2^-{x}: gpu - exact = {v - (2.0 ** sa + 1 + 2.0 ** -x):.3g}")


def ulp_diff(v, probe):
    if not all(np.isfinite([a * b for _, a, b in probe])) or not np.isfinite(v):
        return float("nan"), float(sum(a * b for _, a, b in probe))
    exact = sum(Fraction(a) * Fraction(b) for _, a, b in probe)
    return float((Fraction(v) - exact) / Fraction(2.0 ** -23)), float(exact)


def main():
    for fmt in ("f16", "bf16"):
        print(f"=== {fmt}")
        K = 64
        pairs = list(itertools.combinations(range(1, K), 2))
        probes = [[(0, 1.0, 1.0), (j, T12, T12), (j2, T12, T12)] for j, j2 in pairs]
        res = run(fmt, K, probes)
        together = {p for p, v in zip(pairs, res) if v == 1.0 + 2.0 ** -23}
        print("blocks: positions summed before rounding (groups of k):")
        groups, seen = [], set()
        for j in range(1, K):
            if j in seen:
                continue
            g = [j] + [j2 for j2 in range(j + 1, K) if (j, j2) in together]
            seen.update(g)
            groups.append((min(g), max(g)))
        print("   ", groups)
        fams = {
            "window": [[(0, 1.0, 1.0)] + [(q, T12, 2.0 ** -(e - 12)) for q in range(1, n + 1)]
                       for e in (24, 25, 26) for n in (1, 3, 4, 7)],
            "negative": [[(0, 1.0, 1.0)] + [(q, T12, -(2.0 ** -(e - 12))) for q in range(1, n + 1)]
                         for e in (24, 25) for n in (1, 3, 4, 7)],
            "acc": [[(0, 1.0, 1.0), (1, T12, 2.0 ** -9), (2, T12, 2.0 ** -11), (8, 2.0, 4.0)],
                    [(0, 1.0, 1.0), (1, T12, 2.0 ** -9), (2, T12, 2.0 ** -11), (8, 1.0, 2.0)],
                    [(0, 1.0, 1.0)] + [(8 + q, T12, 2.0 ** -13) for q in range(4)]],
        }
        fams["floor"] = [[(0, 1.0, -1.0), (1, T12, -(2.0 ** -11)), (8, 2.0, 4.0)],
                         [(0, 1.0, 1.0), (1, T12, 2.0 ** -11), (8, -2.0, 4.0)],
                         [(0, 1.0, -1.0), (1, T12, -(2.0 ** -11)), (8, -2.0, 4.0)]]
        if fmt == "f16":
            # 2^-20 and 2^-24 are FP16 subnormals (smallest normal 2^-14)
            fams["subin"] = [[(0, 2.0 ** -20, 1.0)] + [(q, 2.0 ** -20, 2.0 ** -24) for q in (1, 2, 3)],
                             [(0, 1.0, 2.0 ** -20)] + [(q, 2.0 ** -24, 2.0 ** -20) for q in (1, 2, 3)]]
            fams["special"] = [[(0, INF, 1.0)], [(0, INF, 0.0)], [(0, INF, 1.0), (1, -INF, 1.0)],
                               [(0, float("nan"), 1.0)], [(0, INF, 1.0), (8, -INF, 1.0)],
                               [(0, 65504.0, 65504.0)] * 1]
        else:
            # 2^-130 is a BF16 subnormal (smallest normal 2^-126)
            fams["subin"] = [[(0, 2.0 ** -130, 2.0 ** 100)] + [(q, 2.0 ** -130, 2.0 ** 76) for q in (1, 2, 3)],
                             [(0, 2.0 ** 100, 2.0 ** -130)] + [(q, 2.0 ** 76, 2.0 ** -130) for q in (1, 2, 3)]]
            fams["special"] = [[(0, 2.0 ** 127, 2.0)], [(0, 2.0 ** 127, 2.0), (1, 2.0 ** 127, -2.0)],
                               [(0, 2.0 ** 127, 2.0), (8, 2.0 ** 127, -2.0)],
                               [(0, 2.0 ** 127, 1.5), (1, 2.0 ** 127, 1.5)],
                               [(0, 2.0 ** 127, 1.0), (1, 2.0 ** 127, 1.0), (2, 2.0 ** 127, -1.0)],
                               [(0, 2.0 ** 127, 1.0), (8, 2.0 ** 127, 1.0), (16, 2.0 ** 127, -1.0)],
                               [(0, INF, 1.0)], [(0, INF, 0.0)], [(0, INF, 1.0), (1, -INF, 1.0)],
                               [(0, float("nan"), 1.0)], [(0, INF, 1.0), (8, -INF, 1.0)]]
        small = [(q, T12, 2.0 ** -13) for q in (1, 2, 3)]       # 3 x 2^-25 beside 0.5
        big = 2.0 ** 15 if fmt == "f16" else 2.0 ** 127
        fams["zero"] = [[(0, 0.5, 1.0)] + small,
                        [(0, 0.5, 1.0)] + small + [(4, 0.0, big)],
                        [(0, 0.5, 1.0)] + small + [(4, 0.0, big / 2)],
                        [(0, 0.5, 1.0)] + small + [(4, big, 0.0)],
                        [(0, 0.5, 1.0)] + small + [(4, big / 2, 0.0)]]
        fams["width"] = width_probes()
        pair = [(8, 1.0, 1.0), (9, 1.0, -1.0)]                         # block exponent 0
        fams["sumref"] = (
            # running 2^8; block -2^-15 + 2^-17 + 2^x: a tie whose even side is below
            [[(0, 16.0, 16.0)] + pair + [(10, 2.0 ** -8, -(2.0 ** -7)), (11, 2.0 ** -9, 2.0 ** -8),
                                        (12, 2.0 ** -13, 2.0 ** (x + 13))] for x in (-22, -23, -24)]
            # running 2^8; block -2^-17 - 2^x: a tie whose even side is above
            + [[(0, 16.0, 16.0)] + pair + [(10, 2.0 ** -9, -(2.0 ** -8)), (11, 2.0 ** -13, -(2.0 ** (x + 13)))]
               for x in (-23, -24)]
            # running 2^8 - 2^-16; block 2^-15 + 2^x: the sum crosses into the binade above
            + [[(0, 16.0, 16.0), (1, 2.0 ** -8, -(2.0 ** -8))] + pair + [(10, 2.0 ** -8, 2.0 ** -7),
                                                                       (11, 2.0 ** -13, 2.0 ** (x + 13))]
               for x in (-23, -24)])
        if fmt == "f16":   # 2^-20 x 1 beside 3 x 2^-39 (2^-20 x 2^-19): window 2^-38 or 2^-39
            fams["subexp"] = [[(0, 2.0 ** -20, 1.0)] + [(q, 2.0 ** -20, 2.0 ** -19) for q in (1, 2, 3)]]
        else:              # 2^-130 x 2^100 beside 3 x 2^-51 (2^-130 x 2^79): window 2^-50 or 2^-51
            fams["subexp"] = [[(0, 2.0 ** -130, 2.0 ** 100)] + [(q, 2.0 ** -130, 2.0 ** 79) for q in (1, 2, 3)]]
            fams["special"].append([(0, 1.5 * 2.0 ** 127, 1.5), (1, 2.0 ** 127, -1.0)])
            fams["special"].append([(0, 1.5 * 2.0 ** 126, 1.5), (1, 2.0 ** 127, -1.0)])
        if fmt == "bf16":
            fams["subnorm"] = [[(0, 2.0 ** -74, 2.0 ** -75)], [(0, 2.0 ** -75, 2.0 ** -75)],
                               [(q, 2.0 ** -75, 2.0 ** -75) for q in range(4)],
                               [(8 * q, 2.0 ** -75, 2.0 ** -75) for q in range(4)]]
        for name, probes in fams.items():
            res = run(fmt, K, probes)
            print(f"{name}:")
            for pr, v in zip(probes, res):
                d, ex = ulp_diff(v, pr)
                desc = " + ".join(f"{a * b:.3g}@k{k}" for k, a, b in pr)
                print(f"    {desc:60s} gpu {v!r:24s} exact {ex!r:24s} gpu-exact {d:+.4f} x 2^-23")


if __name__ == "__main__":
    main()
    fp8_main()
