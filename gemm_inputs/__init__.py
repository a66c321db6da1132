"""Seeded synthetic inputs for the mixed-precision GEMM, shared by the tests, the smoke
check and the benchmark.

This module holds no GEMM arithmetic: it only draws random numbers, rounds each draw once
(to nearest, ties to even) into its storage format, and lays the draws out as row-major
buffers with explicit leading dimensions.  Padding cells (between the logical row length
and the leading dimension) are filled with a sentinel -- a NaN pattern for floating formats,
0x7F for INT8 -- so that a kernel that reads padding into its result is caught.

Draws use numpy's PCG64 generator; the seed defaults to the workload's index, and the order
is always A, then B, then C.  Floating draws are made in float64 and rounded once to the
storage format (no double rounding through float32).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Optional

import numpy as np

STORAGE = {"f16": np.uint16, "bf16": np.uint16, "i8": np.int8, "f32": np.float32,
           "i32": np.int32, "e4m3": np.uint8, "e5m2": np.uint8}
ELEM_BYTES = {"f16": 2, "bf16": 2, "i8": 1, "f32": 4, "i32": 4, "e4m3": 1, "e5m2": 1}
PAD_SENTINEL = {"f16": 0x7E00, "bf16": 0x7FC0, "i8": 0x7F, "f32": np.float32(np.nan),
                "i32": 0x7F7F7F7F, "e4m3": 0x7F, "e5m2": 0x7E}    # NaN patterns


# ----------------------------------------------------------------------------- rounding
def f64_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> binary16 bit patterns, rounded once to nearest-even (numpy's direct
    double-to-half conversion)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit patterns, rounded once to nearest-even.

    The float64 significand is rounded to 8 significant bits with integer arithmetic on its
    bit pattern (ties to even); the result is then exactly representable in float32, whose
    upper half is the bfloat16 pattern.  Only finite values inside bfloat16's normal range
    (or zero) are accepted, which covers every distribution drawn here."""
    x = np.asarray(x, dtype=np.float64)
    bits = x.view(np.uint64)
    sign = bits & np.uint64(1 << 63)
    mag = bits & np.uint64((1 << 63) - 1)
    drop = np.uint64(45)                          # 52 - 7 fraction bits discarded
    lsb = (mag >> drop) & np.uint64(1)
    half_minus_one = np.uint64((1 << 44) - 1)
    rounded = ((mag + half_minus_one + lsb) >> drop) << drop
    y = (rounded | sign).view(np.float64)
    ay = np.abs(y)
    ok = (ay == 0) | ((ay >= 2.0 ** -126) & (ay < 2.0 ** 128))
    if not np.all(ok):
        raise ValueError("bf16 draw outside the normal range; widen the generator")
    return (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def f64_to_f32(x: np.ndarray) -> np.ndarray:
    """float64 -> float32, rounded once to nearest-even."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


# FP8 formats (OCP): E4M3 has 4 exponent bits (bias 7), 3 fraction bits, no infinities and
# S.1111.111 as NaN; E5M2 has 5 exponent bits (bias 15), 2 fraction bits, IEEE-style specials.
_FP8_FIELDS = {"e4m3": (4, 3, 7), "e5m2": (5, 2, 15)}


def _fp8_finite_table(fmt: str) -> tuple:
    """(values, codes) of the non-negative finite patterns of an FP8 format, ascending."""
    eb, mb, bias = _FP8_FIELDS[fmt]
    vals, codes = [], []
    for code in range(128):
        e, f = code >> mb, code & ((1 << mb) - 1)
        if fmt == "e5m2" and e == (1 << eb) - 1:
            continue                                   # Inf / NaN
        if fmt == "e4m3" and code == 0x7F:
            continue                                   # NaN
        v = (f / (1 << mb)) * 2.0 ** (1 - bias) if e == 0 else (1 + f / (1 << mb)) * 2.0 ** (e - bias)
        vals.append(v)
        codes.append(code)
    return np.array(vals), np.array(codes, dtype=np.uint8)


def f64_to_fp8_bits(x: np.ndarray, fmt: str) -> np.ndarray:
    """float64 -> FP8 patterns, rounded once to nearest with ties to the even pattern; beyond
    the largest finite value the result saturates to it (the draws stay inside the range)."""
    vals, codes = _fp8_finite_table(fmt)
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_hi, d_lo = np.abs(vals[hi] - a), np.abs(a - vals[lo])
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & ((codes[lo] & 1) == 0))
    c = np.where(pick_lo, codes[lo], codes[hi]).astype(np.uint8)
    c = np.where(np.signbit(x), c | 0x80, c).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), c).astype(np.uint8)


def to_storage(x64: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "f16":
        return f64_to_f16_bits(x64)
    if fmt == "bf16":
        return f64_to_bf16_bits(x64)
    if fmt == "f32":
        return f64_to_f32(x64)
    if fmt in _FP8_FIELDS:
        return f64_to_fp8_bits(x64, fmt)
    raise ValueError(fmt)


# ----------------------------------------------------------------------------- layout
def stored_shape(rows_op: int, cols_op: int, trans: bool) -> tuple:
    """Rows and columns of the stored buffer holding an op() of shape rows_op x cols_op."""
    return (cols_op, rows_op) if trans else (rows_op, cols_op)


def place(values: np.ndarray, ld: int, fmt: str) -> np.ndarray:
    """Put a rows x cols array into a rows x ld buffer; padding gets the sentinel."""
    rows, cols = values.shape
    if ld < cols:
        raise ValueError(f"ld={ld} < cols={cols}")
    buf = np.empty((rows, ld), dtype=STORAGE[fmt])
    if fmt in ("f16", "bf16", "i32"):
        buf.view(np.uint16 if fmt != "i32" else np.int32)[...] = PAD_SENTINEL[fmt]
    else:
        buf[...] = PAD_SENTINEL[fmt]
    buf[:, :cols] = values
    return buf


# ----------------------------------------------------------------------------- draws
def draw(rng: np.random.Generator, shape: tuple, dist: str, fmt: str) -> np.ndarray:
    """One operand's logical values in storage format.

    dist: 'uniform(lo,hi)' continuous, 'normal(mu,sigma)', 'int_uniform(lo,hi)' (inclusive
    integers), 'log_uniform(e0,e1)' (random sign, magnitude 2^u with u uniform in [e0, e1):
    values spread evenly over the binades), 'zeros', 'ones'."""
    name, _, rest = dist.partition("(")
    params = [float(p) for p in rest.rstrip(")").split(",")] if rest else []
    if name == "zeros":
        x = np.zeros(shape)
    elif name == "ones":
        x = np.ones(shape)
    elif name == "uniform":
        x = rng.uniform(params[0], params[1], size=shape)
    elif name == "normal":
        x = rng.normal(params[0], params[1], size=shape)
    elif name == "log_uniform":
        x = np.exp2(rng.uniform(params[0], params[1], size=shape)) * rng.choice([-1.0, 1.0], size=shape)
    elif name == "int_uniform":
        x = rng.integers(int(params[0]), int(params[1]) + 1, size=shape).astype(np.float64)
    else:
        raise ValueError(dist)
    if fmt == "i8":
        return x.astype(np.int8)
    if fmt == "i32":
        return x.astype(np.int32)
    return to_storage(x, fmt)


def padded_ld(cols: int, fmt: str) -> int:
    """Smallest leading dimension >= max(cols, 1) whose row size is a multiple of 16 bytes."""
    per = 16 // ELEM_BYTES[fmt]
    return ((max(cols, 1) + per - 1) // per) * per


@dataclass
class Workload:
    """A GEMM problem description plus the recipe of its synthetic inputs."""
    name: str
    in_type: str            # 'f16' | 'bf16' | 'i8' | 'f32' | 'e4m3' | 'e5m2' (A's type)
    out_type: str           # 'f32' | 'f16' | 'bf16' | 'i32'
    m: int
    n: int
    k: int
    transa: bool = False
    transb: bool = False
    alpha: float = 1.0
    beta: float = 0.0
    a_dist: str = "uniform(-1,1)"
    b_dist: str = "uniform(-1,1)"
    c_dist: str = "zeros"
    lda: Optional[int] = None
    ldb: Optional[int] = None
    ldc: Optional[int] = None
    seed: int = 0
    note: str = ""
    b_type: Optional[str] = None   # B's type when it differs from A's (FP8 pairs)
    sparse24: bool = False         # A 2:4 structured-sparse: A holds the kept values (m x k/2)
    ld_meta: Optional[int] = None  # bytes per row of the 2:4 metadata

    def __post_init__(self):
        self.b_type = self.in_type if self.b_type is None else self.b_type
        if self.sparse24:
            self.lda = padded_ld(self.k // 2, self.in_type) if self.lda is None else self.lda
            self.ld_meta = ((max(self.k // 8, 1) + 15) // 16) * 16 if self.ld_meta is None else self.ld_meta
        # default leading dimensions: the row length rounded up to a 16-byte multiple (and at
        # least one element), the library's alignment contract
        ra, ca = stored_shape(self.m, self.k, self.transa)
        rb, cb = stored_shape(self.k, self.n, self.transb)
        self.lda = padded_ld(ca, self.in_type) if self.lda is None else self.lda
        self.ldb = padded_ld(cb, self.b_type) if self.ldb is None else self.ldb
        self.ldc = padded_ld(self.n, self.out_type) if self.ldc is None else self.ldc

    @property
    def flops(self) -> int:
        """Multiply-adds the product needs, two flops each (a 2:4 sparse A: the kept ones)."""
        return 2 * self.m * self.n * (self.k // 2 if self.sparse24 else self.k)

    @property
    def compulsory_bytes(self) -> int:
        """Each input read once, D written once, C read once when beta != 0 (a 2:4 sparse A:
        its kept values and metadata)."""
        es, eb, eo = ELEM_BYTES[self.in_type], ELEM_BYTES[self.b_type], ELEM_BYTES[self.out_type]
        a = (self.m * (self.k // 2) * es + self.m * (self.k // 8) if self.sparse24
             else self.m * self.k * es)
        b = a + self.k * self.n * eb + self.m * self.n * eo
        if self.beta != 0:
            b += self.m * self.n * eo
        return b


@dataclass
class Inputs:
    w: Workload
    A: np.ndarray
    B: np.ndarray
    C: Optional[np.ndarray]   # stored m x ldc in out_type, or None when beta == 0
    meta: Optional[np.ndarray] = None   # 2:4 metadata, m x ld_meta bytes (sparse A only)

    @property
    def transa(self):
        return self.w.transa

    @property
    def transb(self):
        return self.w.transb


def generate(w: Workload, seed: Optional[int] = None, c_when_beta_zero: bool = False) -> Inputs:
    """Draw A, then B, then C for ``w`` with PCG64(seed) (default: w.seed)."""
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    if w.sparse24:
        return _generate_sp24(w, rng, c_when_beta_zero)
    ra, ca = stored_shape(w.m, w.k, w.transa)
    rb, cb = stored_shape(w.k, w.n, w.transb)
    A = place(draw(rng, (ra, ca), w.a_dist, w.in_type), w.lda, w.in_type)
    B = place(draw(rng, (rb, cb), w.b_dist, w.b_type), w.ldb, w.b_type)
    C = None
    if w.beta != 0 or c_when_beta_zero:
        C = place(draw(rng, (w.m, w.n), w.c_dist, w.out_type), w.ldc, w.out_type)
    return Inputs(w, A, B, C)


# ----------------------------------------------------------------------------- workloads
# The five workloads of the headline measurement, with their published shapes and value
# distributions.  Storage is row-major; trans=True means the buffer holds op()^T.
WORKLOADS = {
    "f16_256_nn_beta1": Workload(
        "f16_256_nn_beta1", "f16", "f32", 256, 256, 256, alpha=1.0, beta=1.0,
        a_dist="uniform(-1,1)", b_dist="uniform(-1,1)", c_dist="uniform(-1,1)", seed=0,
        note="FP16 256^3 row-major, C fp32 U[-1,1], alpha=beta=1"),
    "f16_4096_nt": Workload(
        "f16_4096_nt", "f16", "f32", 4096, 4096, 4096, transb=True, alpha=1.0, beta=0.0,
        a_dist="normal(0,1)", b_dist="normal(0,1)", seed=1,
        note="FP16 4096^3, A row-major, B column-major (transb=T), beta=0, fp32 out"),
    "bf16_8192_nn": Workload(
        "bf16_8192_nn", "bf16", "f32", 8192, 8192, 8192, alpha=1.0, beta=0.5,
        a_dist="normal(0,0.5)", b_dist="normal(0,0.5)", c_dist="normal(0,1)", seed=2,
        note="BF16 8192^3 row-major, C fp32 N(0,1), alpha=1, beta=0.5"),
    "i8_4096_nn": Workload(
        "i8_4096_nn", "i8", "i32", 4096, 4096, 4096, alpha=1, beta=0,
        a_dist="int_uniform(-128,127)", b_dist="int_uniform(-128,127)", c_dist="zeros",
        seed=3, note="INT8 4096^3 row-major, int32 accumulate/output, C = 0"),
    "f16_5000x3000x1000_f16out": Workload(
        "f16_5000x3000x1000_f16out", "f16", "f16", 5000, 3000, 1000, alpha=1.0, beta=0.0,
        a_dist="uniform(-2,2)", b_dist="uniform(-2,2)", seed=4,
        note="FP16 ragged 5000x3000x1000, fp16 output rounded RNE from fp32"),
}

# The INT8 workload with beta = 1: C (zeros, 64 MiB of INT32) is read and added.
WORKLOADS["i8_4096_nn_beta1"] = Workload(
    "i8_4096_nn_beta1", "i8", "i32", 4096, 4096, 4096, alpha=1, beta=1,
    a_dist="int_uniform(-128,127)", b_dist="int_uniform(-128,127)", c_dist="zeros", seed=3,
    note="INT8 4096^3 row-major as above, alpha = beta = 1: C = 0 read and added")

# The same ragged workload with genuinely padded leading dimensions.
WORKLOADS["f16_5000x3000x1000_f16out_padded"] = Workload(
    "f16_5000x3000x1000_f16out_padded", "f16", "f16", 5000, 3000, 1000, alpha=1.0, beta=0.0,
    a_dist="uniform(-2,2)", b_dist="uniform(-2,2)", lda=1008, ldb=3008, ldc=3008, seed=4,
    note="as above with lda=1008, ldb=ldc=3008")


# Workloads of the extensions beyond the five configurations, on the same 4096^3 NT shape as
# the FP16 benchmark workload: FP32 operands multiplied as three BF16 products, FP8 inputs.
NEXT_WORKLOADS = {
    "f32_4096_nt_bf16x3": Workload(
        "f32_4096_nt_bf16x3", "f32", "f32", 4096, 4096, 4096, transb=True, alpha=1.0, beta=0.0,
        a_dist="normal(0,1)", b_dist="normal(0,1)", seed=6,
        note="FP32 4096^3, B stored n x k, as three BF16 products with FP32 accumulation"),
    "f16_sp24_4096_nt": Workload(
        "f16_sp24_4096_nt", "f16", "f32", 4096, 4096, 4096, transb=True, alpha=1.0, beta=0.0,
        a_dist="normal(0,1)", b_dist="normal(0,1)", seed=10, sparse24=True,
        note="FP16 4096^3 with a 2:4 sparse A (kept values 4096 x 2048), B stored n x k"),
    "i8_sp24_4096_nn": Workload(
        "i8_sp24_4096_nn", "i8", "i32", 4096, 4096, 4096, alpha=1.0, beta=0.0,
        a_dist="int_uniform(-128,127)", b_dist="int_uniform(-128,127)", seed=12, sparse24=True,
        note="INT8 4096^3 with a 2:4 sparse A (kept values 4096 x 2048), B row-major k x n"),
    "e4m3_sp24_4096_nt": Workload(
        "e4m3_sp24_4096_nt", "e4m3", "f32", 4096, 4096, 4096, transb=True, alpha=1.0, beta=0.0,
        a_dist="normal(0,1)", b_dist="normal(0,1)", seed=14, sparse24=True,
        note="E4M3 4096^3 with a 2:4 sparse A (kept values 4096 x 2048), B stored n x k"),
    "e4m3_4096_nt": Workload(
        "e4m3_4096_nt", "e4m3", "f32", 4096, 4096, 4096, transb=True, alpha=1.0, beta=0.0,
        a_dist="normal(0,1)", b_dist="normal(0,1)", seed=8,
        note="FP8 E4M3 4096^3, B stored n x k, FP32 accumulation and output"),
}


# The six ways to keep two of four positions, in increasing order.
SP24_PAIRS = ((0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3))


def pack_sp24_meta(idx: np.ndarray, ld_meta: int) -> np.ndarray:
    """2-bit indices (m x k/2, values 0..3, in k order) -> m x ld_meta metadata bytes: index j
    of a row in bits 2 (j % 4) .. +1 of byte j / 4; padding bytes 0xFF."""
    m, kh = idx.shape
    meta = np.full((m, ld_meta), 0xFF, np.uint8)
    q = idx.astype(np.uint8).reshape(m, kh // 4, 4)
    meta[:, : kh // 4] = q[..., 0] | (q[..., 1] << 2) | (q[..., 2] << 4) | (q[..., 3] << 6)
    return meta


def _generate_sp24(w: "Workload", rng, c_when_beta_zero: bool) -> "Inputs":
    """A 2:4 sparse A: per group of 4 consecutive k one of the six position pairs (uniform),
    then the kept values from a_dist (m x k/2), then B and C as usual."""
    assert not w.transa and w.k % 4 == 0
    pairs = np.array(SP24_PAIRS, dtype=np.uint8)[rng.integers(0, 6, size=(w.m, w.k // 4))]
    idx = pairs.reshape(w.m, w.k // 2)
    A = place(draw(rng, (w.m, w.k // 2), w.a_dist, w.in_type), w.lda, w.in_type)
    rb, cb = stored_shape(w.k, w.n, w.transb)
    B = place(draw(rng, (rb, cb), w.b_dist, w.b_type), w.ldb, w.b_type)
    C = None
    if w.beta != 0 or c_when_beta_zero:
        C = place(draw(rng, (w.m, w.n), w.c_dist, w.out_type), w.ldc, w.out_type)
    return Inputs(w, A, B, C, meta=pack_sp24_meta(idx, w.ld_meta))


def sample_points(m: int, n: int, count: int, seed: int = 12345) -> tuple:
    """Output coordinates for sampled checks: the four corners, the last row and column,
    and ``count`` uniformly drawn points."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ii = [0, 0, m - 1, m - 1]
    jj = [0, n - 1, 0, n - 1]
    edge = min(64, n)
    ii += [m - 1] * edge
    jj += list(np.linspace(0, n - 1, edge).astype(np.int64))
    edge = min(64, m)
    ii += list(np.linspace(0, m - 1, edge).astype(np.int64))
    jj += [n - 1] * edge
    ii = np.concatenate([np.array(ii, np.int64), rng.integers(0, m, count)])
    jj = np.concatenate([np.array(jj, np.int64), rng.integers(0, n, count)])
    return ii, jj
