"""GPU parity: the HIP path through the C-ABI against the CPU oracle on the same seeded
inputs.  INT8 and exactly representable FP cases must match bit for bit; other FP results
must sit inside the FP32 accumulation bound of the oracle's comparator."""
import ctypes
import os

import numpy as np
import pytest
import torch

from gemm_inputs import WORKLOADS, Workload, generate, place, sample_points
import mixed_precision_dense_amd as mp
import oracle
from tests.gpu_harness import check_case, compare, handle, run_gpu, say

pytestmark = pytest.mark.gpu

LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]


def _assert(rep, res=None):
    assert rep.ok, f"{rep.n_bad}/{rep.n} bad; worst ratio {rep.worst_ratio:.3g}; {rep.detail}"
    if res is not None:
        assert res.guard_ok, "D guard band or ld padding was overwritten"


# ----------------------------------------------------------------------------- closed forms
@pytest.mark.parametrize("in_type", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_identity_times_b_is_b(in_type, ta, tb):
    m = n = k = 96 if in_type != "i8" else 160
    out = "i32" if in_type == "i8" else "f32"
    w = Workload(f"identity_{in_type}", in_type, out, m, n, k, transa=ta, transb=tb,
                 a_dist="zeros", b_dist="int_uniform(-100,100)" if in_type == "i8" else "uniform(-4,4)",
                 seed=40)
    inp = generate(w)
    eye = np.eye(k)
    if in_type == "i8":
        inp.A[:, :k] = eye.astype(np.int8)
    else:
        from gemm_inputs import to_storage
        inp.A[:, :k] = to_storage(eye, in_type)                # symmetric: same for ta
    rep, res = check_case(w, exact=True, inp=inp)
    _assert(rep, res)


@pytest.mark.parametrize("k", [1, 7, 64, 1000, 2049, 2051])
def test_all_ones_gives_k_exactly(k):
    # FP16 output: K = 2049 and 2051 are RNE ties at FP16 precision (2048 and 2052)
    w = Workload(f"ones_k{k}", "f16", "f16", 40, 72, k, a_dist="ones", b_dist="ones", seed=41)
    rep, res = check_case(w, exact=True)
    _assert(rep, res)


@pytest.mark.parametrize("ta,tb", [(False, False), (True, True)])
def test_k1_fp16_exhaustive_products(ta, tb):
    """Every FP16 pattern times a set of B values, K = 1 (the k tail masks 7 padding NaNs per
    row): each product is exact in FP32, so D must equal the oracle bit for bit, subnormal
    inputs included."""
    bvals = np.array([1.0, -1.0, 0.5, 1.5, 2.0 ** -10, 2.0 ** -14, 2.0 ** -24, 3 * 2.0 ** -24,
                      65504.0, -65504.0, 0.0, 1000.0, 0.333251953125, 7.0, -3.25, 2.0 ** 15])
    w = Workload("k1_f16_all", "f16", "f32", 65536, bvals.size, 1, transa=ta, transb=tb, seed=60)
    inp = generate(w)
    patterns = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if ta:
        inp.A[0, :65536] = patterns
    else:
        inp.A[:, 0] = patterns
    from gemm_inputs import f64_to_f16_bits
    bbits = f64_to_f16_bits(bvals)
    if tb:
        inp.B[:, 0] = bbits
    else:
        inp.B[0, : bvals.size] = bbits
    rep, res = check_case(w, exact=True, inp=inp)
    _assert(rep, res)


def test_k1_int8_product_table():
    w = Workload("k1_i8_table", "i8", "i32", 256, 256, 1, a_dist="zeros", b_dist="zeros", seed=61)
    inp = generate(w)
    vals = np.arange(-128, 128).astype(np.int8)
    inp.A[:, 0] = vals
    inp.B[0, :256] = vals
    rep, res = check_case(w, exact=True, inp=inp)
    _assert(rep, res)


# ----------------------------------------------------------------------------- ragged sweep
RAGGED = [1, 2, 7, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


@pytest.mark.parametrize("in_type", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_ragged_sweep_exact(in_type, ta, tb):
    """Integer-valued inputs (exact in FP32 accumulation) over ragged m, n, k; padded ld."""
    rng = np.random.default_rng(hash((in_type, ta, tb)) % 2 ** 32)
    out = {"f16": "f32", "bf16": "f32", "i8": "i32"}[in_type]
    align = 16 if in_type == "i8" else 8
    for t in range(14):
        m, n, k = (int(x) for x in rng.choice(RAGGED, 3))
        if t == 0:
            m, n, k = 257, 255, 129
        pad = lambda v: ((v + align - 1) // align) * align + align * int(rng.integers(0, 2))
        lda = pad(m if ta else k)
        ldb = pad(k if tb else n)
        ldc = ((n + 3) // 4) * 4 + 4 * int(rng.integers(0, 2))
        dist = "int_uniform(-128,127)" if in_type == "i8" else "int_uniform(-8,8)"
        beta = float(rng.choice([0.0, 1.0, -2.0]))
        w = Workload(f"ragged_{in_type}", in_type, out, m, n, k, transa=ta, transb=tb,
                     alpha=float(rng.choice([1.0, 2.0, -0.5])) if in_type != "i8" else int(rng.choice([1, 3, -2])),
                     beta=beta if in_type != "i8" else int(beta),
                     a_dist=dist, b_dist=dist, c_dist="int_uniform(-50,50)",
                     lda=lda, ldb=ldb, ldc=ldc, seed=1000 + t)
        rep, res = check_case(w, exact=True)
        _assert(rep, res)


# Tile-edge cases.  Shapes are chosen for the kernel's edge handling: 256 x 256 tiles (at
# least 192 of them) whose last tile row and column are ragged, K stages ending in a partial
# stage and odd stage counts, leading dimensions equal to the row length (what lies past K in
# a row is the next row's data, not padding), very short rows of a transposed-read operand,
# and tiny outputs.  Inputs are integer-valued, so every result is exact.
EDGE_K = {"f16": (200, 136), "bf16": (200, 136), "i8": (208, 272)}   # stage tails; odd counts


@pytest.mark.parametrize("in_type", ["f16", "bf16", "i8"])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_tile_edges_exact(in_type, ta, tb):
    out = "i32" if in_type == "i8" else "f32"
    dist = "int_uniform(-128,127)" if in_type == "i8" else "int_uniform(-8,8)"
    k1, k2 = EDGE_K[in_type]
    shapes = [(256 * 14 + 37, 256 * 14 + 5, k1), (256 * 15 + 255, 256 * 13 + 1, k2),
              (5, 3, k1), (300, 9, k2), (17, 260, 320), (1, 1, 1), (2, 513, 48), (257, 1, 4112)]
    for t, (m, n, k) in enumerate(shapes):
        w = Workload(f"edge_{in_type}", in_type, out, m, n, k, transa=ta, transb=tb,
                     a_dist=dist, b_dist=dist, seed=3000 + t)
        say(f"  edge case {in_type} ta={ta} tb={tb} m={m} n={n} k={k} lda={w.lda} ldb={w.ldb}")
        rep, res = check_case(w, exact=True)
        _assert(rep, res)


@pytest.mark.parametrize("in_type,out_type", [("f16", "f32"), ("f16", "f16"), ("bf16", "f32"),
                                              ("bf16", "bf16")])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_random_within_bound(in_type, out_type, ta, tb):
    """Normal-distributed inputs over shapes spanning several tiles with ragged tails."""
    for (m, n, k) in [(300, 200, 333), (513, 771, 1000), (64, 64, 4095)]:
        w = Workload(f"rand_{in_type}_{out_type}", in_type, out_type, m, n, k, transa=ta,
                     transb=tb, alpha=1.0, beta=0.5, a_dist="normal(0,1)", b_dist="normal(0,1)",
                     c_dist="normal(0,1)", seed=7 + m)
        rep, res = check_case(w)
        _assert(rep, res)


# ----------------------------------------------------------------------------- the five workloads
# Each configuration's whole output is compared with the oracle element by element (the
# oracle's full pass takes about 2 s at 4096^3 and 20 s at 8192^3 on 16 host cores), and each
# shape also runs once on integer-valued inputs, where every partial sum is exact in FP32 and
# the output must equal the oracle bit for bit.
def _int_valued(w, a_dist="int_uniform(-2,2)", c_dist=None, seed=None):
    return Workload(w.name + "_int", w.in_type, w.out_type, w.m, w.n, w.k, transa=w.transa,
                    transb=w.transb, alpha=w.alpha, beta=w.beta, a_dist=a_dist, b_dist=a_dist,
                    c_dist=c_dist or w.c_dist, lda=w.lda, ldb=w.ldb, ldc=w.ldc,
                    seed=w.seed if seed is None else seed)


def test_workload_fp16_256_nn_beta1_full():
    rep, res = check_case(WORKLOADS["f16_256_nn_beta1"])
    _assert(rep, res)
    say(f"  worst error / bound = {rep.worst_ratio:.4f}")


def test_workload_fp16_256_nn_beta1_exact_integer_valued():
    w = _int_valued(WORKLOADS["f16_256_nn_beta1"], "int_uniform(-8,8)", "int_uniform(-100,100)")
    rep, res = check_case(w, exact=True)
    _assert(rep, res)


def test_workload_fp16_4096_nt_full():
    rep, res = check_case(WORKLOADS["f16_4096_nt"])
    _assert(rep, res)
    say(f"  worst error / bound = {rep.worst_ratio:.4f}")


def test_workload_fp16_4096_nt_exact_integer_valued():
    rep, res = check_case(_int_valued(WORKLOADS["f16_4096_nt"]), exact=True)
    _assert(rep, res)


def test_workload_bf16_8192_nn_full():
    rep, res = check_case(WORKLOADS["bf16_8192_nn"])
    _assert(rep, res)
    say(f"  worst error / bound = {rep.worst_ratio:.4f}")


def test_workload_bf16_8192_nn_exact_integer_valued():
    """Integers in [-2, 2] for A and B and in [-64, 64] for C with beta = 0.5: |sum| <= 2^15
    and beta * c is exact, so every partial sum and the epilogue are exact in FP32."""
    w = _int_valued(WORKLOADS["bf16_8192_nn"], "int_uniform(-2,2)", "int_uniform(-64,64)")
    rep, res = check_case(w, exact=True)
    _assert(rep, res)


def test_workload_int8_4096_nn_full_and_in_place_beta1():
    w = WORKLOADS["i8_4096_nn"]
    rep, res = check_case(w)
    _assert(rep, res)
    # beta = 1 with C = 0 and D written over C in place: identical bits
    w1 = WORKLOADS["i8_4096_nn_beta1"]
    assert (w1.a_dist, w1.b_dist, w1.seed, w1.c_dist) == (w.a_dist, w.b_dist, w.seed, "zeros")
    inp1 = generate(w1)
    res1 = run_gpu(inp1, in_place=True)
    assert np.array_equal(res1.D[:, : w.n], res.D[:, : w.n])
    assert res1.guard_ok


@pytest.mark.parametrize("name", ["f16_5000x3000x1000_f16out", "f16_5000x3000x1000_f16out_padded"])
def test_workload_fp16_ragged_f16out_full(name):
    rep, res = check_case(WORKLOADS[name])
    _assert(rep, res)
    say(f"  {name}: worst error / bound = {rep.worst_ratio:.4f}")


@pytest.mark.parametrize("name", ["f16_5000x3000x1000_f16out", "f16_5000x3000x1000_f16out_padded"])
def test_workload_fp16_ragged_exact_full(name):
    rep, res = check_case(_int_valued(WORKLOADS[name], seed=5), exact=True)
    _assert(rep, res)


# ----------------------------------------------------------------------------- special values
def test_nan_inf_propagation_and_beta_zero_ignores_c():
    w = Workload("special", "f16", "f32", 70, 90, 130, beta=0.0, a_dist="uniform(-1,1)",
                 b_dist="uniform(-1,1)", seed=50)
    inp = generate(w, c_when_beta_zero=True)
    inp.A[3, 5] = 0x7E00       # NaN: row 3 all NaN
    inp.A[10, :] = 0           # row 10: zero times inf below -> NaN where B has inf
    inp.B[7, 11] = 0x7C00      # +inf in column 11
    inp.A[20, :] = 0x3C00      # row 20 all ones -> +inf in column 11
    inp.B[:, 11] = np.where(np.arange(w.k) == 7, 0x7C00, 0x3C00)
    inp.C[...] = np.float32(np.nan)  # never read with beta = 0
    res = run_gpu(inp)
    rep = compare(inp, res)
    _assert(rep, res)
    D = res.D[:, : w.n]
    assert np.all(np.isnan(D[3])) and np.isnan(D[10, 11]) and D[20, 11] == np.inf
    assert np.isfinite(np.delete(D[0], 11)).all()


def test_k_zero_gives_beta_c():
    w = Workload("k0", "f16", "f32", 33, 65, 0, alpha=1.0, beta=2.0, c_dist="uniform(-1,1)", seed=51)
    rep, res = check_case(w, exact=True)
    _assert(rep, res)
    w = Workload("k0b0", "bf16", "bf16", 33, 65, 0, alpha=1.0, beta=0.0, seed=52)
    rep, res = check_case(w, exact=True)
    _assert(rep, res)


def test_in_place_d_equals_c():
    w = Workload("inplace", "bf16", "f32", 300, 260, 200, alpha=1.0, beta=0.5, ldc=264,
                 a_dist="normal(0,1)", b_dist="normal(0,1)", c_dist="normal(0,1)", seed=53)
    rep, res = check_case(w, in_place=True)
    _assert(rep, res)


def test_page_accumulator_vector_within_bound():
    """The numerics page's K = 3 vector (section 2.2.1) through the GPU: within the bound."""
    w = Workload("p4vec", "f16", "f32", 1, 1, 3, seed=54)
    inp = generate(w)
    inp.A[0, :3] = [0x3E00, 0x0002, 0x0001]      # 1.5, 2^-23, 2^-24 (FP16 subnormals)
    inp.B[:3, 0] = [0x3E00, 0x3C00, 0x3C00]      # 1.5, 1, 1
    res = run_gpu(inp)
    rep = compare(inp, res)
    _assert(rep, res)


def test_determinism_bitwise():
    w = Workload("det", "f16", "f32", 1000, 1000, 2000, transb=True, a_dist="normal(0,1)",
                 b_dist="normal(0,1)", seed=55)
    inp = generate(w)
    first = run_gpu(inp).D.copy()
    for _ in range(3):
        again = run_gpu(inp, repeat=3).D
        assert np.array_equal(first.view(np.uint32), again.view(np.uint32))


def test_error_left_pending_by_the_caller_does_not_fail_the_launch():
    """A HIP error the caller left pending on the thread (here from hipSetDevice on a device
    that does not exist) is neither returned as the launch's status nor stops the GEMM."""
    hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD)   # the runtime already loaded
    w = Workload("pending", "f16", "f32", 100, 72, 64, a_dist="normal(0,1)",
                 b_dist="normal(0,1)", seed=56)
    inp = generate(w)
    want = run_gpu(inp).D
    dA = mp.device_buffer(inp.A, "f16")
    dB = mp.device_buffer(inp.B, "f16")
    dD = torch.zeros(w.m * w.ldc, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    assert hip.hipSetDevice(ctypes.c_int(1 << 20)) != 0
    try:
        st = mp.mpgemm_run(handle().h, w.transa, w.transb, w.m, w.n, w.k, w.alpha, dA, "f16",
                           w.lda, dB, "f16", w.ldb, w.beta, None, "f32", w.ldc, dD, "f32",
                           check=False)
    finally:
        hip.hipGetLastError()   # leave nothing pending for torch's own launch checks
    assert st == mp.SUCCESS
    torch.cuda.synchronize()
    got = dD.cpu().numpy().reshape(w.m, w.ldc)
    assert np.array_equal(got[:, :w.n].view(np.uint32), want[:, :w.n].view(np.uint32))


@pytest.mark.parametrize("in_type,out_type", [("f16", "f32"), ("i8", "i32")])
def test_largest_accepted_strides_mn_contiguous(in_type, out_type):
    """A stored k x m and B stored k x n at the largest leading dimension the argument check
    accepts (256 rows just under 2 GiB), on 256 x 256 tiles: every offset of the 32-bit buffer
    addressing within a stage stays in range (exact small integers, the whole output)."""
    eb = 2 if in_type == "f16" else 1
    ld = ((1 << 31) - 4096) // (256 * eb)
    assert (ld * eb) % 16 == 0
    w = Workload(f"maxld_{in_type}", in_type, out_type, 4096, 3072, 128, transa=True,
                 lda=ld, ldb=ld, a_dist="int_uniform(-3,3)", b_dist="int_uniform(-3,3)",
                 seed=57)
    rep, res = check_case(w, exact=True)
    _assert(rep, res)


@pytest.mark.parametrize("dist,exact", [("int_uniform(-3,3)", True), ("normal(0,1)", False)])
def test_column_major_caller_through_the_operand_swap(dist, exact):
    """A column-major caller (the CUDA 9 page's cuBLAS example: lda = M, ldb = K, ldc = M)
    obtains D^T = op(B)^T op(A)^T by passing (transb, transa, n, m, k, B, ldb, A, lda).  Read
    back column-major, D matches the oracle evaluated on the column-major operands directly
    (through its transposed-storage flags, without the swap)."""
    from gemm_inputs import draw
    M, N, K = 304, 200, 136
    rng = np.random.Generator(np.random.PCG64(59))
    Acm = draw(rng, (K, M), dist, "f16")           # M x K, column-major: a(i, p) = Acm[p, i]
    Bcm = draw(rng, (N, K), dist, "f16")           # K x N, column-major: b(p, j) = Bcm[j, p]
    Ccm = draw(rng, (N, M), dist, "f32")           # M x N, column-major: c(i, j) = Ccm[j, i]
    alpha, beta = 1.0, 0.5
    say(f"[gpu case] column-major caller M={M} N={N} K={K} {dist}")
    dA = mp.device_buffer(Acm, "f16")
    dB = mp.device_buffer(Bcm, "f16")
    dC = mp.device_buffer(Ccm, "f32")
    dD = torch.empty(N * M * 4, dtype=torch.uint8, device="cuda")
    mp.mpgemm_run(handle().h, False, False, N, M, K, alpha, dB, "f16", K, dA, "f16", M, beta,
                  dC, "f32", M, dD, "f32")
    torch.cuda.synchronize()
    D = dD.cpu().numpy().view(np.float32).reshape(N, M).T      # back to M x N
    ref = oracle.gemm_fp(True, True, M, N, K, alpha, Acm, "f16", M, Bcm, "f16", K, beta,
                         np.ascontiguousarray(Ccm.T), "f32", N)
    rep = oracle.check_fp(np.ascontiguousarray(D), "f32", ref, K, alpha, exact=exact)
    assert rep.ok, f"{rep.n_bad}/{rep.n} bad; {rep.detail}"


@pytest.mark.parametrize("n", [2560, 3072])
def test_shapes_on_one_partial_round_of_large_tiles(n):
    """Squares that the tile rule puts on one round of 256 x 256 tiles with part of the chip
    idle (100 and 144 workgroups): exact integer inputs, the whole output against the oracle."""
    assert mp.mpgemm_tile_shape(n, n, "f16") == (256, 256)
    w = Workload(f"round_{n}", "f16", "f32", n, n, n, transb=True, a_dist="int_uniform(-2,2)",
                 b_dist="int_uniform(-2,2)", seed=60)
    rep, res = check_case(w, exact=True)
    _assert(rep, res)


@pytest.mark.parametrize("m,n,tile", [(4096, 8192, 256), (8192, 4096, 256), (12288, 4096, 256),
                                      (2048, 2048, 128)])
def test_tile_grids_of_whole_16_by_16_regions(m, n, tile):
    """Tile grids whose sides are multiples of 16 tiles (several rounds of 16 x 16-tile regions
    taken in a serpentine, or one region of smaller tiles): every tile written once, exactly."""
    assert mp.mpgemm_tile_shape(m, n, "bf16") == (tile, tile)
    w = Workload(f"regions_{m}x{n}", "bf16", "f32", m, n, 160, a_dist="int_uniform(-2,2)",
                 b_dist="int_uniform(-2,2)", beta=0.5, c_dist="int_uniform(-4,4)", seed=61)
    rep, res = check_case(w, exact=True)
    _assert(rep, res)


@pytest.mark.parametrize("entry", ["mpgemm_run", "mpgemm_run_sp24", "mpgemm_run_bf16x3"])
def test_captured_in_a_graph_every_replay_matches_eager(entry):
    """Each entry point queued under HIP graph capture (torch.cuda.graph): the calls make no
    allocation, memset or synchronisation (the three-product GEMM's workspace is the caller's),
    so the captured launches replay.  Each replay, with eager work and synchronisations between
    them, reproduces the eager result bit for bit."""
    h = handle().h
    if entry == "mpgemm_run_sp24":
        w = Workload("graph_sp", "f16", "f32", 256, 256, 256, transb=True, sparse24=True,
                     alpha=1.0, beta=1.0, a_dist="uniform(-1,1)", b_dist="uniform(-1,1)",
                     c_dist="uniform(-1,1)", seed=62)
        inp = generate(w)
        dA, dM = mp.device_buffer(inp.A, "f16"), mp.device_buffer(inp.meta, "i8")
        dB, dC = mp.device_buffer(inp.B, "f16"), mp.device_buffer(inp.C, "f32")
        dD = torch.empty(w.m * w.ldc, dtype=torch.float32, device="cuda")

        def call():
            mp.mpgemm_run_sp24(h, w.transb, w.m, w.n, w.k, w.alpha, dA, "f16", w.lda, dM,
                               w.ld_meta, dB, "f16", w.ldb, w.beta, dC, "f32", w.ldc, dD, "f32")
    elif entry == "mpgemm_run_bf16x3":
        w = Workload("graph_3", "f32", "f32", 256, 256, 256, alpha=1.0, beta=1.0,
                     a_dist="normal(0,1)", b_dist="normal(0,1)", c_dist="normal(0,1)", seed=63)
        inp = generate(w)
        dA, dB, dC = (mp.device_buffer(x, "f32") for x in (inp.A, inp.B, inp.C))
        dD = torch.empty(w.m * w.ldc, dtype=torch.float32, device="cuda")
        need = mp.mpgemm_bf16x3_workspace_size(False, False, w.m, w.n, w.k)
        ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
        ws_ptr = (ws.data_ptr() + 255) // 256 * 256

        def call():
            mp.mpgemm_run_bf16x3(h, False, False, w.m, w.n, w.k, w.alpha, dA, w.lda, dB, w.ldb,
                                 w.beta, dC, w.ldc, dD, ws_ptr, need)
    else:
        w = Workload("graph", "f16", "f32", 256, 256, 256, alpha=1.0, beta=1.0,
                     a_dist="uniform(-1,1)", b_dist="uniform(-1,1)", c_dist="uniform(-1,1)",
                     seed=61)
        inp = generate(w)
        dA, dB = mp.device_buffer(inp.A, "f16"), mp.device_buffer(inp.B, "f16")
        dC = mp.device_buffer(inp.C, "f32")
        dD = torch.empty(w.m * w.ldc, dtype=torch.float32, device="cuda")

        def call():
            mp.mpgemm_run(h, False, False, w.m, w.n, w.k, w.alpha, dA, "f16", w.lda, dB, "f16",
                          w.ldb, w.beta, dC, "f32", w.ldc, dD, "f32")

    call()
    torch.cuda.synchronize()
    want = dD.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):      # a first call on a side stream before capture
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for _ in range(4):
        dD.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(dD.view(torch.int32), want.view(torch.int32))
    say(f"[gpu case] graph capture of {entry}: 4 replays bit-identical to the eager call")


@pytest.mark.parametrize("in_type,out_type", [("f16", "f32"), ("bf16", "bf16")])
def test_line_alignment_of_c_and_d_changes_no_bit(in_type, out_type):
    """Whole tiles: C and D stream past the caches only when the row pitch and both pointers
    lie on 128-byte lines, otherwise they take the default cache policy.  C and D placed on a
    line or 16, 48 or 80 bytes past one give the same bits, equal to the block-FMA model, and
    leave the bytes around D untouched."""
    from tests.gpu_harness import GUARD_ROWS, SENTINEL, GpuResult, compare_model
    w = Workload(f"align_{in_type}_{out_type}", in_type, out_type, 512, 768, 320, beta=0.5,
                 alpha=1.5, a_dist="normal(0,1)", b_dist="normal(0,1)", c_dist="normal(0,1)",
                 seed=91)
    inp = generate(w)
    ob = np.dtype(np.float32 if out_type == "f32" else np.uint16).itemsize
    nbytes = w.m * w.ldc * ob
    guard = GUARD_ROWS * w.ldc * ob
    assert (w.ldc * ob) % 128 == 0                       # the row pitch itself is whole lines
    dA, dB = mp.device_buffer(inp.A, in_type), mp.device_buffer(inp.B, in_type)
    c_bytes = torch.from_numpy(np.ascontiguousarray(inp.C).view(np.uint8).reshape(-1))
    first = None
    for c_off, d_off in [(0, 0), (16, 0), (0, 16), (48, 80)]:
        say(f"[gpu case] {w.name} m={w.m} n={w.n} k={w.k} C at line + {c_off} B, "
            f"D at line + {d_off} B")
        craw = torch.zeros(nbytes + 256, dtype=torch.uint8, device="cuda")
        cs = (-craw.data_ptr()) % 128 + c_off
        craw[cs: cs + nbytes].copy_(c_bytes)
        draw = torch.full((nbytes + guard + 512,), SENTINEL, dtype=torch.uint8, device="cuda")
        ds = (-draw.data_ptr()) % 128 + 128 + d_off       # 128 or more sentinel bytes before D
        mp.mpgemm_run(handle().h, w.transa, w.transb, w.m, w.n, w.k, w.alpha, dA, in_type,
                      w.lda, dB, in_type, w.ldb, w.beta, craw.data_ptr() + cs, out_type, w.ldc,
                      draw.data_ptr() + ds, "f32")
        torch.cuda.synchronize()
        raw = draw.cpu().numpy()
        assert np.all(raw[:ds] == SENTINEL) and np.all(raw[ds + nbytes:] == SENTINEL)
        assert np.array_equal(craw[cs: cs + nbytes].cpu(), c_bytes)   # C is only read
        D = raw[ds: ds + nbytes].copy()
        if first is None:
            first = D
            storage = np.float32 if out_type == "f32" else np.uint16
            res = GpuResult(D=D.view(storage).reshape(w.m, w.ldc), guard_ok=True)
            rep = compare_model(inp, res)
            assert rep.ok, f"{rep.n_bad}/{rep.n} differ from the model; {rep.detail}"
        else:
            assert np.array_equal(D, first), "a C or D placement changed the result"
