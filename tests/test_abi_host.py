"""The C-ABI library on the host: it loads, exports every function include/mpgemm.h declares,
and checks its arguments before touching a device.  CPU only (no compute call is made)."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mpgemm.h")

import mixed_precision_dense_amd as mp  # noqa: E402

if not os.path.exists(mp.LIB_PATH):
    from mixed_precision_dense_amd import build as _b
    _b.build()

ST = {v: k for k, v in mp.STATUS.items()}


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mpgemm_[a-z_]+)\s*\(", text)))


def test_header_declares_the_abi():
    names = declared_functions()
    for n in ("mpgemm_create", "mpgemm_run", "mpgemm_destroy", "mpgemm_status_string",
              "mpgemm_check", "mpgemm_tile_shape"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mp.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings():
    for code in range(0, 10):
        s = mp.status_string(code)
        assert isinstance(s, str) and len(s) > 3
    assert "unknown" in mp.status_string(99)


@pytest.mark.skipif(torch.cuda.is_available(), reason="host without a GPU only")
def test_create_without_device_returns_no_device():
    h = ctypes.c_void_p(123)
    assert mp.load().mpgemm_create(ctypes.byref(h)) == ST["NO_DEVICE"]
    assert h.value is None
    assert mp.load().mpgemm_create(None) == ST["INVALID_VALUE"]


def test_destroy_and_run_reject_unknown_handles():
    lib = mp.load()
    assert lib.mpgemm_destroy(None) == ST["NOT_INITIALIZED"]
    fake = ctypes.c_void_p(0x1000)
    assert lib.mpgemm_destroy(fake) == ST["NOT_INITIALIZED"]
    assert mp.mpgemm_run(0x1000, False, False, 8, 8, 8, 1.0, 16, "f16", 8, 16, "f16", 8, 0.0,
                         None, "f32", 8, 16, "f32", stream=0, check=False) == ST["NOT_INITIALIZED"]


P = 1 << 20   # a 16-byte aligned fake device address (never dereferenced on the host)


def chk(**kw):
    a = dict(transa=False, transb=False, m=64, n=64, k=64, alpha=1.0, A=P, a_type="f16", lda=64,
             B=P, b_type="f16", ldb=64, beta=0.0, C=None, c_type="f32", ldc=64, D=P,
             compute_type="f32")
    a.update(kw)
    return mp.mpgemm_check(a["transa"], a["transb"], a["m"], a["n"], a["k"], a["alpha"], a["A"],
                           a["a_type"], a["lda"], a["B"], a["b_type"], a["ldb"], a["beta"],
                           a["C"], a["c_type"], a["ldc"], a["D"], a["compute_type"])


def test_valid_problems_pass():
    assert chk() == ST["SUCCESS"]
    assert chk(transa=True, transb=True) == ST["SUCCESS"]
    assert chk(a_type="bf16", b_type="bf16", c_type="bf16", ldc=64) == ST["SUCCESS"]
    assert chk(a_type="i8", b_type="i8", c_type="i32", compute_type="i32", lda=64, ldb=64,
               alpha=1, beta=0) == ST["SUCCESS"]
    assert chk(c_type="f16", ldc=64) == ST["SUCCESS"]
    # the five workloads' argument sets
    assert chk(m=4096, n=4096, k=4096, lda=4096, ldb=4096, ldc=4096, transb=True) == ST["SUCCESS"]
    assert chk(m=5000, n=3000, k=1000, lda=1000, ldb=3000, ldc=3000, c_type="f16") == ST["SUCCESS"]
    assert chk(m=256, n=256, k=256, lda=256, ldb=256, ldc=256, beta=1.0, C=P) == ST["SUCCESS"]


def test_sizes_and_nulls():
    assert chk(m=-1) == ST["INVALID_VALUE"]
    assert chk(k=-5) == ST["INVALID_VALUE"]
    assert chk(m=0, A=None, B=None, D=None) == ST["SUCCESS"]          # empty output: no-op
    assert chk(n=0) == ST["SUCCESS"]
    assert chk(k=0, A=None, B=None, lda=8, ldb=64) == ST["SUCCESS"]    # D = beta * C
    assert chk(k=0, A=None, B=None, lda=1, ldb=64) == ST["NOT_SUPPORTED"]  # stride still aligned
    assert chk(A=None) == ST["INVALID_VALUE"]
    assert chk(D=None) == ST["INVALID_VALUE"]
    assert chk(beta=1.0, C=None) == ST["INVALID_VALUE"]                # C needed when beta != 0
    assert chk(beta=0.0, C=None) == ST["SUCCESS"]                      # not read when beta == 0
    assert chk(beta=-0.0, C=None) == ST["SUCCESS"]                     # -0 is zero: not read
    assert chk(beta=float("nan"), C=None) == ST["INVALID_VALUE"]       # NaN beta reads C
    lib = mp.load()
    one = ctypes.c_float(1.0)
    # null alpha / beta pointers
    assert lib.mpgemm_check(0, 0, 8, 8, 8, None, P, 0, 8, P, 0, 8, ctypes.byref(one), None, 3, 8,
                            P, 3) == ST["INVALID_VALUE"]
    assert lib.mpgemm_check(0, 0, 8, 8, 8, ctypes.byref(one), P, 0, 8, P, 0, 8, None, None, 3, 8,
                            P, 3) == ST["INVALID_VALUE"]
    assert lib.mpgemm_check(2, 0, 8, 8, 8, ctypes.byref(one), P, 0, 8, P, 0, 8, ctypes.byref(one),
                            P, 3, 8, P, 3) == ST["INVALID_VALUE"]    # bad transpose flag


def test_size_limits():
    """m and n up to 2^31 - 1; k up to 2^31 - 256, so that the kernel's stage count (k rounded
    up to a whole stage, in 32-bit arithmetic) cannot overflow."""
    big = (1 << 31) - 1
    kmax = (1 << 31) - 256
    # A stored k x m and B stored k x n: k is limited by neither leading dimension
    tall = dict(transa=True, transb=False, m=1, n=1, lda=8, ldb=8, ldc=4)
    assert chk(k=kmax, **tall) == ST["SUCCESS"]
    assert chk(k=kmax + 1, **tall) == ST["NOT_SUPPORTED"]
    assert chk(k=big, **tall) == ST["NOT_SUPPORTED"]
    assert chk(k=big + 1, **tall) == ST["NOT_SUPPORTED"]
    assert chk(m=big + 1) == ST["NOT_SUPPORTED"]


def test_leading_dimension_minimums():
    assert chk(lda=56) == ST["INVALID_VALUE"]               # lda < k
    assert chk(transa=True, m=72, lda=64) == ST["INVALID_VALUE"]   # lda < m
    assert chk(ldb=56) == ST["INVALID_VALUE"]               # ldb < n
    assert chk(transb=True, k=72, lda=72, ldb=64) == ST["INVALID_VALUE"]
    assert chk(ldc=60) == ST["INVALID_VALUE"]


def test_types_outside_the_matrix_are_not_supported():
    assert chk(a_type="f16", b_type="bf16") == ST["NOT_SUPPORTED"]           # mixed inputs
    assert chk(c_type="bf16") == ST["NOT_SUPPORTED"]                          # f16 in, bf16 out
    assert chk(compute_type="i32") == ST["NOT_SUPPORTED"]
    assert chk(a_type="i8", b_type="i8", c_type="f32", compute_type="f32") == ST["NOT_SUPPORTED"]
    assert chk(a_type="f32", b_type="f32") == ST["NOT_SUPPORTED"]
    assert chk(a_type=9, b_type=9) == ST["NOT_SUPPORTED"]


def test_alignment_contract():
    assert chk(A=P + 8) == ST["NOT_SUPPORTED"]
    assert chk(D=P + 4) == ST["NOT_SUPPORTED"]
    assert chk(beta=1.0, C=P + 8) == ST["NOT_SUPPORTED"]                    # C read: aligned
    assert chk(beta=0.0, C=P + 8) == ST["SUCCESS"]                          # C not read
    assert chk(k=60, lda=60, ldb=64) == ST["NOT_SUPPORTED"]                  # 120 B rows
    assert chk(n=60, ldb=60, ldc=64) == ST["NOT_SUPPORTED"]
    assert chk(ldc=66) == ST["NOT_SUPPORTED"]
    assert chk(a_type="i8", b_type="i8", c_type="i32", compute_type="i32", alpha=1, beta=0,
               lda=72, ldb=64) == ST["NOT_SUPPORTED"]                       # 72 B rows of int8
    # strides whose 256 rows span 2 GiB or more
    assert chk(lda=1 << 22, ldb=64) == ST["NOT_SUPPORTED"]
    assert chk(lda=(1 << 22) - 8, ldb=64) == ST["SUCCESS"]                  # largest FP16 stride
    # strides so large that 256 * ld * element size wraps around in 64 bits
    for big in (1 << 56, 1 << 61, (1 << 63) - 8):
        assert chk(lda=big) == ST["NOT_SUPPORTED"]
        assert chk(ldb=big) == ST["NOT_SUPPORTED"]
        assert chk(ldc=big) == ST["NOT_SUPPORTED"]


def test_tile_shape():
    assert mp.mpgemm_tile_shape(4096, 4096) == (256, 256)
    assert mp.mpgemm_tile_shape(256, 256) == (64, 64)
    assert mp.mpgemm_tile_shape(256, 256, "i8") == (128, 128)
    assert mp.mpgemm_tile_shape(5000, 3000) == (256, 256)
    # one round of 144 large tiles beats three rounds of 576 half-size ones
    assert mp.mpgemm_tile_shape(3072, 3072) == (256, 256)
    assert mp.mpgemm_tile_shape(2048, 2048) == (128, 128)   # 64 large tiles would idle 3/4 of the CUs
    assert mp.mpgemm_tile_shape(1024, 1024) == (64, 64)
    assert mp.mpgemm_tile_shape(1024, 1024, "e4m3") == (128, 128)


def test_bf16x3_check():
    """mpgemm_check_bf16x3 returns the status mpgemm_run_bf16x3 would return before any
    device call, the workspace's size and alignment included."""
    W = 1 << 24                                    # a 256-byte aligned fake workspace address

    def c(**kw):
        a = dict(transa=False, transb=True, m=64, n=64, k=64, alpha=1.0, A=P, lda=64, B=P,
                 ldb=64, beta=0.0, C=None, ldc=64, D=P, workspace=W, workspace_bytes=None)
        a.update(kw)
        need = mp.mpgemm_bf16x3_workspace_size(a["transa"], a["transb"], a["m"], a["n"], a["k"])
        wb = need if a["workspace_bytes"] is None else a["workspace_bytes"]
        return mp.mpgemm_check_bf16x3(a["transa"], a["transb"], a["m"], a["n"], a["k"],
                                      a["alpha"], a["A"], a["lda"], a["B"], a["ldb"], a["beta"],
                                      a["C"], a["ldc"], a["D"], a["workspace"], wb)

    assert c() == ST["SUCCESS"]
    assert c(transa=True, transb=False, m=5, n=3, k=7, lda=8, ldb=4, ldc=4) == ST["SUCCESS"]
    assert c(m=0, A=None, B=None, D=None, workspace=None) == ST["SUCCESS"]     # no-op
    assert c(k=0, A=None, B=None, lda=4, workspace=None) == ST["SUCCESS"]      # D = beta C
    assert c(workspace_bytes=1000) == ST["INVALID_VALUE"]                     # too small
    assert c(workspace=None) == ST["INVALID_VALUE"]
    assert c(workspace=W + 16) == ST["NOT_SUPPORTED"]                         # 256-byte alignment
    assert c(m=-1) == ST["INVALID_VALUE"]
    assert c(lda=60) == ST["INVALID_VALUE"]
    assert c(lda=66) == ST["NOT_SUPPORTED"]                                   # 4-element strides
    assert c(beta=1.0) == ST["INVALID_VALUE"]                                 # C needed
    assert c(beta=1.0, C=P + 8) == ST["NOT_SUPPORTED"]                        # C misaligned
    assert c(transa=True, transb=False, m=4, n=4, k=(1 << 31) // 3, lda=4, ldb=4,
             ldc=4) == ST["NOT_SUPPORTED"]                                    # 3 kp past int32
    assert mp.load().mpgemm_check_bf16x3(2, 0, 8, 8, 8, None, P, 8, P, 8, None, None, 8, P, W,
                                         1 << 20) == ST["INVALID_VALUE"]


def test_bf16x3_workspace_size():
    ws = mp.mpgemm_bf16x3_workspace_size
    # 4096^3 NT: A3 = 4096 x 12288 BF16, B3 = 4096 x 12288 BF16, no padding between them
    assert ws(False, True, 4096, 4096, 4096) == 2 * 4096 * 12288 * 2
    # transposed storage, ragged: kp = 8, k3 = 24; A3 = 24 x 8 (ld = m rounded up) = 384 B,
    # B3 at 512: 3 x 24 = 144 B
    assert ws(True, True, 5, 3, 7) == 512 + 144
    assert ws(False, False, 5, 3, 7) == 256 + 24 * 8 * 2       # A3 5 x 24 = 240 B -> 256
    assert ws(False, False, 5, 3, 0) == 0 and ws(False, False, 0, 3, 5) == 0
    assert ws(False, False, -1, 3, 5) == 0
    assert mp.load().mpgemm_bf16x3_workspace_size(2, 0, 8, 8, 8) == 0


def test_bf16x3_rejects_unknown_handles():
    assert mp.mpgemm_run_bf16x3(0x1000, False, False, 8, 8, 8, 1.0, P, 8, P, 8, 0.0, None, 8, P,
                                P, 1 << 20, stream=0, check=False) == ST["NOT_INITIALIZED"]


def test_fp8_type_matrix():
    for a in ("e4m3", "e5m2"):
        for b in ("e4m3", "e5m2"):
            assert chk(a_type=a, b_type=b, c_type="f32") == ST["SUCCESS"]
            assert chk(a_type=a, b_type=b, c_type="bf16") == ST["SUCCESS"]
            assert chk(a_type=a, b_type=b, c_type="f16") == ST["NOT_SUPPORTED"]
            assert chk(a_type=a, b_type=b, c_type="f32", compute_type="i32") == ST["NOT_SUPPORTED"]
    assert chk(a_type="e4m3", b_type="f16") == ST["NOT_SUPPORTED"]
    assert chk(a_type="e4m3", b_type="e4m3", lda=72) == ST["NOT_SUPPORTED"]     # 16-element rows
    assert mp.mpgemm_tile_shape(256, 256, "e4m3") == (128, 128)


def chk_sp(**kw):
    a = dict(transb=True, m=300, n=200, k=256, alpha=1.0, Ac=P, a_type="f16", lda=128, meta=P,
             ld_meta=32, B=P, b_type="f16", ldb=256, beta=0.0, C=None, c_type="f32", ldc=200,
             D=P, compute_type="f32")
    a.update(kw)
    return mp.mpgemm_check_sp24(a["transb"], a["m"], a["n"], a["k"], a["alpha"], a["Ac"],
                                a["a_type"], a["lda"], a["meta"], a["ld_meta"], a["B"],
                                a["b_type"], a["ldb"], a["beta"], a["C"], a["c_type"], a["ldc"],
                                a["D"], a["compute_type"])


def test_sp24_contract():
    assert chk_sp() == ST["SUCCESS"]
    assert chk_sp(transb=False, ldb=200) == ST["SUCCESS"]
    for a, c in (("f16", "f16"), ("bf16", "f32"), ("bf16", "bf16")):
        assert chk_sp(a_type=a, b_type=a, c_type=c) == ST["SUCCESS"]
    # types outside the matrix
    assert chk_sp(a_type="f16", b_type="bf16") == ST["NOT_SUPPORTED"]
    assert chk_sp(c_type="bf16") == ST["NOT_SUPPORTED"]
    assert chk_sp(a_type="i8", b_type="i8", c_type="i32", compute_type="i32", alpha=2,
                  beta=0) == ST["SUCCESS"]
    assert chk_sp(a_type="i8", b_type="i8", c_type="i32", compute_type="i32", lda=144,
                  ldb=272) == ST["SUCCESS"]                 # 16-byte rows of 1-byte elements
    assert chk_sp(a_type="i8", b_type="i8", c_type="i32", compute_type="i32", lda=136,
                  ldb=272) == ST["NOT_SUPPORTED"]
    assert chk_sp(a_type="i8", b_type="i8", c_type="i32", compute_type="i32",
                  lda=132) == ST["NOT_SUPPORTED"]
    assert chk_sp(a_type="i8", b_type="i8", c_type="f32", compute_type="f32") == ST["NOT_SUPPORTED"]
    assert chk_sp(a_type="i8", b_type="i8", c_type="i32", compute_type="f32") == ST["NOT_SUPPORTED"]
    assert chk_sp(a_type="i8", b_type="f16", c_type="i32", compute_type="i32") == ST["NOT_SUPPORTED"]
    for a in ("e4m3", "e5m2"):
        for b in ("e4m3", "e5m2"):
            assert chk_sp(a_type=a, b_type=b, lda=144, ldb=272) == ST["SUCCESS"]
            assert chk_sp(a_type=a, b_type=b, c_type="bf16", lda=144, ldb=272) == ST["SUCCESS"]
            assert chk_sp(a_type=a, b_type=b, c_type="f16", lda=144, ldb=272) == ST["NOT_SUPPORTED"]
            assert chk_sp(a_type=a, b_type=b, lda=136, ldb=272) == ST["NOT_SUPPORTED"]
    assert chk_sp(a_type="e4m3", b_type="f16") == ST["NOT_SUPPORTED"]
    assert chk_sp(compute_type="i32") == ST["NOT_SUPPORTED"]
    # k a multiple of 128; k = 0 allowed (D = beta C), with null operands
    assert chk_sp(k=200, lda=104, ld_meta=32, ldb=200) == ST["NOT_SUPPORTED"]
    assert chk_sp(k=192, lda=96, ld_meta=32, ldb=192) == ST["NOT_SUPPORTED"]   # 64 | k, 128 does not
    assert chk_sp(k=64, lda=32, ld_meta=16, ldb=64) == ST["NOT_SUPPORTED"]
    assert chk_sp(k=0, lda=8, ld_meta=16, ldb=8, Ac=None, meta=None, B=None) == ST["SUCCESS"]
    # leading-dimension minimums and alignment
    assert chk_sp(lda=120) == ST["INVALID_VALUE"]
    assert chk_sp(ld_meta=16) == ST["INVALID_VALUE"]          # 256 / 8 = 32 bytes per row
    assert chk_sp(ldb=200) == ST["INVALID_VALUE"]
    assert chk_sp(ldc=199) == ST["INVALID_VALUE"]
    assert chk_sp(lda=132) == ST["NOT_SUPPORTED"]             # 264-byte rows
    assert chk_sp(ld_meta=40) == ST["NOT_SUPPORTED"]
    assert chk_sp(Ac=P + 8) == ST["NOT_SUPPORTED"]
    assert chk_sp(meta=P + 4) == ST["NOT_SUPPORTED"]
    # nulls, negative sizes, empty outputs
    assert chk_sp(meta=None) == ST["INVALID_VALUE"]
    assert chk_sp(D=None) == ST["INVALID_VALUE"]
    assert chk_sp(beta=1.0) == ST["INVALID_VALUE"]            # C needed
    assert chk_sp(beta=1.0, C=P) == ST["SUCCESS"]
    assert chk_sp(m=-1) == ST["INVALID_VALUE"]
    assert chk_sp(m=0, Ac=None, meta=None, B=None, D=None) == ST["SUCCESS"]
    # strides past what 32-bit tile offsets reach
    assert chk_sp(lda=1 << 22) == ST["NOT_SUPPORTED"]
    for big in (1 << 56, 1 << 61, (1 << 63) - 16):
        assert chk_sp(lda=big) == ST["NOT_SUPPORTED"]
        assert chk_sp(ld_meta=big) == ST["NOT_SUPPORTED"]
        assert chk_sp(ldb=big) == ST["NOT_SUPPORTED"]
        assert chk_sp(ldc=big) == ST["NOT_SUPPORTED"]


def test_sp24_rejects_unknown_handles():
    assert mp.mpgemm_run_sp24(0x1000, True, 8, 8, 128, 1.0, P, "f16", 64, P, 16, P, "f16", 128,
                              0.0, None, "f32", 8, P, stream=0, check=False) == ST["NOT_INITIALIZED"]


def test_missing_library_fails_loudly(monkeypatch):
    """Without the built HIP library every entry point of the binding raises: there is no
    fallback path."""
    monkeypatch.setattr(mp, "_lib", None)
    monkeypatch.setattr(mp, "LIB_PATH", "/nonexistent/libmpgemm.so")
    with pytest.raises(RuntimeError, match="not built"):
        mp.load()
    with pytest.raises(RuntimeError, match="not built"):
        mp.Handle()
    with pytest.raises(RuntimeError, match="not built"):
        mp.mpgemm_run(0x1000, False, False, 8, 8, 8, 1.0, 16, "f16", 8, 16, "f16", 8, 0.0,
                      None, "f32", 8, 16, "f32", stream=0)
    with pytest.raises(RuntimeError, match="not built"):
        mp.mpgemm_run_sp24(0x1000, True, 8, 8, 128, 1.0, 16, "f16", 64, 16, 16, 16, "f16", 128,
                           0.0, None, "f32", 8, 16, stream=0)
    with pytest.raises(RuntimeError, match="not built"):
        mp.mpgemm_check(False, False, 8, 8, 8, 1.0, 16, "f16", 8, 16, "f16", 8, 0.0, None,
                        "f32", 8, 16, "f32")


def test_binding_rejects_host_tensors_and_unknown_flags():
    """A CPU tensor would hand a host address to the kernels; an unknown transpose letter would
    silently mean N.  Both are refused before the library is called."""
    cpu = torch.zeros(64, dtype=torch.float16)
    with pytest.raises(ValueError, match="device memory"):
        mp.mpgemm_check(False, False, 8, 8, 8, 1.0, cpu, "f16", 8, P, "f16", 8, 0.0, None, "f32",
                        8, P, "f32")
    with pytest.raises(ValueError, match="'N' or 'T'"):
        mp.mpgemm_check("X", False, 8, 8, 8, 1.0, P, "f16", 8, P, "f16", 8, 0.0, None, "f32", 8,
                        P, "f32")
    assert chk(transa="t", transb="N") == ST["SUCCESS"]
    i8 = dict(a_type="i8", b_type="i8", c_type="i32", compute_type="i32", lda=64, ldb=64)
    assert chk(alpha=(1 << 31) - 1, beta=-(1 << 31), C=P, **i8) == ST["SUCCESS"]
    with pytest.raises(ValueError, match="int32"):
        chk(alpha=1 << 31, beta=0, **i8)
