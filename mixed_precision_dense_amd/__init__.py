"""Python binding of ``libmpgemm.so`` (declared in ``include/mpgemm.h``).

Argument marshalling only: every step of D = alpha * op(A) * op(B) + beta * C runs in the HIP
kernels of the library.  PyTorch provides device memory and streams (a tensor argument is
passed as its ``data_ptr()``; a missing stream means torch's current stream).  There is no
CPU fallback: if the library is not built, importing works but every call raises.

The names follow the C ABI: ``mpgemm_create``, ``mpgemm_run``, ``mpgemm_destroy``,
``mpgemm_check``, ``mpgemm_status_string`` and ``mpgemm_tile_shape``; ``Handle`` is a small
owner of one handle.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Union

import torch  # noqa: F401  (loads the HIP runtime the library binds to)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmpgemm.so")

OP_N, OP_T = 0, 1
R_16F, R_16BF, R_8I, R_32F, R_32I, R_8F_E4M3, R_8F_E5M2 = 0, 1, 2, 3, 4, 5, 6
DTYPES = {"f16": R_16F, "bf16": R_16BF, "i8": R_8I, "f32": R_32F, "i32": R_32I,
          "e4m3": R_8F_E4M3, "e5m2": R_8F_E5M2}
STATUS = {0: "SUCCESS", 1: "NOT_INITIALIZED", 2: "INVALID_VALUE", 3: "NOT_SUPPORTED",
          4: "ALLOC_FAILED", 5: "NO_DEVICE", 6: "LAUNCH_FAILED", 7: "INTERNAL_ERROR",
          8: "WRONG_DEVICE", 9: "SCRATCH_TOO_SMALL"}
SUCCESS = 0
NOALLOC_SCRATCH_BYTES = 64 << 20   # MPGEMM_NOALLOC_SCRATCH_BYTES

_lib: Optional[ctypes.CDLL] = None


class MpgemmError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_string(status)})")


_i64, _i32, _u64, _vp = ctypes.c_int64, ctypes.c_int, ctypes.c_uint64, ctypes.c_void_p
# (restype, argtypes) of every function include/mpgemm.h declares
SIGNATURES = {
    "mpgemm_create": (_i32, [ctypes.POINTER(_vp)]),
    "mpgemm_destroy": (_i32, [_vp]),
    "mpgemm_run": (_i32, [_vp, _i32, _i32, _i64, _i64, _i64, _vp, _vp, _i32, _i64, _vp, _i32,
                          _i64, _vp, _vp, _i32, _i64, _vp, _i32, _vp]),
    "mpgemm_check": (_i32, [_i32, _i32, _i64, _i64, _i64, _vp, _vp, _i32, _i64, _vp, _i32, _i64,
                            _vp, _vp, _i32, _i64, _vp, _i32]),
    "mpgemm_status_string": (ctypes.c_char_p, [_i32]),
    "mpgemm_tile_shape": (_i32, [_i64, _i64, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "mpgemm_run_sp24": (_i32, [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _i32, _i64, _vp, _i64, _vp,
                               _i32, _i64, _vp, _vp, _i32, _i64, _vp, _i32, _vp]),
    "mpgemm_check_sp24": (_i32, [_i32, _i64, _i64, _i64, _vp, _vp, _i32, _i64, _vp, _i64, _vp,
                                 _i32, _i64, _vp, _vp, _i32, _i64, _vp, _i32]),
    "mpgemm_run_bf16x3": (_i32, [_vp, _i32, _i32, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _i64,
                                 _vp, _vp, _i64, _vp, _vp, _u64, _vp]),
    "mpgemm_run_bf16x3_noalloc": (_i32, [_vp, _i32, _i32, _i64, _i64, _i64, _vp, _vp, _i64, _vp,
                                         _i64, _vp, _vp, _i64, _vp, _vp]),
    "mpgemm_check_bf16x3": (_i32, [_i32, _i32, _i64, _i64, _i64, _vp, _vp, _i64, _vp, _i64, _vp,
                                   _vp, _i64, _vp, _vp, _u64]),
    "mpgemm_bf16x3_workspace_size": (_u64, [_i32, _i32, _i64, _i64, _i64]),
}


def declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    """Set the C signature of every ABI function the loaded library exports."""
    for name, (res, args) in SIGNATURES.items():
        if hasattr(lib, name):
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
    return lib


def load() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run mixed_precision_dense_amd/build.py "
                               "(or __graft_entry__.build())")
        _lib = declare(ctypes.CDLL(LIB_PATH))
    return _lib


# ----------------------------------------------------------------------------- marshalling
def _dtype(t: Union[str, int]) -> int:
    return DTYPES[t] if isinstance(t, str) else int(t)


def _op(t: Union[bool, int, str]) -> int:
    if isinstance(t, str):
        if t.upper() not in ("N", "T"):
            raise ValueError(f"transpose flag {t!r}: expected 'N' or 'T'")
        return OP_T if t.upper() == "T" else OP_N
    return OP_T if t else OP_N


def _ptr(x) -> Optional[int]:
    """Device address of a tensor (which must live on a GPU), or an integer address as is."""
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        if not x.is_cuda:
            raise ValueError(f"tensor on {x.device}: the kernels read and write device memory")
        return x.data_ptr()
    return int(x)


def _scalar(v, compute_type: int):
    """alpha / beta as the compute type's host scalar (float or int32_t)."""
    if compute_type == R_32I:
        if not -(1 << 31) <= int(v) < (1 << 31):
            raise ValueError(f"integer scalar {v} does not fit in int32")
        return ctypes.c_int32(int(v))
    return ctypes.c_float(float(v))


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


# ----------------------------------------------------------------------------- C ABI
def status_string(status: int) -> str:
    return load().mpgemm_status_string(int(status)).decode()


mpgemm_status_string = status_string


def mpgemm_create() -> int:
    h = ctypes.c_void_p()
    st = load().mpgemm_create(ctypes.byref(h))
    if st != SUCCESS:
        raise MpgemmError(st, "mpgemm_create")
    return h.value


def mpgemm_destroy(handle: int) -> int:
    return load().mpgemm_destroy(handle)


def mpgemm_run(handle, transa, transb, m, n, k, alpha, A, a_type, lda, B, b_type, ldb, beta, C,
               c_type, ldc, D, compute_type, stream=None, check: bool = True) -> int:
    """Queue one GEMM.  Pointers may be ints or tensors; types names or enum values."""
    ct = _dtype(compute_type)
    al, be = _scalar(alpha, ct), _scalar(beta, ct)
    st = load().mpgemm_run(handle, _op(transa), _op(transb), m, n, k, ctypes.byref(al),
                           _ptr(A), _dtype(a_type), lda, _ptr(B), _dtype(b_type), ldb,
                           ctypes.byref(be), _ptr(C), _dtype(c_type), ldc, _ptr(D), ct,
                           _stream(stream))
    if check and st != SUCCESS:
        raise MpgemmError(st, "mpgemm_run")
    return st


def mpgemm_run_bf16x3(handle, transa, transb, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, D,
                      workspace, workspace_bytes, stream=None, check: bool = True) -> int:
    """Queue the FP32 GEMM computed from BF16 pieces (three products); FP32 A, B, C, D."""
    al, be = ctypes.c_float(float(alpha)), ctypes.c_float(float(beta))
    st = load().mpgemm_run_bf16x3(handle, _op(transa), _op(transb), m, n, k, ctypes.byref(al),
                                  _ptr(A), lda, _ptr(B), ldb, ctypes.byref(be), _ptr(C), ldc,
                                  _ptr(D), _ptr(workspace), int(workspace_bytes),
                                  _stream(stream))
    if check and st != SUCCESS:
        raise MpgemmError(st, "mpgemm_run_bf16x3")
    return st


def mpgemm_run_bf16x3_noalloc(handle, transa, transb, m, n, k, alpha, A, lda, B, ldb, beta, C,
                              ldc, D, stream=None, check: bool = True) -> int:
    """mpgemm_run_bf16x3 with the library's fixed scratch buffer in place of a workspace (no
    allocation; calls that overlap on one device race)."""
    al, be = ctypes.c_float(float(alpha)), ctypes.c_float(float(beta))
    st = load().mpgemm_run_bf16x3_noalloc(handle, _op(transa), _op(transb), m, n, k,
                                          ctypes.byref(al), _ptr(A), lda, _ptr(B), ldb,
                                          ctypes.byref(be), _ptr(C), ldc, _ptr(D),
                                          _stream(stream))
    if check and st != SUCCESS:
        raise MpgemmError(st, "mpgemm_run_bf16x3_noalloc")
    return st


def mpgemm_run_sp24(handle, transb, m, n, k, alpha, Ac, a_type, lda, meta, ld_meta, B, b_type,
                    ldb, beta, C, c_type, ldc, D, compute_type="f32", stream=None,
                    check: bool = True) -> int:
    """Queue the GEMM with a 2:4 structured-sparse A given as kept values Ac and metadata
    (alpha and beta are float for F32 compute, int for I32)."""
    ct = _dtype(compute_type)
    al, be = _scalar(alpha, ct), _scalar(beta, ct)
    st = load().mpgemm_run_sp24(handle, _op(transb), m, n, k, ctypes.byref(al), _ptr(Ac),
                                _dtype(a_type), lda, _ptr(meta), ld_meta, _ptr(B), _dtype(b_type),
                                ldb, ctypes.byref(be), _ptr(C), _dtype(c_type), ldc, _ptr(D),
                                ct, _stream(stream))
    if check and st != SUCCESS:
        raise MpgemmError(st, "mpgemm_run_sp24")
    return st


def mpgemm_check_sp24(transb, m, n, k, alpha, Ac, a_type, lda, meta, ld_meta, B, b_type, ldb,
                      beta, C, c_type, ldc, D, compute_type="f32") -> int:
    """Host-only argument check of mpgemm_run_sp24."""
    ct = _dtype(compute_type)
    al, be = _scalar(alpha, ct), _scalar(beta, ct)
    return load().mpgemm_check_sp24(_op(transb), m, n, k, ctypes.byref(al), _ptr(Ac),
                                    _dtype(a_type), lda, _ptr(meta), ld_meta, _ptr(B),
                                    _dtype(b_type), ldb, ctypes.byref(be), _ptr(C), _dtype(c_type),
                                    ldc, _ptr(D), ct)


def mpgemm_check_bf16x3(transa, transb, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, D,
                        workspace, workspace_bytes) -> int:
    """Host-only argument check of mpgemm_run_bf16x3 (the workspace included)."""
    al, be = ctypes.c_float(float(alpha)), ctypes.c_float(float(beta))
    return load().mpgemm_check_bf16x3(_op(transa), _op(transb), m, n, k, ctypes.byref(al),
                                      _ptr(A), lda, _ptr(B), ldb, ctypes.byref(be), _ptr(C), ldc,
                                      _ptr(D), _ptr(workspace), int(workspace_bytes))


def mpgemm_bf16x3_workspace_size(transa, transb, m: int, n: int, k: int) -> int:
    """Workspace bytes mpgemm_run_bf16x3 needs (host-only)."""
    return int(load().mpgemm_bf16x3_workspace_size(_op(transa), _op(transb), m, n, k))


def mpgemm_check(transa, transb, m, n, k, alpha, A, a_type, lda, B, b_type, ldb, beta, C,
                 c_type, ldc, D, compute_type) -> int:
    """Host-only argument check; returns the status mpgemm_run would return before launching."""
    ct = _dtype(compute_type)
    al, be = _scalar(alpha, ct), _scalar(beta, ct)
    return load().mpgemm_check(_op(transa), _op(transb), m, n, k, ctypes.byref(al), _ptr(A),
                               _dtype(a_type), lda, _ptr(B), _dtype(b_type), ldb,
                               ctypes.byref(be), _ptr(C), _dtype(c_type), ldc, _ptr(D), ct)


def mpgemm_tile_shape(m: int, n: int, a_type="f16") -> tuple:
    tm, tn = ctypes.c_int(), ctypes.c_int()
    st = load().mpgemm_tile_shape(m, n, _dtype(a_type), ctypes.byref(tm), ctypes.byref(tn))
    if st != SUCCESS:
        raise MpgemmError(st, "mpgemm_tile_shape")
    return tm.value, tn.value


class Handle:
    """Owns one library handle bound to the current device."""

    def __init__(self):
        self.h = mpgemm_create()

    def run(self, *args, **kwargs) -> int:
        return mpgemm_run(self.h, *args, **kwargs)

    def close(self):
        if self.h is not None:
            mpgemm_destroy(self.h)
            self.h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ----------------------------------------------------------------------------- buffers
def device_buffer(host_array, fmt: str, device="cuda", extra_bytes: int = 0):
    """Copy raw host storage (a numpy array) to a new device tensor holding the same bytes.

    ``extra_bytes`` > 0 appends that many bytes (0xFF-filled) after the data, so reads that
    run past the last row would see them."""
    import numpy as np
    arr = np.ascontiguousarray(host_array)
    flat = torch.from_numpy(arr.view(np.uint8).reshape(-1).copy())
    if extra_bytes:
        flat = torch.cat([flat, torch.full((extra_bytes,), 0xFF, dtype=torch.uint8)])
    dev = flat.to(device)
    return dev


def host_array(dev_buf, fmt: str, shape):
    """Copy a device byte buffer back to numpy raw storage of ``fmt`` with ``shape``."""
    import numpy as np
    storage = {"f16": np.uint16, "bf16": np.uint16, "i8": np.int8, "f32": np.float32,
               "i32": np.int32}[fmt]
    raw = dev_buf.cpu().numpy()
    count = int(np.prod(shape))
    return raw[: count * np.dtype(storage).itemsize].view(storage).reshape(shape)
