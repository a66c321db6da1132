"""Helpers shared by the GPU tests: run one workload through the C-ABI on the GPU and
compare against the oracle (full output or sampled points)."""
import sys
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

import mixed_precision_dense_amd as mp
import oracle
from gemm_inputs import ELEM_BYTES, Inputs, Workload, generate, sample_points

GUARD_ROWS = 2
SENTINEL = 0x5A


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@dataclass
class GpuResult:
    D: np.ndarray           # m x ldc raw storage of the output type
    guard_ok: bool          # sentinel rows after D and the ld padding untouched


_handle = None


def handle():
    global _handle
    if _handle is None:
        _handle = mp.Handle()
    return _handle


def run_gpu(inp: Inputs, d_init: Optional[np.ndarray] = None, in_place: bool = False,
            repeat: int = 1) -> GpuResult:
    """Run inp's workload; D is allocated with GUARD_ROWS extra rows filled with a sentinel
    byte (or from d_init); with in_place=True D aliases C."""
    w = inp.w
    ob = ELEM_BYTES[w.out_type]
    dA = mp.device_buffer(inp.A, w.in_type)
    dB = mp.device_buffer(inp.B, w.b_type)
    d_bytes = (w.m + GUARD_ROWS) * w.ldc * ob
    if in_place:
        assert inp.C is not None
        cbuf = np.concatenate([inp.C.view(np.uint8).reshape(-1),
                               np.full(GUARD_ROWS * w.ldc * ob, SENTINEL, np.uint8)])
        dC = mp.device_buffer(cbuf, "i8")
        dD = dC
    else:
        dC = mp.device_buffer(inp.C, w.out_type) if inp.C is not None else None
        if d_init is not None:
            dD = mp.device_buffer(d_init, w.out_type)
        else:
            dD = torch.full((d_bytes,), SENTINEL, dtype=torch.uint8, device="cuda")
    compute = "i32" if w.in_type == "i8" else "f32"
    alpha = int(w.alpha) if compute == "i32" else w.alpha
    beta = int(w.beta) if compute == "i32" else w.beta
    for _ in range(repeat):
        mp.mpgemm_run(handle().h, w.transa, w.transb, w.m, w.n, w.k, alpha, dA, w.in_type,
                      w.lda, dB, w.b_type, w.ldb, beta, dC, w.out_type, w.ldc, dD, compute)
    torch.cuda.synchronize()
    raw = dD.cpu().numpy()
    D = raw[: w.m * w.ldc * ob].view(np.uint8)
    guard_ok = True
    if d_init is None:
        guard_ok = bool(np.all(raw[w.m * w.ldc * ob:] == SENTINEL))
        if w.ldc > w.n:
            pad = D.reshape(w.m, w.ldc * ob)[:, w.n * ob:]
            if in_place:
                cpad = inp.C.view(np.uint8).reshape(w.m, w.ldc * ob)[:, w.n * ob:]
                guard_ok &= bool(np.array_equal(pad, cpad))
            else:
                guard_ok &= bool(np.all(pad == SENTINEL))
    storage = {"f16": np.uint16, "bf16": np.uint16, "f32": np.float32, "i32": np.int32}[w.out_type]
    return GpuResult(D=D.view(storage).reshape(w.m, w.ldc), guard_ok=guard_ok)


def oracle_ref(inp: Inputs, points=None):
    w = inp.w
    if w.in_type == "i8":
        return oracle.gemm_int(w.transa, w.transb, w.m, w.n, w.k, int(w.alpha), inp.A, w.lda,
                               inp.B, w.ldb, int(w.beta), inp.C, w.ldc, points=points)
    if w.in_type in oracle.FP8:
        return oracle.gemm_fp8(w.transa, w.transb, w.m, w.n, w.k, w.alpha, inp.A, w.in_type,
                               w.lda, inp.B, w.b_type, w.ldb, w.beta, inp.C, w.out_type, w.ldc,
                               points=points)
    return oracle.gemm_fp(w.transa, w.transb, w.m, w.n, w.k, w.alpha, inp.A, w.in_type, w.lda,
                          inp.B, w.in_type, w.ldb, w.beta, inp.C, w.out_type, w.ldc,
                          points=points)


def compare(inp: Inputs, res: GpuResult, exact: bool = False, points=None,
            underflow_floor: bool = False):
    """Compare the GPU output with the oracle; returns a CheckReport."""
    w = inp.w
    ref = oracle_ref(inp, points)
    D = res.D[:, : w.n]
    if points is not None:
        D = D[points[0], points[1]]
    if w.in_type == "i8":
        return oracle.check_int(np.ascontiguousarray(D), ref)
    return oracle.check_fp(np.ascontiguousarray(D), w.out_type, ref, w.k, w.alpha, exact=exact,
                           underflow_floor=underflow_floor, fp8=w.in_type in oracle.FP8)


def check_case(w: Workload, exact: bool = False, sample: Optional[int] = None, seed=None,
               inp: Optional[Inputs] = None, in_place: bool = False):
    say(f"[gpu case] {w.name} {w.in_type}->{w.out_type} m={w.m} n={w.n} k={w.k} "
        f"ta={w.transa} tb={w.transb} lda={w.lda} ldb={w.ldb} ldc={w.ldc} "
        f"alpha={w.alpha} beta={w.beta} exact={exact} sample={sample}")
    if inp is None:
        inp = generate(w, seed=seed)
    res = run_gpu(inp, in_place=in_place)
    points = None if sample is None else sample_points(w.m, w.n, sample)
    rep = compare(inp, res, exact=exact, points=points)
    return rep, res


def model_ref(inp: Inputs, points=None):
    """The oracle's block-FMA model of the matrix-core accumulation (FP16/BF16 inputs)."""
    w = inp.w
    return oracle.gemm_mfma(w.transa, w.transb, w.m, w.n, w.k, w.alpha, inp.A, w.in_type, w.lda,
                            inp.B, w.in_type, w.ldb, w.beta, inp.C, w.out_type, w.ldc, w.out_type,
                            points=points)


def compare_model(inp: Inputs, res: GpuResult, points=None):
    """Bitwise comparison of the GPU output with the block-FMA model (+0 == -0, NaN == NaN)."""
    w = inp.w
    D = res.D[:, : w.n]
    if points is not None:
        D = D[points[0], points[1]]
    return oracle.check_bits(np.ascontiguousarray(D), w.out_type, model_ref(inp, points))


def run_bf16x3(inp: Inputs, in_place: bool = False, workspace_bytes: Optional[int] = None,
               ws_offset: int = 0, check: bool = True):
    """Run mpgemm_run_bf16x3 on inp (FP32 A, B, C, D).  Returns (GpuResult, workspace bytes as
    numpy uint8, status).  D carries GUARD_ROWS sentinel rows; the workspace is a fresh
    256-byte-aligned allocation (plus ws_offset bytes) filled with 0xA5 before the call."""
    w = inp.w
    need = mp.mpgemm_bf16x3_workspace_size(w.transa, w.transb, w.m, w.n, w.k)
    size = need if workspace_bytes is None else workspace_bytes
    dA = mp.device_buffer(inp.A, "f32")
    dB = mp.device_buffer(inp.B, "f32")
    d_bytes = (w.m + GUARD_ROWS) * w.ldc * 4
    if in_place:
        cbuf = np.concatenate([inp.C.view(np.uint8).reshape(-1),
                               np.full(GUARD_ROWS * w.ldc * 4, SENTINEL, np.uint8)])
        dC = dD = mp.device_buffer(cbuf, "i8")
    else:
        dC = mp.device_buffer(inp.C, "f32") if inp.C is not None else None
        dD = torch.full((d_bytes,), SENTINEL, dtype=torch.uint8, device="cuda")
    raw_ws = torch.full((size + 512 + ws_offset,), 0xA5, dtype=torch.uint8, device="cuda")
    base = raw_ws.data_ptr()
    ws_ptr = ((base + 255) // 256) * 256 + ws_offset if size else None
    st = mp.mpgemm_run_bf16x3(handle().h, w.transa, w.transb, w.m, w.n, w.k, w.alpha, dA, w.lda,
                              dB, w.ldb, w.beta, dC, w.ldc, dD, ws_ptr, size, check=check)
    torch.cuda.synchronize()
    raw = dD.cpu().numpy()
    D = raw[: w.m * w.ldc * 4].view(np.uint8)
    guard_ok = bool(np.all(raw[w.m * w.ldc * 4:] == SENTINEL))
    if w.ldc > w.n:
        pad = D.reshape(w.m, w.ldc * 4)[:, w.n * 4:]
        if in_place:
            guard_ok &= bool(np.array_equal(pad, inp.C.view(np.uint8).reshape(w.m, w.ldc * 4)[:, w.n * 4:]))
        else:
            guard_ok &= bool(np.all(pad == SENTINEL))
    ws = raw_ws.cpu().numpy()
    if ws_ptr is not None:
        ws = ws[ws_ptr - base: ws_ptr - base + size]
    res = GpuResult(D=D.view(np.float32).reshape(w.m, w.ldc), guard_ok=guard_ok)
    return res, ws, st


def run_sp24(inp: Inputs, in_place: bool = False, check: bool = True):
    """Run mpgemm_run_sp24 on inp (2:4 sparse A: kept values inp.A, metadata inp.meta).
    D carries GUARD_ROWS sentinel rows; returns (GpuResult, status)."""
    w = inp.w
    ob = ELEM_BYTES[w.out_type]
    dA = mp.device_buffer(inp.A, w.in_type)
    dM = mp.device_buffer(inp.meta, "i8")
    dB = mp.device_buffer(inp.B, w.b_type)
    d_bytes = (w.m + GUARD_ROWS) * w.ldc * ob
    if in_place:
        cbuf = np.concatenate([inp.C.view(np.uint8).reshape(-1),
                               np.full(GUARD_ROWS * w.ldc * ob, SENTINEL, np.uint8)])
        dC = dD = mp.device_buffer(cbuf, "i8")
    else:
        dC = mp.device_buffer(inp.C, w.out_type) if inp.C is not None else None
        dD = torch.full((d_bytes,), SENTINEL, dtype=torch.uint8, device="cuda")
    compute = "i32" if w.in_type == "i8" else "f32"
    st = mp.mpgemm_run_sp24(handle().h, w.transb, w.m, w.n, w.k, w.alpha, dA, w.in_type, w.lda,
                            dM, w.ld_meta, dB, w.b_type, w.ldb, w.beta, dC, w.out_type, w.ldc,
                            dD, compute, check=check)
    torch.cuda.synchronize()
    raw = dD.cpu().numpy()
    D = raw[: w.m * w.ldc * ob].view(np.uint8)
    guard_ok = bool(np.all(raw[w.m * w.ldc * ob:] == SENTINEL))
    if w.ldc > w.n:
        pad = D.reshape(w.m, w.ldc * ob)[:, w.n * ob:]
        if in_place:
            guard_ok &= bool(np.array_equal(pad, inp.C.view(np.uint8).reshape(w.m, w.ldc * ob)[:, w.n * ob:]))
        else:
            guard_ok &= bool(np.all(pad == SENTINEL))
    storage = {"f16": np.uint16, "bf16": np.uint16, "f32": np.float32, "i32": np.int32}[w.out_type]
    return GpuResult(D=D.view(storage).reshape(w.m, w.ldc), guard_ok=guard_ok), st


def sp24_ref(inp: Inputs, points=None):
    w = inp.w
    if w.in_type == "i8":
        return oracle.gemm_sp24_int(w.transb, w.m, w.n, w.k, int(w.alpha), inp.A, w.lda,
                                    inp.meta, w.ld_meta, inp.B, w.ldb, int(w.beta), inp.C, w.ldc,
                                    points=points)
    return oracle.gemm_sp24(w.transb, w.m, w.n, w.k, w.alpha, inp.A, w.in_type, w.lda, inp.meta,
                            w.ld_meta, inp.B, w.ldb, w.beta, inp.C, w.out_type, w.ldc,
                            points=points, btype=w.b_type)


def compare_sp24(inp: Inputs, res: GpuResult, exact: bool = False, points=None):
    """The sparse output against the oracle: exact, or within the FP bound over k/2 products."""
    w = inp.w
    D = res.D[:, : w.n]
    if points is not None:
        D = D[points[0], points[1]]
    if w.in_type == "i8":
        return oracle.check_int(np.ascontiguousarray(D), sp24_ref(inp, points))
    return oracle.check_fp(np.ascontiguousarray(D), w.out_type, sp24_ref(inp, points),
                           max(w.k // 2, 1), w.alpha, exact=exact, fp8=w.in_type in oracle.FP8)


def compare_sp24_model(inp: Inputs, res: GpuResult, points=None):
    """Bitwise comparison of the sparse output with the sparse block model."""
    w = inp.w
    D = res.D[:, : w.n]
    if points is not None:
        D = D[points[0], points[1]]
    ref = oracle.gemm_sp24_mfma(w.transb, w.m, w.n, w.k, w.alpha, inp.A, w.in_type, w.lda,
                                inp.meta, w.ld_meta, inp.B, w.ldb, w.beta, inp.C, w.out_type,
                                w.ldc, w.out_type, points=points)
    return oracle.check_bits(np.ascontiguousarray(D), w.out_type, ref)


def compare_fp8_model(inp: Inputs, res: GpuResult, points=None):
    """Bitwise comparison of an FP8 GEMM output with the oracle's two-level FP8 model."""
    w = inp.w
    D = res.D[:, : w.n]
    if points is not None:
        D = D[points[0], points[1]]
    ref = oracle.gemm_fp8_mfma(w.transa, w.transb, w.m, w.n, w.k, w.alpha, inp.A, w.in_type,
                               w.lda, inp.B, w.b_type, w.ldb, w.beta, inp.C, w.out_type, w.ldc,
                               w.out_type, points=points)
    return oracle.check_bits(np.ascontiguousarray(D), w.out_type, ref)


def compare_sp24_fp8_model(inp: Inputs, res: GpuResult, points=None):
    """Bitwise comparison of a sparse FP8 output with the FP8 block model over kept products."""
    w = inp.w
    D = res.D[:, : w.n]
    if points is not None:
        D = D[points[0], points[1]]
    ref = oracle.gemm_sp24_fp8_mfma(w.transb, w.m, w.n, w.k, w.alpha, inp.A, w.in_type, w.lda,
                                    inp.meta, w.ld_meta, inp.B, w.b_type, w.ldb, w.beta, inp.C,
                                    w.out_type, w.ldc, w.out_type, points=points)
    return oracle.check_bits(np.ascontiguousarray(D), w.out_type, ref)
