"""mpgemm_run_bf16x3_noalloc (the three-product FP32 GEMM on the library's fixed scratch
buffer, for callers that cannot allocate) against mpgemm_run_bf16x3 with a caller-provided
workspace: bit-identical outputs on two calls in a row, the second on a smaller problem
(the buffer keeps the first call's contents), and a problem beyond the buffer refused
without a launch."""
import numpy as np
import pytest
import torch

import mixed_precision_dense_amd as mp
from gemm_inputs import Workload, generate
from tests.gpu_harness import handle, say

pytestmark = pytest.mark.gpu

ST = {v: k for k, v in mp.STATUS.items()}


def _both(w):
    say(f"[gpu noalloc] {w.name} m={w.m} n={w.n} k={w.k} ta={w.transa} tb={w.transb} "
        f"alpha={w.alpha} beta={w.beta}")
    inp = generate(w)
    dA, dB = mp.device_buffer(inp.A, "f32"), mp.device_buffer(inp.B, "f32")
    dC = mp.device_buffer(inp.C, "f32") if inp.C is not None else None
    need = mp.mpgemm_bf16x3_workspace_size(w.transa, w.transb, w.m, w.n, w.k)
    assert 0 < need <= mp.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    ws_ptr = (ws.data_ptr() + 255) // 256 * 256
    d_ref = torch.full((w.m * w.ldc,), float("nan"), dtype=torch.float32, device="cuda")
    d_new = torch.full((w.m * w.ldc,), float("nan"), dtype=torch.float32, device="cuda")
    h = handle().h
    mp.mpgemm_run_bf16x3(h, w.transa, w.transb, w.m, w.n, w.k, w.alpha, dA, w.lda, dB, w.ldb,
                         w.beta, dC, w.ldc, d_ref, ws_ptr, need)
    mp.mpgemm_run_bf16x3_noalloc(h, w.transa, w.transb, w.m, w.n, w.k, w.alpha, dA, w.lda, dB,
                                 w.ldb, w.beta, dC, w.ldc, d_new)
    torch.cuda.synchronize()
    ref = d_ref.cpu().numpy().reshape(w.m, w.ldc)[:, : w.n]
    new = d_new.cpu().numpy().reshape(w.m, w.ldc)[:, : w.n]
    assert np.isfinite(ref).all()
    assert np.array_equal(ref.view(np.uint32), new.view(np.uint32))


def test_noalloc_equals_workspace_entry_point_on_two_calls():
    # first call: 3.2 MB of pieces; second, smaller, on transposed storage with beta != 0
    _both(Workload("noalloc_1", "f32", "f32", 1000, 770, 1000, transb=True,
                   a_dist="normal(0,1)", b_dist="normal(0,1)", seed=90))
    _both(Workload("noalloc_2", "f32", "f32", 300, 200, 136, transa=True, alpha=0.5, beta=-1.0,
                   a_dist="normal(0,1)", b_dist="normal(0,1)", c_dist="normal(0,1)", seed=91))


def test_noalloc_refuses_a_problem_beyond_the_scratch_buffer():
    m = n = k = 4096            # 192 MiB of pieces
    assert mp.mpgemm_bf16x3_workspace_size(False, True, m, n, k) > mp.NOALLOC_SCRATCH_BYTES
    dA = torch.zeros(m * k, dtype=torch.float32, device="cuda")
    dB = torch.zeros(n * k, dtype=torch.float32, device="cuda")
    dD = torch.full((m * n,), 7.0, dtype=torch.float32, device="cuda")
    st = mp.mpgemm_run_bf16x3_noalloc(handle().h, False, True, m, n, k, 1.0, dA, k, dB, k, 0.0,
                                      None, n, dD, check=False)
    assert st == ST["SCRATCH_TOO_SMALL"]
    torch.cuda.synchronize()
    assert bool((dD == 7.0).all())            # nothing was launched
    # an argument error is reported as such, before the size limit
    st = mp.mpgemm_run_bf16x3_noalloc(handle().h, False, True, m, n, k, 1.0, dA, k - 1, dB, k,
                                      0.0, None, n, dD, check=False)
    assert st == ST["INVALID_VALUE"]
