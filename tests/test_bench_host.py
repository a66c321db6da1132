"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the source digest that ties a
counters summary to the kernel sources it was taken on, and the reading of that summary."""
import os
import shutil
import subprocess
import sys

import pytest

import bench
from gemm_inputs import NEXT_WORKLOADS, WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


@pytest.fixture
def tree(tmp_path, monkeypatch):
    """A copy of the kernel sources under a temporary root that bench.py reads from."""
    shutil.copytree(os.path.join(ROOT, "mixed_precision_dense_amd", "csrc"),
                    tmp_path / "mixed_precision_dense_amd" / "csrc")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def test_digest_separates_the_dense_and_sparse_sources(tree):
    csrc = tree / "mixed_precision_dense_amd" / "csrc"
    dense, sparse = bench.kernel_source_digest(), bench.kernel_source_digest(True)
    assert dense != sparse and len(dense) == len(sparse) == 16
    with open(csrc / "sp24_kernel.inc", "a") as f:
        f.write("\n// edited\n")
    assert bench.kernel_source_digest() == dense           # a sparse edit leaves dense alone
    assert bench.kernel_source_digest(True) != sparse
    sparse2 = bench.kernel_source_digest(True)
    with open(csrc / "mpgemm_kernel.hpp", "a") as f:
        f.write("\n// edited\n")
    assert bench.kernel_source_digest() != dense           # a shared header changes both
    assert bench.kernel_source_digest(True) != sparse2


def _write_counters(tree, w, digest, busy=1.0e9, active=1.2e7, avg_ns=7.5e5, hbm=2.5e9):
    path = tree / "profiles" / f"mpgemm_{w.name}_counters.txt"
    path.write_text("\n".join([
        "# a counters summary", f"workload = {w.name}", f"kernel_source_sha256 = {digest}",
        f"rocprof_avg_ns = {avg_ns:.0f}", f"hbm_bytes_per_launch = {hbm:.0f}",
        f"sq_SQ_VALU_MFMA_BUSY_CYCLES = {busy:.0f}", f"sq_GRBM_GUI_ACTIVE = {active:.0f}", ""]))
    return path


def test_counters_are_read_only_for_their_workload_and_sources(tree):
    w = WORKLOADS["bf16_8192_nn"]
    path = _write_counters(tree, w, bench.kernel_source_digest())
    c = bench.recorded_counters(w)
    assert c is not None
    # busy cycles over 1024 SIMDs x (GRBM_GUI_ACTIVE / 8 XCDs)
    assert c["mfma_busy_pct"] == pytest.approx(100 * 1.0e9 / (1024 * 1.2e7 / 8), abs=0.01)
    assert c["hbm_GBs"] == pytest.approx(2.5e9 / 7.5e-4 / 1e9, abs=0.1)
    assert c["rocprof_avg_us"] == 750.0
    assert c["clock_GHz_from_counters"] == pytest.approx(1.2e7 / 8 / 7.5e5, abs=1e-3)
    _write_counters(tree, w, "0" * 16)                      # other sources
    assert bench.recorded_counters(w) is None
    path.write_text(path.read_text().replace("workload = bf16_8192_nn", "workload = f16_4096_nt"))
    assert bench.recorded_counters(w) is None               # another workload's numbers
    assert bench.recorded_counters(WORKLOADS["i8_4096_nn"]) is None   # no file at all


def test_an_impossible_counter_clock_is_not_reported(tree):
    # GRBM_GUI_ACTIVE counts a window around the dispatch; over a short kernel's duration it
    # can imply more than the chip's 2.4 GHz, and then the clock is withheld and the busy
    # share flagged as a lower bound
    w = WORKLOADS["f16_5000x3000x1000_f16out"]
    _write_counters(tree, w, bench.kernel_source_digest(), active=8 * 2.6e3 * 34.6, avg_ns=34.6e3)
    c = bench.recorded_counters(w)
    assert c["clock_GHz_from_counters"] is None
    assert "lower bound" in c["counter_window_note"] and "2.60 GHz" in c["counter_window_note"]
    _write_counters(tree, w, bench.kernel_source_digest(), active=8 * 2.3e3 * 34.6, avg_ns=34.6e3)
    c = bench.recorded_counters(w)
    assert c["clock_GHz_from_counters"] == pytest.approx(2.3, abs=1e-3)
    assert "counter_window_note" not in c


def test_sparse_counters_use_the_sparse_digest(tree):
    w = NEXT_WORKLOADS["f16_sp24_4096_nt"]
    _write_counters(tree, w, bench.kernel_source_digest())
    assert bench.recorded_counters(w) is None
    _write_counters(tree, w, bench.kernel_source_digest(True))
    assert bench.recorded_counters(w) is not None
