"""The CPU oracle and the library's host-only argument checks, built with gcc's address and
undefined-behaviour sanitizers and exercised by the existing oracle pins and host ABI tests.

Both are compiled here from the committed sources (``oracle/mpgemm_oracle.c``;
``mixed_precision_dense_amd/csrc/mpgemm_host.cpp``, which holds mpgemm_check,
mpgemm_check_sp24, mpgemm_check_bf16x3, the tile rule and the three-product GEMM's workspace
layout) with ``-fsanitize=address,undefined -fno-sanitize-recover=all``.  A child pytest
process preloads the sanitizer runtime and loads these builds in place of the ordinary ones
(``MPGEMM_ORACLE_LIB``, ``MPGEMM_HOST_CHECK_LIB``); any invalid memory access or undefined
behaviour aborts it, which fails the test here.  CPU only.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixed_precision_dense_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]

# the oracle pins and the host ABI tests that need no device and no HIP library symbol
ORACLE_TESTS = ["tests/test_oracle_gemm.py", "tests/test_oracle_mfma_model.py",
                "tests/test_oracle_fp8_model.py", "tests/test_oracle_fp8.py",
                "tests/test_oracle_sp24.py", "tests/test_oracle_bf16x3.py",
                "tests/test_oracle_formats.py", "tests/test_compare.py"]
HOST_TESTS = ["tests/test_abi_host.py"]
HOST_DESELECT = ("not exports and not create and not unknown_handles and not missing_library "
                 "and not binding_rejects")


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


needs_toolchain = pytest.mark.skipif(
    shutil.which("gcc") is None or shutil.which("g++") is None or _runtime("libasan.so") is None,
    reason="gcc with the address sanitizer runtime is required")


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    out = tmp_path_factory.mktemp("san")
    oracle_so = str(out / "libmpgemm_oracle_san.so")
    host_so = str(out / "libmpgemm_host_san.so")
    subprocess.run(["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                    "-fPIC", "-shared", *SAN, "-o", oracle_so,
                    os.path.join(ROOT, "oracle", "mpgemm_oracle.c"), "-lm"], check=True)
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared", "-Wall", *SAN,
                    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-o", host_so,
                    os.path.join(CSRC, "mpgemm_host.cpp")], check=True)
    return oracle_so, host_so


def _child(args, extra_env, timeout):
    env = dict(os.environ)
    env.update(extra_env)
    env["LD_PRELOAD"] = _runtime("libasan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["OMP_NUM_THREADS"] = "4"
    # -s: a sanitizer report goes to the terminal before the abort, not into pytest's capture
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
           "-m", "not gpu", *args]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    tail = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    return r.stdout


@needs_toolchain
def test_oracle_pins_under_address_and_ub_sanitizers(sanitized):
    oracle_so, _ = sanitized
    out = _child(ORACLE_TESTS, {"MPGEMM_ORACLE_LIB": oracle_so}, timeout=900)
    assert " passed" in out


@needs_toolchain
def test_host_checks_under_address_and_ub_sanitizers(sanitized):
    _, host_so = sanitized
    out = _child([*HOST_TESTS, "-k", HOST_DESELECT], {"MPGEMM_HOST_CHECK_LIB": host_so},
                 timeout=300)
    assert " passed" in out
