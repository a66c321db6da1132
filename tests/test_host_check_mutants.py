"""The host ABI tests catch mistakes in the library's host-only argument checks: each mistake
below, planted in one function of a copy of csrc/mpgemm_host.cpp (built alone with g++ and
loaded through MPGEMM_HOST_CHECK_LIB, as the sanitizer test does), makes at least one test of
tests/test_abi_host.py fail.  CPU only."""
import shutil

import pytest

from tests.planted import host_survivors

# the host ABI tests that need no device and no HIP library symbol
HOST_TESTS = ["tests/test_abi_host.py"]
HOST_ONLY = ("not exports and not create and not unknown_handles and not missing_library "
             "and not binding_rejects")
CHK = "mpgemm_status_t mpgemm_check("
SP = "mpgemm_status_t mpgemm_check_sp24("

# name: (function the mistake is planted in, original text, planted text)
CODE = {
    "lda checked against the wrong size": (
        CHK, "const int64_t min_lda = ta ? m : k,", "const int64_t min_lda = ta ? k : m,"),
    "ldb checked against the wrong size": (CHK, "min_ldb = tb ? k : n,", "min_ldb = tb ? n : k,"),
    "C's alignment not checked": (
        CHK, "if (!aligned16(D) || (read_c && !aligned16(C)))", "if (!aligned16(D))"),
    "C required although beta is zero": (CHK, "if (read_c && !C) return", "if (!C) return"),
    "ldc's byte stride not checked": (
        CHK, "if ((lda * ea) % 16 || (ldb * ea) % 16 || (ldc * ec) % 16)",
        "if ((lda * ea) % 16 || (ldb * ea) % 16)"),
    "k up to INT32_MAX accepted": (CHK, "k > kMaxK", "k > INT32_MAX"),
    "stride limit not checked": (
        CHK, "if (lda > max_ld(ea) || ldb > max_ld(ea) || ldc > max_ld(ec)) "
             "return MPGEMM_STATUS_NOT_SUPPORTED;", ""),
    "null A accepted": (CHK, "if (k > 0 && (!A || !B)) return", "if (k > 0 && !B) return"),
    "negative sizes accepted": (
        CHK, "if (m < 0 || n < 0 || k < 0) return MPGEMM_STATUS_INVALID_VALUE;", ""),
    "sparse: k a multiple of 64 accepted": (SP, "if (k % 128)", "if (k % 64)"),
    "sparse: metadata stride not checked": (SP, "ld_meta < (k / 8 > 1 ? k / 8 : 1) ||", ""),
    "sparse: metadata alignment not checked": (SP, "!aligned16(meta) || ", ""),
    "sparse: mixed 16-bit inputs accepted": (
        SP, "} else if (a_type != b_type) {\n        return MPGEMM_STATUS_NOT_SUPPORTED;\n    }",
        "}"),
    "beta = -0 taken as nonzero": (
        "bool beta_is_zero(", "    return b == 0.0f;",
        "    uint32_t u; memcpy(&u, &b, sizeof u); return u == 0;"),
    "three-BF16 workspace: B not 256-byte aligned": (
        "bool bf16x3_layout(", "const unsigned __int128 off_b = (bytes_a + 255) / 256 * 256;",
        "const unsigned __int128 off_b = bytes_a;"),
    "three-BF16 workspace: k not padded to 8": (
        "bool bf16x3_layout(", "L.k3 = 3 * ((k + 7) / 8 * 8);", "L.k3 = 3 * k;"),
}


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ builds the mutated host checks")
def test_every_planted_host_check_mistake_fails_a_test():
    assert host_survivors(CODE, HOST_TESTS, args=("-k", HOST_ONLY)) == []


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ builds the host checks")
def test_the_unchanged_host_checks_pass_the_tests():
    same = "if (k > 0 && (!A || !B)) return"
    assert host_survivors({"unchanged": (CHK, same, same)}, HOST_TESTS,
                          args=("-k", HOST_ONLY)) == ["unchanged"]
