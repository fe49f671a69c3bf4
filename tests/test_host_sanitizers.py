"""The C-ABI host layer (argument validation, workspace sizing, dispatch:
qsa_api.hip) built with AddressSanitizer and UBSan on the host pass only,
with UB fatal, runs the ABI host tests (tests/test_abi_host.py) in a
subprocess that preloads the ASan runtime.  No GPU: every call in those
tests returns before anything is launched."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC) or not os.path.exists("/opt/rocm/llvm/bin/clang++"),
                    reason="ROCm toolchain not available")
def test_abi_host_tests_under_asan_and_ubsan():
    from block_sparse_trainable_amd import build as Bd
    out = os.path.join(ROOT, "_build", "libqsa_san.so")
    Bd.build_sanitized(out)
    syms = subprocess.run(["nm", "-D", out], capture_output=True, text=True, check=True).stdout
    assert "__asan_init" in syms or "__asan_report_load" in syms, "library is not instrumented"
    assert "__ubsan_handle" in syms, "library is not instrumented for UB"
    env = dict(os.environ)
    env.update({"QSA_LIBRARY": out, "LD_PRELOAD": Bd.asan_runtime(),
                "ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    code = ("import sys, pytest\n"
            "from block_sparse_trainable_amd import _binding as B\n"
            f"assert B.library_path() == {out!r}, B.library_path()\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', "
            "'tests/test_abi_host.py']))\n")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=600)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert " passed" in res.stdout, tail
