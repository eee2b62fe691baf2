"""The ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds the library with host-side sanitizers (weight_quantized_mlp_amd.build.SAN_FLAGS; the gfx950 code
objects are unchanged) and runs tests/test_abi.py against it in a child process with the ASan runtime
preloaded: every validation path of every entry point then runs with bounds, use-after-free and
undefined-behaviour checks, and any report fails the run.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.cpu


def test_abi_checks_under_host_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from weight_quantized_mlp_amd import build as b
    try:
        hipcc = b._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang")
    rt = subprocess.run([clang if os.path.exists(clang) else "/opt/rocm/llvm/bin/clang",
                         "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.exists(rt):
        pytest.skip("no ASan runtime")
    lib = b.build(sanitize=True, out=str(tmp_path / "libwqmlp.so"))
    env = dict(os.environ, WQMLP_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = p.stdout + p.stderr
    assert p.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
