"""The C-ABI host code (argument checks, sizes, launch set-up) under AddressSanitizer and
UndefinedBehaviorSanitizer: every host-side case of test_abi.py runs against a library whose
fp2_api.cpp / fp2_validate.cpp are built with both sanitizers (block_sparse_long_blocks_amd/build.py,
build_sanitized), in a child process with the sanitizer runtime preloaded.  A sanitizer report
aborts the child, so the test fails on any out-of-bounds access, use after free, signed overflow,
misaligned or null access in those files.  No GPU is used: every case is rejected or sized on the
host before any launch."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location("fp2_build_san", os.path.join(ROOT, "block_sparse_long_blocks_amd",
                                                                               "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_abi_host_checks_under_asan_and_ubsan():
    b = _build_module()
    lib = b.build_sanitized()
    env = dict(os.environ, FP2_TEST_LIBRARY=lib, LD_PRELOAD=b.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the two cases that build or copy the package are not about the host checks
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
           "-p", "no:cacheprovider", "-k", "not build_entry and not no_fallback"]
    r = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in r.stdout and "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
