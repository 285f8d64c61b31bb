"""The host side of libmdt under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Every source is built with the sanitizers on its host compilation
(``build.build_host_sanitized``), and the host tests (exports, tree builders, every
entry point's argument checks) run against that build in a subprocess with the
sanitizer runtime preloaded; any report aborts the subprocess.  No kernel runs: every
call there fails validation before a launch, or is host-only code.
"""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.timeout(900)
def test_host_checks_clean_under_asan_and_ubsan():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime under /opt/rocm/llvm")
    sys.path.insert(0, os.path.join(ROOT, "medusa_tree_verification_heads_amd"))
    try:
        import build
    finally:
        sys.path.pop(0)
    lib = build.build_host_sanitized(verbose=False)
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, MDT_LIB_PATH=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_lib_host.py"), "-q",
                        "-p", "no:cacheprovider", "-x"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "failed" not in r.stdout, tail
