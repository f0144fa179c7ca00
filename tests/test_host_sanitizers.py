"""The host-side ABI tests again, against the library's host code built with
AddressSanitizer and UndefinedBehaviorSanitizer (head_routed_sparse_amd/build_sanitize.py):
any out-of-bounds access, use after free or undefined behaviour in argument validation,
layout, ring bookkeeping, planning or the host reductions aborts the run."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_tests_pass_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from head_routed_sparse_amd import build_sanitize as bs
    lib = bs.build()
    env = dict(os.environ, HEADCAST_LIBRARY=lib, LD_PRELOAD=bs.runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_host_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "Sanitizer" not in r.stderr, tail
