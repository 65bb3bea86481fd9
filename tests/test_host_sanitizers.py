"""The host suites (C-ABI validation, planning, budgets, the plain-C consumer, bench's host logic) run
against a build of the library whose host code is under AddressSanitizer and UndefinedBehaviorSanitizer.
CPU only: no kernel is launched; device code is compiled as usual and not instrumented."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from block_sparse_attention_oam_amd import build as b  # noqa: E402


def test_host_suites_pass_under_asan_and_ubsan():
    try:
        b._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    rt = b.asan_runtime()
    if not os.path.exists(rt):
        pytest.skip("clang's ASan runtime not found")
    lib = b.build_host_sanitized(verbose=False)
    env = dict(os.environ, STEM_LIB=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_abi_host.py"), os.path.join(ROOT, "tests", "test_bench_host.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
