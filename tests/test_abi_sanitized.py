"""The argument validation of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer: every case of test_abi_cpu.py (bad shapes,
pointers, alignment, workspaces, the allocation-free variant's limit, the
labeller's checks) run against the same sources built with both sanitizers
on the host code (tests/_build/libhas_san.so, built by build()), in a
subprocess that preloads the sanitizer runtime.  Any invalid memory access or
undefined behaviour in the host code aborts that process.  No GPU needed."""
import os
import subprocess
import sys

from head_aware_sparse_amd import _build

RUNNER = r"""
import sys
sys.path.insert(0, {root!r})
import head_aware_sparse_amd.binding as b
b._LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu", {test!r}]))
"""


def test_validation_cases_under_sanitizers():
    assert os.path.exists(_build.SAN_LIB), "sanitized library missing: run __graft_entry__.build()"
    rt = _build.asan_runtime()
    assert rt, "clang AddressSanitizer runtime not found"
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    code = RUNNER.format(root=_build.ROOT, lib=_build.SAN_LIB, test=os.path.join(_build.ROOT, "tests", "test_abi_cpu.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600,
                       cwd=_build.ROOT)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
