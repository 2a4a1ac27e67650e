"""The host-side ABI tests (tests/test_abi_host.py: exports, host helpers
against the oracle, argument errors before any launch) run again in a child
process against libpkv_hostsan.so, the library with its host code built
under AddressSanitizer and UndefinedBehaviorSanitizer; any report aborts the
child. No GPU is needed."""

import os
import subprocess
import sys

import pytest

from conftest import ROOT


def test_abi_host_tests_under_asan_and_ubsan():
    from paged_kv_attention_scatter_amd import build as b
    if not os.path.exists(b.SAN_LIB):
        b.build(sanitized=True)
    env = dict(os.environ)
    env.update(LD_PRELOAD=b.sanitizer_runtime(), PKV_LIB_PATH=b.SAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_host.py"), "-q",
                          "-p", "no:cacheprovider", "-m", "not gpu"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "Sanitizer" not in res.stderr, tail
    assert " passed" in res.stdout, tail
