"""The C-ABI argument checks of every entry point, built against host-only
launch stubs with the address and undefined-behaviour sanitizers (CPU only):
each case's status and whether it reaches a launch, including extreme sizes
for the 64-bit size arithmetic."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c", "host_checks")


def test_sanitized_host_checks():
    if not os.path.exists(BIN):
        pytest.fail(f"{BIN} is not built (run __graft_entry__.build())")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120, env=env)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "host_checks: ok" in res.stdout
