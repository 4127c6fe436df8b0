"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code
(CPU only): the oracle (oracle/mx_oracle.c) and the C-ABI validation layer
(mx_api.cpp with stub launchers).  A subprocess that preloads the ASan
runtime runs the oracle's pin tests and the C-ABI tests against those
builds, then calls every entry point with valid arguments down to the
(stubbed) launch; any sanitizer report aborts it."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "sanitize"))


def test_sanitized_oracle_and_validation_layer():
    import build
    try:
        build.build()
    except (OSError, RuntimeError) as e:
        pytest.fail(f"sanitizer build failed: {e}")
    env = dict(os.environ)
    env["LD_PRELOAD"] = build.runtime_preload()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1:allocator_may_return_null=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, os.path.join(HERE, "sanitize", "driver.py")], env=env,
                       capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "sanitized valid calls" in out
