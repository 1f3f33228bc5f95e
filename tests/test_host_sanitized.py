"""The C-ABI host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): build api.hip with host-side sanitizers and launch stand-ins
that abort if reached, then run tests/test_abi.py against that library in a
child process with the sanitizer runtime preloaded.  Validation, workspace
sizing and every error path those tests take must run clean: no sanitizer
report, and no launch reached."""
import os
import subprocess
import sys

import pytest

from long_context_decode_fd_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_clean_under_asan_and_ubsan():
    try:
        lib = B.build_sanitized_host()
        runtime = B.sanitizer_runtime()
    except RuntimeError as e:   # no hipcc / sanitizer runtime on this host
        pytest.skip(str(e))
    env = dict(os.environ)
    env.update(
        FD_AMD_LIB=lib,
        LD_PRELOAD=runtime,
        # Python itself is not instrumented and keeps its arenas: leak
        # reports would be about the interpreter, not the library
        ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
        UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
    )
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=600)
    out = p.stdout
    assert p.returncode == 0, out[-4000:]
    for marker in ("AddressSanitizer", "runtime error:", "LeakSanitizer", "launch was reached"):
        assert marker not in out, out[-4000:]
    assert " passed" in out
