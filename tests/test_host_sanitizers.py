"""The host side of libtq (argument checks, codebooks, matrices, sizes, error
paths) under AddressSanitizer and UndefinedBehaviorSanitizer: the host-only
tests of test_lib_host.py run against a build of tq_host.cpp with both
sanitizers (device code unchanged), in a child process with the ASan runtime
preloaded.  Any report fails the run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_host_library_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from kv_cache_compression_04_amd import build_lib
    try:
        rt = build_lib.sanitizer_runtime()
        lib = build_lib.build_sanitized(str(tmp_path))
    except RuntimeError as e:  # pragma: no cover - toolchain without sanitizer runtimes
        pytest.skip(f"no sanitizer toolchain: {e}")
    env = dict(os.environ, LD_PRELOAD=rt, TQ_LIBRARY=lib, PYTHONMALLOC="malloc",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_lib_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
