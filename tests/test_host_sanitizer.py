"""The host half of libpagedkv under AddressSanitizer and
UndefinedBehaviorSanitizer: pool.cpp, prefix.cpp and plan.cpp are built with
g++ -fsanitize=address,undefined (device launches stubbed out, see
csrc/sanitize_stubs.cpp) and the host test suites -- the allocator, slot
mapping and reservation properties against the oracle, the prefix cache,
copy-on-write and window release, every argument check -- run in a child
process that loads that build.  Any sanitizer report aborts the child and
fails the test.  The checks of the gather probe and of the no-allocation
step are left out: they sit in device sources, which this build does not
contain."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def san_lib():
    import paged_kv_cache_271_amd.build as b
    try:
        return b.build_host_sanitized()
    except (RuntimeError, FileNotFoundError) as e:   # no g++ sanitizer runtime in this image
        pytest.skip(f"sanitizer build unavailable: {e}")


def test_host_suites_clean_under_asan_ubsan(san_lib):
    import paged_kv_cache_271_amd.build as b
    env = b.sanitizer_env(san_lib)
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           "-k", "not probe_argument_checks and not noalloc",
           os.path.join(ROOT, "tests", "test_host_library.py"), os.path.join(ROOT, "tests", "test_host_prefix.py")]
    r = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert " passed" in out and "failed" not in out
