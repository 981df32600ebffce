"""The C-ABI argument tests (tests/test_abi.py) again, against a build of
the library whose host code is compiled with AddressSanitizer and
UndefinedBehaviorSanitizer (text_image_flow_amd.build.build_sanitized: the
sanitizer flags apply to the host pass only).  Runs on the CPU in a child
process with the ASan runtime preloaded; any sanitizer report aborts the
child and fails this test.  No compute call is made."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_tests_pass_under_host_asan_and_ubsan():
    from text_image_flow_amd import build as B
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    lib = B.build_sanitized()
    rt = B.asan_runtime()
    assert os.path.isabs(rt) and os.path.exists(rt), rt
    env = dict(os.environ, LD_PRELOAD=rt, LENS_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    tail = "\n".join((r.stdout + r.stderr).splitlines()[-40:])
    assert r.returncode == 0, tail
    assert "Sanitizer" not in r.stdout + r.stderr, tail
    assert " passed" in r.stdout, tail
