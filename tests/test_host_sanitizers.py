"""The host code of the C ABI (argument validation, index maps, workspace
sizing) under AddressSanitizer and UndefinedBehaviorSanitizer: the ABI tests
run in a child process against the host-sanitizer build of libvda, with the
clang ASan runtime preloaded; any sanitizer report fails the test.  CPU only,
no compute call."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(600)
def test_abi_tests_pass_under_host_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from frame_wise_delta_amd import build_sanitized as bs
    lib = bs.build_sanitized()
    log = str(tmp_path / "san")
    env = dict(os.environ, VDA_LIBRARY=lib, LD_PRELOAD=bs.runtime(),
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:log_path={log}",
               UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=1:log_path={log}")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=540)
    reports = [open(os.path.join(tmp_path, f)).read() for f in sorted(os.listdir(tmp_path)) if f.startswith("san")]
    assert not reports, reports[0][-4000:]
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert " passed" in r.stdout
