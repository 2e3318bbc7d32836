"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer
(host code only): oracle/selftest.c drives every entry point on small inputs
at all bit widths and page sizes."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "selftest")
    cmd = ["gcc", "-O1", "-g", "-std=gnu11", "-ffp-contract=off", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "kvq_oracle.c"), os.path.join(ROOT, "oracle", "selftest.c"),
           "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "selftest: ok" in r.stdout
