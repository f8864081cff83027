"""Host sanitizers over the CPU oracle (test infrastructure, no GPU).

Builds the oracle's C source together with tests/sanitize/oracle_sanitize_main.c
under gcc's AddressSanitizer and UndefinedBehaviorSanitizer (recovery off, leak
checking on) and runs the driver, which calls every oracle entry point on
small inputs covering its branches.  A report from either sanitizer fails the
test."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c99", "-D_GNU_SOURCE", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(HERE, "sanitize", "oracle_sanitize_main.c"),
           os.path.join(ROOT, "oracle", "wedlm_oracle.c"), "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle sanitizer driver: ok" in r.stdout
