"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host code only).

tests/oracle_sanitize_driver.c calls every oracle function over many shapes, modes and edge
cases with exactly sized heap buffers; built together with oracle/rmsq_oracle.c with the
sanitizers on, any out-of-bounds access, overflow or undefined shift aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no host C compiler")
    exe = str(tmp_path / "oracle_sanitize_driver")
    cmd = [gcc, "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "oracle"), os.path.join(ROOT, "oracle", "rmsq_oracle.c"),
           os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"), "-lm", "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr and "cannot find" in build.stderr:
        pytest.skip("sanitizer runtimes not installed")
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stderr[-4000:]
    assert "all calls ok" in run.stdout
