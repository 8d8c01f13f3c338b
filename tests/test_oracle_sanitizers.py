"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer: a
driver calls every function of oracle/fp8_oracle.c on small ragged and
strided inputs held in exactly sized heap buffers (tests/
oracle_sanitize_driver.c); any out-of-bounds access or undefined operation
aborts the run.  Host code only, built with gcc."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_runs_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "fp8_oracle.c"), os.path.join(HERE, "oracle_sanitize_driver.c"),
           "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    # verify_asan_link_order=0: a library preloaded by the environment may
    # come before the ASan runtime in the load order
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle sanitizer run: ok" in r.stdout
    assert "runtime error" not in r.stderr, r.stderr
