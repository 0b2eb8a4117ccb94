"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds oracle/moe_oracle.c together with tests/sanitize/oracle_sanitize_main.c
(a driver that calls every oracle entry point on small inputs allocated at
their exact sizes, edge cases included) with gcc's -fsanitize=address,undefined
and runs it; any out-of-bounds access, use after free, leak or undefined
behaviour aborts the run.  CPU only (no GPU code is built here).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "moe_oracle.c")
DRIVER_C = os.path.join(ROOT, "tests", "sanitize", "oracle_sanitize_main.c")


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitize")
    flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-fopenmp", "-ffp-contract=off", "-std=c11"]
    build = subprocess.run(["gcc", *flags, ORACLE_C, DRIVER_C, "-o", exe, "-lm"],
                           capture_output=True, text=True)
    if build.returncode != 0 and "asan" in build.stderr.lower():
        pytest.skip("gcc has no sanitizer runtime here: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, (run.stdout[-2000:] + run.stderr[-4000:])
    assert "all calls ok" in run.stdout
