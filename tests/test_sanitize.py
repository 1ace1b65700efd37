"""AddressSanitizer + UndefinedBehaviorSanitizer run of the CPU oracle and the
input generator (host code only, gcc): tests/sanitize/driver.c calls every
exported function of oracle/oracle.c and synth/gen.c on small inputs and edge
cases; any out-of-bounds access, leak or undefined operation aborts it."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_and_generator_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "sanitized")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-mfma", "-ffp-contract=off", "-pthread",
           os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "synth", "gen.c"),
           os.path.join(ROOT, "tests", "sanitize", "driver.c"), "-o", exe, "-lm"]
    b = subprocess.run(cmd, capture_output=True, text=True)
    if b.returncode != 0 and "asan" in (b.stderr or "").lower() and "cannot find" in (b.stderr or "").lower():
        pytest.skip("sanitizer runtime not installed")
    assert b.returncode == 0, b.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1", ORACLE_THREADS="3")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "sanitized run ok" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr
