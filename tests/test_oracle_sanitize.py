"""The CPU oracle under gcc's AddressSanitizer and UndefinedBehaviorSanitizer:
tests/pins/oracle_sanitize.c drives every exported oracle function over
empty, ragged and strided shapes with buffers of exactly the needed size; any
out-of-bounds access, leak or undefined operation aborts it."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer",
                           "-fno-fast-math", "-ffp-contract=off",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-I", os.path.join(ROOT, "oracle"),
                           os.path.join(ROOT, "tests", "pins", "oracle_sanitize.c"),
                           os.path.join(ROOT, "oracle", "fp8_oracle.c"), "-o", str(exe), "-lm"])
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("OK"), (r.stdout[-2000:], r.stderr[-4000:])
