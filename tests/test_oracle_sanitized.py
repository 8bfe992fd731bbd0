"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only): gcc builds
oracle/sage_oracle.c with -fsanitize=address,undefined into the driver tests/oracle_sanitized_main.c,
which calls every entry point on small seeded inputs (ragged tiles, every format and role, causal
and not, selected rows, slack and lse, rejected arguments). Any invalid access, leak or undefined
behaviour makes the run fail with the sanitizer's report."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "sage_oracle.c"), os.path.join(HERE, "oracle_sanitized_main.c"),
           "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "all entry points ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
