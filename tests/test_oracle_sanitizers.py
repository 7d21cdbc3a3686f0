"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Builds the oracle source together with ``oracle_sanitize_driver.c`` into one
host executable with gcc's ``-fsanitize=address,undefined`` (no GPU code is
involved) and runs it: every oracle entry point on small seeded inputs in
fp64, fp32 and bf16 storage, with padded cache strides and lengths 0, 1 and
full.  Any out-of-bounds access, use of freed memory, leak or undefined
behaviour aborts the run; the driver also checks the identities between the
entry points (absorbed = naive, prefill rows, W_UV of the merged latent, the
fold, the rotary embedding and the cache-size formula)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(HERE, "oracle_sanitize_driver.c"),
           os.path.join(ROOT, "oracle", "mla_oracle.c"), "-o", str(exe), "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=180)
    if build.returncode != 0 and "asan" in build.stderr.lower():
        pytest.skip("gcc's sanitizer runtimes are not installed: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="abort_on_error=0:halt_on_error=1:detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "all checks hold" in run.stdout, out[-4000:]
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
