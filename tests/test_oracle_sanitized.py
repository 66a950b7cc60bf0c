"""Host sanitizers on the CPU oracle: every entry point runs under address and
undefined-behaviour sanitizer instrumentation (gcc, CPU only) on small
pseudo-random inputs -- both element formats, every combine transport, FP32
and double accumulation, the compact expert map -- and must finish without a
report."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-std=c99", "-g", "-O1", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(HERE, "oracle_sanitizer_driver.c"), os.path.join(ROOT, "oracle", "moe_oracle.c"),
           "-o", exe, "-lm"]
    build = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if build.returncode != 0 and "asan" in build.stdout.lower():
        pytest.skip("sanitizer runtime not installed: " + build.stdout[-200:])
    assert build.returncode == 0, build.stdout
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    run = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                         env=env, timeout=120)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), run.stdout[-4000:]
