"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer:
a driver calls every entry point on small ragged shapes with exactly sized
buffers, built with gcc -fsanitize=address,undefined and no recovery, so any
out-of-bounds access, use of freed memory or undefined arithmetic aborts the
run.  The same driver built without sanitizers must print the same checksum
(the instrumented build computes the same bits)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE = os.path.join(os.path.dirname(HERE), "oracle")
SRCS = [os.path.join(ORACLE, f) for f in ("bi_oracle.c", "bi_oracle_layer.c",
                                          "bi_oracle_sample.c")]
DRIVER = os.path.join(HERE, "oracle_sanitize_driver.c")
# the oracle's own arithmetic flags (no contraction, no fast math)
BASE = ["-std=c11", "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra", "-I", ORACLE]


def _build_and_run(tmp_path, name, extra):
    exe = str(tmp_path / name)
    subprocess.check_call(["gcc", *BASE, *extra, "-o", exe, DRIVER, *SRCS, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_asan_and_ubsan(tmp_path):
    san = _build_and_run(tmp_path, "oracle_san", [
        "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
        "-fno-sanitize-recover=all"])
    assert san.returncode == 0, san.stdout + san.stderr
    assert "runtime error" not in san.stderr and "AddressSanitizer" not in san.stderr
    plain = _build_and_run(tmp_path, "oracle_plain", ["-O2"])
    assert plain.returncode == 0, plain.stderr
    assert san.stdout.startswith("ok ") and san.stdout == plain.stdout
