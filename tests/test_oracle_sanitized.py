"""The fp64 oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

mala_oracle.c addresses its arrays with hand-written index arithmetic (tiles,
blocks, packed sequences, unit lists, cache lengths).  This builds it with
gcc, -fsanitize=address,undefined and -fno-sanitize-recover=all, together with
tests/oracle_sanitize_driver.c, which calls every entry point on small ragged
shapes with exactly sized heap arrays, and runs the program on the CPU: any
out-of-bounds access, use after free, leak or undefined operation ends it
with a report and a non-zero status.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_C = os.path.join(os.path.dirname(HERE), "oracle", "mala_oracle.c")
DRIVER_C = os.path.join(HERE, "oracle_sanitize_driver.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = tmp_path / "oracle_sanitized"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-Wall", "-Wno-unknown-pragmas",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           ORACLE_C, DRIVER_C, "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    assert "all calls OK" in r.stdout
