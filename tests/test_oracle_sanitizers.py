"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: oracle/cgo.c
and a host driver (tests/oracle_sanitize_main.c) built with gcc, every entry point run
on small seeded caches with fp16 and 8-bit anchors, sinks, the outlier table, and
damaged payloads; any out-of-bounds access, leak or undefined behaviour ends the run
with an error."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-ffp-contract=off", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra",
           os.path.join(ROOT, "oracle", "cgo.c"), os.path.join(HERE, "oracle_sanitize_main.c"),
           "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stderr[-4000:]
    assert "oracle sanitizer run ok" in res.stdout
