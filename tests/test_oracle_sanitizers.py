"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code, gcc) and driven through every entry point by
tests/oracle_sanitize_main.c: no memory error, leak or undefined behaviour,
and its internal consistency checks (thread counts agree, row offsets
continue the broadcast, rows sum to one, binary16 round trips) hold."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(ROOT, "oracle", "skipln_oracle.c"), os.path.join(HERE, "oracle_sanitize_main.c")]
FLAGS = ["-O1", "-g", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-ffp-contract=off", "-Wall", "-Wextra", "-Werror",
         "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed for the host-side sanitizer build")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    sanitize = "-fsanitize=" + ",".join(("address", "undefined"))
    build = subprocess.run(["gcc"] + FLAGS + [sanitize] + SOURCES + ["-lm", "-pthread", "-o", exe],
                           capture_output=True, text=True)
    assert build.returncode == 0, build.stdout + build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "all checks passed" in run.stdout
