"""The CPU oracle built with sanitizers (host code only, gcc; no GPU).

The oracle's C source and a small driver (tests/sanitize/oracle_driver.c)
are built twice, with AddressSanitizer + UndefinedBehaviorSanitizer and
with ThreadSanitizer, and run: exactly sized buffers, the 3-thread paths,
full versus sampled forms, the exact zero-weight closed form and the
invalid-argument paths.  Any sanitizer report fails the test.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "oracle", "fconv_oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c")]
FLAGS = ["-std=c99", "-D_POSIX_C_SOURCE=200809L", "-O1", "-g", "-fno-omit-frame-pointer", "-pthread", "-Wall",
         "-Wextra", "-Werror"]


def build_and_run(tmp_path, name, sanitize, env_extra):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / name)
    cmd = ["gcc", *FLAGS, *sanitize, "-o", exe, *SRC, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, **env_extra)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "all checks passed" in r.stdout
    assert "ERROR" not in r.stderr and "WARNING" not in r.stderr, r.stderr[-4000:]


def test_oracle_asan_ubsan(tmp_path):
    build_and_run(tmp_path, "oracle_asan", ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
                  {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0", "UBSAN_OPTIONS": "print_stacktrace=1"})


def test_oracle_tsan(tmp_path):
    build_and_run(tmp_path, "oracle_tsan", ["-fsanitize=thread"], {"TSAN_OPTIONS": "halt_on_error=1"})
