"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only): a small
C driver calls every entry point, including empty prefixes and empty lists, and any invalid
access or undefined operation aborts it."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    exe = tmp_path / "oracle_sanitize"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "vegas_oracle.c"), os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"),
           "-lm", "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "asan" in build.stderr.lower():
        pytest.skip("this gcc has no sanitizer runtime")
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, OMP_NUM_THREADS="4", ASAN_OPTIONS="detect_leaks=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "ok" in run.stdout
