"""The host side of libvegas.so (csrc/api.cpp: validation, split planning, workspace layout) built
for the CPU under AddressSanitizer and UndefinedBehaviorSanitizer, with the kernel launchers
replaced by stubs that capture what the host computed.  tests/host_plan_check.cpp calls every
planning entry point on 120,000 seeded random batches (1..1024 sequences, empty, short, equal and
ragged lengths, paged caches, local windows, up to 64 query rows per KV head) and checks the bounds
the kernels rely on: split counts within the partial slots and the grid, every sequence covered by
non-empty splits no longer than the LDS buffers, the balanced plan's tables, workspace regions and
the selection's geometry.  An undersized bound there would be an out-of-bounds device write."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "verification_guided_sparse_verify_amd", "csrc")
HIP_INCLUDE = "/opt/rocm/include"


def test_host_plan_bounds_under_asan_and_ubsan(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ is not available")
    if not os.path.isdir(os.path.join(HIP_INCLUDE, "hip")):
        pytest.skip("HIP headers are not installed")
    exe = tmp_path / "host_plan_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host_plan_check.cpp"), "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "asan" in build.stderr.lower():
        pytest.skip("this g++ has no sanitizer runtime")
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1")
    seen_balanced = seen_multiround = 0
    for seed, n in ((1, 60000), (2, 60000)):
        run = subprocess.run([str(exe), str(n), str(seed)], capture_output=True, text=True, env=env, timeout=600)
        assert run.returncode == 0, run.stdout + run.stderr
        assert run.stdout.startswith(f"ok {n} cases"), run.stdout
        seen_balanced += int(run.stdout.split(",")[1].split()[0])
        seen_multiround += int(run.stdout.split(",")[2].split()[0])
    # the ragged batches exercise the balanced plan's tables too, and long sequences (or small
    # pages) the plans over several rounds of workgroups
    assert seen_balanced >= 1000, seen_balanced
    assert seen_multiround >= 1000, seen_multiround
