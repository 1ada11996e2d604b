"""The library's host-side descriptor checks and split planner under the
address and undefined-behaviour sanitizers (CPU only).

tests/host_check.cpp includes the same host headers the C ABI's entry points
use (validation, launch planning) and is built here with g++ and
-fsanitize=address,undefined (no GPU code is involved).  It fuzzes seeded
descriptors with extreme field values (every one must give a status code,
and every valid one must plan within its bounds at 1 to 1024 compute units)
and checks that the plan's grid, workspace and one-resident-round bound
follow the device's compute-unit count at 32, 80 and 256 CUs.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host_check.cpp")


@pytest.fixture(scope="module")
def host_check(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("host") / "host_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include",
           f"-I{ROOT}/paged_asymmetric_head_amd/csrc", "-I/opt/rocm/include", SRC, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    return exe


def run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe, *args], capture_output=True, text=True, env=env, timeout=300)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_descriptor_fuzz_under_sanitizers(host_check, seed):
    run(host_check, "fuzz", str(seed), "200000")


def test_plan_scales_with_compute_units(host_check):
    run(host_check, "scale")


def test_multiply_high_division_is_exact(host_check):
    run(host_check, "fastdiv")
