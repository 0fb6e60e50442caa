"""The host planner under AddressSanitizer and UndefinedBehaviorSanitizer.

fsdp_flat.cpp (validation, layout, descriptor-table construction, plan
cache) is built with g++ -fsanitize=address,undefined, without the device
kernels, and driven by tests/host_sanitizer_driver.cpp over ragged, empty,
non-zero-dim and misaligned buckets.  With no GPU visible every call plans
in full and then fails its upload (FSDP_EHIP), so any out-of-bounds access,
overflow or leak in the planner is reported.  CPU only.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hsdp_parameter_gradient_amd", "csrc")


def test_planner_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if not gxx or not os.path.exists("/opt/rocm/lib/libamdhip64.so"):
        pytest.skip("needs g++ and the ROCm runtime library")
    exe = str(tmp_path / "host_sanitizer_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "fsdp_flat.cpp"), os.path.join(ROOT, "tests", "host_sanitizer_driver.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    if r.stdout.strip() == "skip":
        pytest.skip("a GPU is visible: the driver needs the uploads to fail")
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout + r.stderr)[-4000:]
