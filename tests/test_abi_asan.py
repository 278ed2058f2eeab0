"""The C ABI's host code (validation, the AutoCP planner, workspace layout and
argument checks of gdn_api.cpp) built for the CPU with AddressSanitizer and
UndefinedBehaviorSanitizer, the kernel launchers replaced by stand-ins, and
driven through many descriptors (tests/asan/abi_driver.cpp). No GPU: every
case fails validation before a launch or reaches the stand-ins."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_deltanet_chunked_03_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "asan")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists("/opt/rocm/lib/libamdhip64.so"),
                    reason="needs g++ and the HIP runtime library")
def test_host_code_under_sanitizers(tmp_path):
    exe = tmp_path / "abi_asan"
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(CSRC, "gdn_api.cpp"), os.path.join(HERE, "abi_stubs.cpp"), os.path.join(HERE, "abi_driver.cpp"),
           "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0 and "ok" in run.stdout, (run.stdout[-2000:], run.stderr[-4000:])
