"""The C ABI layer and the workspace layout under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU: api.cpp and layout.cpp are built with g++
and the sanitizers against tests/host/abi_harness.cpp, which replaces the HIP
runtime calls and the kernel launchers with stubs that write every workspace
region the kernels would write (into workspaces allocated at exactly the size the
library reports) and count live timing events."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_learnable_sinks_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the ROCm headers")
def test_abi_layer_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_harness")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", ROCM_INCLUDE,
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "layout.cpp"),
           os.path.join(ROOT, "tests", "host", "abi_harness.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    print(run.stdout[-2000:], run.stderr[-4000:])
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert "0 failed" in run.stdout
