"""The C ABI layer (csrc/nvkv_api.cpp) built for the CPU with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer, with stub launchers (tests/native/abi_host_driver.cpp), and driven
through every validation, planning, sizing and dispatch path; any sanitizer report fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIP_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(HIP_INCLUDE),
                    reason="needs g++ and the HIP headers")
def test_abi_layer_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_host_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I" + HIP_INCLUDE,
           os.path.join(ROOT, "bit_paged_kv_amd", "csrc", "nvkv_api.cpp"),
           os.path.join(ROOT, "tests", "native", "abi_host_driver.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "0 failed" in run.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
