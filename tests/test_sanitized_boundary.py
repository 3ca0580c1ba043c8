"""The C-ABI layer (tattn.cpp) built by the host compiler with
AddressSanitizer and UndefinedBehaviorSanitizer, its kernel launchers
replaced by host stand-ins (tests/sanitize/launch_stub.cpp), and driven by
tests/sanitize/boundary_driver.cpp through every entry point with bad and
valid arguments on a host where no GPU is visible. The sanitizers abort the
driver on any memory error or undefined behaviour in the validation code."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_c_abi_under_address_and_ub_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("needs g++ and the HIP runtime library")
    exe = str(tmp_path / "boundary_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include",
           f"-I{ROOT}/tiled_attention_12_amd/csrc",
           os.path.join(ROOT, "tiled_attention_12_amd", "csrc", "tattn.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "launch_stub.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "boundary_driver.cpp"),
           f"-L{ROCM}/lib", f"-Wl,-rpath,{ROCM}/lib", "-lamdhip64", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1", CUDA_VISIBLE_DEVICES="-1",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr[-4000:]
    assert "all statuses as expected" in run.stdout
