"""The C-ABI layer (csrc/nvfp4_abi.cpp) built for the host alone with
AddressSanitizer and UndefinedBehaviorSanitizer, its kernel launchers replaced
by stubs (tests/abi_sanitize/launch_stubs.cpp), then the ctypes ABI tests run
against it in a child process with the ASan runtime preloaded.  Any invalid
memory access or undefined behaviour in argument validation, status mapping
or the CU-count cache aborts the child."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "nvfp4_w4a4_block_quantize_amd", "csrc")


def _rocm():
    for p in (os.environ.get("ROCM_PATH"), "/opt/rocm"):
        if p and os.path.exists(os.path.join(p, "include", "hip", "hip_runtime.h")):
            return p
    return None


def test_abi_layer_under_asan_and_ubsan(tmp_path):
    gxx, rocm = shutil.which("g++"), _rocm()
    if gxx is None or rocm is None:
        pytest.skip("needs g++ and the HIP headers")
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("no ASan runtime for g++")
    lib = str(tmp_path / "libnvfp4_abi_sanitized.so")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "nvfp4_abi.cpp"), os.path.join(ROOT, "tests", "abi_sanitize", "launch_stubs.cpp"),
           "-o", lib, "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, NVFP4_ABI_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    try:
        import torch

        if torch.cuda.device_count() == 0:
            env["NVFP4_NO_GPU"] = "1"  # the child then also runs the no-device calls
    except ImportError:
        pass
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"), "-k", "not binding"],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
