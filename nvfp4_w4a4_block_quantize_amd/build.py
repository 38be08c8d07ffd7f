"""Builds libnvfp4.so (the HIP kernels and the C ABI) in-tree for gfx950.

Every HIP source is compiled with hipcc for --offload-arch=gfx950 only; the
library is written next to this file so it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libnvfp4.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
# not part of the library: a test program and the bench's measurement probes,
# each built beside the file that uses it
CONFORMANCE_SRC = os.path.join(ROOT, "tests", "conformance_cvt.hip")
CONFORMANCE_PATH = os.path.join(ROOT, "tests", "conformance_cvt")
PROBES_SRC = os.path.join(ROOT, "bench_probes.hip")
PROBES_PATH = os.path.join(ROOT, "libnvfp4_probes.so")

SOURCES = ["nvfp4_abi.cpp", "quantize.hip", "fuse_rescale.hip", "gemm.hip", "gemm_fast.hip", "gemm_decode.hip", "gemm_stream.hip", "kv_quantize.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",  # the quantiser's fp32 steps are single IEEE operations, never fused
    "-fno-gpu-flush-denormals-to-zero",
    # packed fp32 VALU instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libnvfp4.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    # conformance check of the conversion instructions the kernels rely on
    # (a standalone program, run by the GPU tests)
    cmd = [HIPCC, *COMMON_FLAGS, CONFORMANCE_SRC, "-o", CONFORMANCE_PATH + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for conformance_cvt.hip:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(CONFORMANCE_PATH + ".tmp", CONFORMANCE_PATH)
    # measurement probes for the benchmark (MFMA-only loop, streaming read)
    cmd = [HIPCC, *COMMON_FLAGS, "-shared", PROBES_SRC, "-o", PROBES_PATH + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for bench_probes.hip:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(PROBES_PATH + ".tmp", PROBES_PATH)
    if verbose:
        print(f"built {LIB_PATH}, {CONFORMANCE_PATH} and {PROBES_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
