"""The gfx950 conversion instructions the kernels rely on, checked against the
rules they implement: the quantiser's E2M1 encoding, the GEMM epilogue's
fp32 -> bf16 rounding and the FP8 KV quantiser's E4M3 encoding for every
non-NaN fp32 input, and the GEMM's E2M1 / E4M3 decodes for every code (see
tests/conformance_cvt.hip, built beside it by the package's build step)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "conformance_cvt")


def test_conversion_instructions_match_the_format_rules(gpu_lib):
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: build the package first (build.build())")
    print("[case] conformance_cvt", flush=True)
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=100)
    print(res.stdout, flush=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.count(": 0 mismatches") == 4, res.stdout
