"""The FP8 W8A8 comparison that bench.py times beside the W4A4 path is a
library call (hipBLASLt through torch._scaled_mm), so its figures are only a
baseline if the call computes what it claims.  Checked here on the GPU with
the same helpers bench.py times:

* the E4M3 bytes of both operands are the oracle's E4M3FN encoding (round to
  nearest even, the same encoder as the FP8 KV cache) of the fp32 values that
  were cast;
* the bf16 output equals the float64 product of those operands, decoded by
  the oracle and multiplied by the per-tensor decode scales, within the
  output's bf16 rounding plus an fp32 accumulation bound of K * 2^-24 of the
  sum of absolute products.
"""
import sys

import numpy as np
import pytest

import bench
from nvfp4_w4a4_block_quantize_amd import synth
from oracle import nvfp4_oracle as O

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def log(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("m,n,k", [(200, 1104, 2048), (32, 2048, 5120)])
def test_fp8_leg_is_the_product_of_its_own_e4m3_operands(gpu_lib, m, n, k):
    if not hasattr(torch, "float8_e4m3fn") or not hasattr(torch, "_scaled_mm"):
        pytest.skip("torch has no float8_e4m3fn / _scaled_mm")
    log("fp8 baseline", m, n, k)
    a, _ = synth.activations(11, "tiny", 901, m, k, dist="t3")
    w = synth.weights(11, "tiny", 902, n, k, row_outlier_fraction=0.01)
    a_dev = torch.from_numpy(a).cuda().to(torch.bfloat16)
    w_dev = torch.from_numpy(w).cuda()

    sa = bench.fp8_decode_scale(a_dev)
    sw = bench.fp8_decode_scale(w_dev)
    inv_sa = (1.0 / sa).to(a_dev.dtype)
    a8 = bench.fp8_activation(torch, a_dev, inv_sa)
    w8 = bench.fp8_weight(torch, w_dev, sw)
    c = bench.fp8_gemm(torch, a8, w8, sa, sw)
    # the fp32 values the casts above took as input, by the same expressions
    ya = (a_dev * inv_sa).float().cpu().numpy()
    yw = (w_dev.float() / sw).cpu().numpy()
    torch.cuda.synchronize()

    a8b = a8.view(torch.uint8).cpu().numpy()
    w8b = w8.view(torch.uint8).cpu().numpy()
    assert np.array_equal(a8b, O.kv_quantize_ref(ya, np.float32(1.0)))
    assert np.array_equal(w8b, O.kv_quantize_ref(yw, np.float32(1.0)))
    # the scales put the largest magnitude at 448 (up to the bf16 roundings)
    assert np.abs(ya).max() <= 448.0 * (1 + 2.0 ** -7)
    assert np.abs(yw).max() <= 448.0 * (1 + 2.0 ** -22)

    sa64, sw64 = float(sa.item()), float(sw.item())
    A = O.e4m3_decode(a8b) * sa64
    W = O.e4m3_decode(w8b) * sw64
    ref = A @ W.T
    basis = np.abs(A) @ np.abs(W).T
    got = c.float().cpu().numpy().astype(np.float64)
    tol = 2.0 ** -8 * np.abs(ref) + k * 2.0 ** -24 * basis
    err = np.abs(got - ref)
    assert np.all(err <= tol), f"worst excess {np.max(err - tol):.3e}"
