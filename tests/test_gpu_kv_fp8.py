"""Static FP8 KV-cache quantisation on the GPU (through the C ABI) against
the oracle: bytes bit-exact for every input dtype, strided rows, saturation,
signed zeros and subnormal ties; the scale from the calibration observer is
bit-exact too."""
import sys

import numpy as np
import pytest

from nvfp4_w4a4_block_quantize_amd import synth
from oracle import nvfp4_oracle as O

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def log(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def to_dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return {"f32": t, "bf16": t.to(torch.bfloat16), "f16": t.to(torch.float16)}[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_kv_fp8_matches_oracle(gpu_lib, dtype):
    nv = gpu_lib
    # K/V-shaped activations: tokens x (8 heads x 128), calibrated on a separate draw
    x, oc = synth.activations(3, "long", 700, 1000, 1024, dist="t3", bf16=(dtype == "bf16"))
    xc, _ = synth.activations(3, "long", 701, 1000, 1024, dist="t3", bf16=(dtype == "bf16"), outlier_cols=oc)
    if dtype == "f16":
        x, xc = x.astype(np.float16).astype(np.float32), xc.astype(np.float16).astype(np.float32)
    log("kv fp8", dtype, x.shape)
    state = torch.zeros(1, dtype=torch.float32, device="cuda")
    nv.nvfp4_amax_observe(to_dev(xc, dtype), state)
    s = nv.nvfp4_kv_scale_from_amax(state)
    q = nv.nvfp4_kv_quantize_fp8(to_dev(x, dtype), s)
    torch.cuda.synchronize()
    ref_s = O.kv_scale_ref(O.calibrate_ref([xc])[0])
    assert np.float32(s.item()) == ref_s
    assert np.array_equal(q.cpu().numpy(), O.kv_quantize_ref(x, ref_s))


def test_kv_fp8_edges_and_strides(gpu_lib):
    nv = gpu_lib
    vals = np.array([1.0, -1.5, 448.0, 500.0, -1e6, -0.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 17.0, 0.0, -2.0 ** -12,
                     447.9, 464.0, 1e-30, 3.0e4], dtype=np.float32)
    x = np.tile(vals, (24, 4))  # 24 x 64
    big = np.full((24, 96), 7.0e5, dtype=np.float32)
    big[:, :64] = x
    t = torch.from_numpy(big).cuda()[:, :64]  # ldx 96 > cols 64
    for sv in (1.0, 0.5, 3.0):
        s = torch.tensor([sv], dtype=torch.float32, device="cuda")
        q = nv.nvfp4_kv_quantize_fp8(t, s)
        torch.cuda.synchronize()
        log("kv fp8 edges", sv)
        assert np.array_equal(q.cpu().numpy(), O.kv_quantize_ref(x, np.float32(sv)))
