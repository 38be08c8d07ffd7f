"""Full-size workloads on the GPU, every output against the oracle.

Every GEMM of every workload runs exactly as bench.py runs it (bf16
activations with a static, calibrated global scale; weights quantised per
module with their own dynamic scale, fused by the global-scale repair), with
bf16 and fp32 outputs.  The oracle quantises the same host arrays itself and
must match every code byte, scale byte and global scale; then every entry of
both outputs is checked against the oracle's float64 product of its own
operands, in row chunks (|err| <= 1e-5 sum|a w|, plus one bf16 unit for the
bf16 output).
"""
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
    return t if dtype == "f32" else t.to(torch.bfloat16)


@pytest.mark.parametrize("config,index", [("tiny", 0), ("gdn", 0), ("decode", 0), ("mlp", 0), ("mlp", 1), ("long", 0),
                                          ("long", 1)])
def test_workload_full_tensors(gpu_lib, config, index):
    """Every code and scale byte of the workload's quantised operands against the
    oracle, not samples: the activation under its calibrated static scale, each
    weight module under its own dynamic scale, and the scales after the
    global-scale repair of the fused modules.  Then every entry of the GEMM's
    output, fp32 and bf16, against the oracle's float64 product of its own
    operands (|err| <= 1e-5 sum|a w|, plus one bf16 unit for the bf16 output)."""
    nv = gpu_lib
    dev = torch.device("cuda:0")
    log("full tensor", config, index, "generating inputs")
    lin = synth.make_workload(config, seed=0)[index]
    config = f"{config}/{lin.name}"
    m, k = lin.a.shape
    ga = torch.zeros(1, dtype=torch.float32, device=dev)
    nv.nvfp4_quantize(to_dev(lin.a_calib, lin.a_dtype), ga, "dynamic")
    ac, asc = nv.nvfp4_quantize(to_dev(lin.a, lin.a_dtype), ga, "static")
    g_a = O.global_scale(lin.a_calib)
    assert np.float32(ga.item()) == g_a
    log("full tensor", config, "activation", (m, k))
    ref_ac, ref_as = [], []
    for r0 in range(0, m, 2048):
        rc, rs, _ = O.quantize_ref(lin.a[r0:r0 + 2048], g_a)
        assert np.array_equal(ac[r0:r0 + 2048].cpu().numpy(), rc), f"activation codes, rows {r0}+"
        assert np.array_equal(asc[r0:r0 + 2048].cpu().numpy(), rs), f"activation scales, rows {r0}+"
        ref_ac.append(rc)
        ref_as.append(rs)

    ws = torch.empty((lin.n, k // 16), dtype=torch.uint8, device=dev)
    wc = torch.empty((lin.n, k // 2), dtype=torch.uint8, device=dev)
    gs, rows, ref_wc, ref_scales, r0 = [], [], [], [], 0
    for name, w in lin.modules:
        g = torch.zeros(1, dtype=torch.float32, device=dev)
        nv.nvfp4_quantize(to_dev(w, lin.a_dtype), g, "dynamic", codes=wc[r0:r0 + w.shape[0]], scales=ws[r0:r0 + w.shape[0]])
        g_i = O.global_scale(w)
        assert np.float32(g.item()) == g_i, name
        log("full tensor", config, name, w.shape)
        for q0 in range(0, w.shape[0], 4096):
            rc, rs, _ = O.quantize_ref(w[q0:q0 + 4096], g_i)
            assert np.array_equal(wc[r0 + q0:r0 + q0 + rc.shape[0]].cpu().numpy(), rc), f"{name} codes, rows {q0}+"
            assert np.array_equal(ws[r0 + q0:r0 + q0 + rc.shape[0]].cpu().numpy(), rs), f"{name} scales, rows {q0}+"
            ref_wc.append(rc)
            ref_scales.append(rs)
        gs.append(float(g.item()))
        rows.append(w.shape[0])
        r0 += w.shape[0]
    if len(rows) > 1:
        g_star, lossy = nv.nvfp4_fuse_rescale(ws, k, rows, gs)
        folded, ref_gstar, ref_lossy = O.fuse_rescale_ref(np.concatenate(ref_scales), rows, gs)
        assert np.float32(g_star) == ref_gstar
        assert int(lossy.item()) == ref_lossy
        assert np.array_equal(ws.cpu().numpy(), folded), "fused scales"
    else:
        g_star, folded, ref_gstar = gs[0], np.concatenate(ref_scales), O.global_scale(lin.modules[0][1])

    # the whole output, in the kernels bench.py times for this shape
    gw = torch.tensor([g_star], dtype=torch.float32, device=dev)
    c32 = nv.nvfp4_gemm(ac, asc, ga, wc, ws, gw, torch.float32)
    c16 = nv.nvfp4_gemm(ac, asc, ga, wc, ws, gw, torch.bfloat16)
    torch.cuda.synchronize()
    ref_ac, ref_as, ref_wc = np.concatenate(ref_ac), np.concatenate(ref_as), np.concatenate(ref_wc)
    worst = 0.0
    for r0 in range(0, m, 4096):
        log("full tensor", config, "output rows", r0, "of", m)
        val, bound = O.gemm_ref(ref_ac[r0:r0 + 4096], ref_as[r0:r0 + 4096], g_a, ref_wc, folded, ref_gstar)
        got32 = c32[r0:r0 + 4096].double().cpu().numpy()
        got16 = c16[r0:r0 + 4096].double().cpu().numpy()
        err32 = np.abs(got32 - val)
        assert np.all(err32 <= 1e-5 * bound), f"fp32 output, rows {r0}+"
        assert np.all(np.abs(got16 - val) <= 1e-5 * bound + 2.0 ** -8 * np.abs(val)), f"bf16 output, rows {r0}+"
        worst = max(worst, float(np.max(err32 / np.maximum(bound, 1e-300))))
    log("full tensor", config, "output max err/bound", worst)
