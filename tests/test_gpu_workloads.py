"""Full-size workloads on the GPU, checked against the oracle on samples.

Every workload runs exactly as bench.py runs it (bf16 activations with a
static, calibrated global scale; weights quantised per module with their own
dynamic scale, fused by the global-scale repair; bf16 output), plus an fp32
output for the tighter bound.  The GPU computes the full tensors; the oracle
re-derives sampled rows of every quantised operand (bit-exact), the global
scales (bit-exact) and sampled GEMM entries (|err| <= 1e-5 sum|a w|, plus one
bf16 unit for the bf16 output).
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


def sample_rows(n, k, rng):
    rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, k)]))
    return rows


def to_dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return t if dtype == "f32" else t.to(torch.bfloat16)


def run_linear(nv, lin, rng, n_entries=2048):
    dev = torch.device("cuda:0")
    m, k = lin.a.shape
    n = lin.n
    # activations: static scale calibrated on a separate draw, then the online quantiser
    ga = torch.zeros(1, dtype=torch.float32, device=dev)
    nv.nvfp4_quantize(to_dev(lin.a_calib, lin.a_dtype), ga, "dynamic")
    ac, asc = nv.nvfp4_quantize(to_dev(lin.a, lin.a_dtype), ga, "static")
    # weights: one dynamic scale per module, written into the rows of one buffer
    wc = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
    ws = torch.empty((n, k // 16), dtype=torch.uint8, device=dev)
    gs, rows, r0 = [], [], 0
    for _, w in lin.modules:
        g = torch.zeros(1, dtype=torch.float32, device=dev)
        nv.nvfp4_quantize(to_dev(w, lin.a_dtype), g, "dynamic", codes=wc[r0:r0 + w.shape[0]], scales=ws[r0:r0 + w.shape[0]])
        gs.append(float(g.item()))
        rows.append(w.shape[0])
        r0 += w.shape[0]
    ws_before = ws.clone()
    if len(rows) > 1:
        g_star, lossy = nv.nvfp4_fuse_rescale(ws, k, rows, gs)
    else:
        g_star, lossy = gs[0], None
    gw = torch.tensor([g_star], dtype=torch.float32, device=dev)
    c16 = nv.nvfp4_gemm(ac, asc, ga, wc, ws, gw, torch.bfloat16)
    c32 = nv.nvfp4_gemm(ac, asc, ga, wc, ws, gw, torch.float32)
    torch.cuda.synchronize()

    # ---- oracle on samples
    g_a = O.global_scale(lin.a_calib)
    assert np.float32(ga.item()) == g_a
    ra = sample_rows(m, 96, rng)
    rac, rasc, _ = O.quantize_ref(lin.a[ra], g_a)
    assert np.array_equal(ac[torch.from_numpy(ra).cuda()].cpu().numpy(), rac), "activation codes"
    assert np.array_equal(asc[torch.from_numpy(ra).cuda()].cpu().numpy(), rasc), "activation scales"

    w_codes, w_scales_pre, w_rows_global, counts = [], [], [], []
    r0 = 0
    for (name, w), g_gpu in zip(lin.modules, gs):
        g_i = O.global_scale(w)
        assert np.float32(g_gpu) == g_i, name
        rw = sample_rows(w.shape[0], 96, rng)
        c_i, s_i, _ = O.quantize_ref(w[rw], g_i)
        idx = torch.from_numpy(r0 + rw).cuda()
        assert np.array_equal(wc[idx].cpu().numpy(), c_i), f"{name} codes"
        assert np.array_equal(ws_before[idx].cpu().numpy(), s_i), f"{name} scales"
        w_codes.append(c_i)
        w_scales_pre.append(s_i)
        w_rows_global.append(r0 + rw)
        counts.append(len(rw))
        r0 += w.shape[0]
    if len(counts) > 1:
        folded, ref_gstar, _ = O.fuse_rescale_ref(np.concatenate(w_scales_pre), counts, [O.global_scale(w) for _, w in lin.modules])
        assert np.float32(g_star) == ref_gstar
    else:
        folded, ref_gstar = w_scales_pre[0], O.global_scale(lin.modules[0][1])
    rw_all = np.concatenate(w_rows_global)
    assert np.array_equal(ws[torch.from_numpy(rw_all).cuda()].cpu().numpy(), folded), "fused scales"
    wcodes = np.concatenate(w_codes)

    # sampled GEMM entries from the sampled rows/columns
    pi = rng.integers(0, len(ra), n_entries)
    pj = rng.integers(0, len(rw_all), n_entries)
    val, bound = O.gemm_ref_entries(rac, rasc, g_a, wcodes, folded, ref_gstar, pi, pj)
    mi = torch.from_numpy(ra[pi]).cuda()
    nj = torch.from_numpy(rw_all[pj]).cuda()
    got32 = c32[mi, nj].double().cpu().numpy()
    got16 = c16[mi, nj].double().cpu().numpy()
    err32 = np.abs(got32 - val)
    err16 = np.abs(got16 - val)
    assert np.all(err32 <= 1e-5 * bound), f"fp32 worst {float(np.max(err32 / np.maximum(bound, 1e-300)))}"
    assert np.all(err16 <= 1e-5 * bound + 2.0 ** -8 * np.abs(val)), "bf16 output"
    # every output row of the tile grid was written (no NaN / garbage in unsampled tails)
    assert torch.isfinite(c16).all().item()
    return float(np.max(err32 / np.maximum(bound, 1e-300)))


@pytest.mark.parametrize("config", ["tiny", "gdn", "decode", "mlp", "long"])
def test_workload_full_size(gpu_lib, config):
    rng = np.random.default_rng([7, synth.CONFIG_IDS[config]])
    log("workload", config, "generating inputs")
    lins = synth.make_workload(config, seed=0)
    for lin in lins:
        log("workload", config, lin.name, lin.a.shape, "x", lin.n)
        worst = run_linear(gpu_lib, lin, rng)
        log("workload", config, lin.name, "max err/bound", worst)


@pytest.mark.parametrize("config", ["gdn", "decode"])
def test_workload_full_tensor_bytes(gpu_lib, config):
    """Every code and scale byte of the workload's quantised operands against the
    oracle, not samples: the activation under its calibrated static scale, each
    weight module under its own dynamic scale, and the scales after the
    global-scale repair of the fused modules."""
    nv = gpu_lib
    dev = torch.device("cuda:0")
    log("full tensor", config, "generating inputs")
    lin = synth.make_workload(config, seed=0)[0]
    m, k = lin.a.shape
    ga = torch.zeros(1, dtype=torch.float32, device=dev)
    nv.nvfp4_quantize(to_dev(lin.a_calib, lin.a_dtype), ga, "dynamic")
    ac, asc = nv.nvfp4_quantize(to_dev(lin.a, lin.a_dtype), ga, "static")
    g_a = O.global_scale(lin.a_calib)
    assert np.float32(ga.item()) == g_a
    log("full tensor", config, "activation", (m, k))
    for r0 in range(0, m, 2048):
        rc, rs, _ = O.quantize_ref(lin.a[r0:r0 + 2048], g_a)
        assert np.array_equal(ac[r0:r0 + 2048].cpu().numpy(), rc), f"activation codes, rows {r0}+"
        assert np.array_equal(asc[r0:r0 + 2048].cpu().numpy(), rs), f"activation scales, rows {r0}+"

    ws = torch.empty((lin.n, k // 16), dtype=torch.uint8, device=dev)
    wc = torch.empty((lin.n, k // 2), dtype=torch.uint8, device=dev)
    gs, rows, ref_scales, r0 = [], [], [], 0
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
