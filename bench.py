"""Throughput of the NVFP4 W4A4 linear layer on one MI355X.

One step = the whole hot path over one batch: online quantisation of the
activations (static, calibrated global scale) followed by the block-scaled
W4A4 GEMM against pre-quantised, fuse-rescaled weights (weight preparation is
offline, as on the pages, and not timed).  Default workload: the GDN fused
input projection at 8K-token prefill, A[8192x5120] bf16 -> W[14432x5120]
(qkv 8192 + z 6144 + a 48 + b 48, four modules calibrated separately and
fused by global-scale repair), bf16 output.

Prints one JSON line.  `value` is whole-step TFLOP/s = 2*M*N*K / step time
(quantisation included); `roofline` covers the dominant kernel (the GEMM),
launched back to back with HIP events around the loop on the stream it runs
on, beside the ceilings measured on the chip by the probes library (an
MFMA-only loop, a streaming read); `cpu_baseline` times the CPU oracle on a
bounded row sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--workload gdn|mlp|decode|long]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A4 GEMM TFLOP/s incl. act-quant at 8K-token prefill; % of MFMA/HBM roofline"
PEAK_F16_MFMA_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_FP4_MFMA_TFLOPS = 10100.0  # MI355X dense fp4 MFMA
CSRC = os.path.join(ROOT, "nvfp4_w4a4_block_quantize_amd", "csrc")
# sources of the kernels each workload's dominant call runs, with the dispatch
# that picks them (traffic counters are tied to these; once they change, the
# stored counters no longer apply).  A prefill call may end with a ragged
# column strip on the decode-shaped kernel.
KERNEL_SRCS = {
    "gemm_fast": ("gemm.hip", "gemm_fast.hip", "gemm_decode.hip", "gemm_common.h", "nvfp4_device.h"),
    "gemm_decode": ("gemm.hip", "gemm_decode.hip", "gemm_stream.hip", "gemm_common.h", "nvfp4_device.h"),
    "amax_observe": ("quantize.hip", "nvfp4_device.h"),
    "kv_quantize_fp8": ("kv_quantize.hip", "nvfp4_device.h"),
}
WORKLOAD_KERNEL = {"gdn": "gemm_fast", "mlp": "gemm_fast", "long": "gemm_fast", "decode": "gemm_decode",
                   "calib": "amax_observe", "kv8": "kv_quantize_fp8"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None, help="timed steps (default 50; 1000 for decode)")
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed steps first (default 40; 1000 for decode, 200 for calib and kv8): the chip's "
                        "clock settles over the first 30-40 prefill steps and 600-800 decode steps")
    p.add_argument("--workload", default="gdn", choices=["gdn", "mlp", "decode", "long", "calib", "kv8"],
                   help="calib: the calibration observer over 32K-token batches; kv8: static FP8 K/V "
                        "quantisation of a 32K-token context (both HBM-bound, GB/s)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=8192, help="activation rows in the oracle's timed sample")
    p.add_argument("--fp8-compare", action="store_true",
                   help="also time an FP8 E4M3 W8A8 GEMM (hipBLASLt through torch._scaled_mm, per-tensor scales, "
                        "activation cast included) on the same shapes")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain device copy of known size (for HBM counter scaling)")
    p.add_argument("--shapes", default=None,
                   help="comma-separated MxNxK: the GPU time per nvfp4_gemm call on each shape from HIP graph "
                        "replays (random codes, rotated weight copies) instead of a workload")
    p.add_argument("--no-secondary", action="store_true",
                   help="gdn only: skip the decode-shaped and MLP workloads and the FP8 comparison that the "
                        "default line carries beside the headline")
    args = p.parse_args()
    if args.warmup is None:
        args.warmup = {"decode": 1000, "calib": 200, "kv8": 200}.get(args.workload, 40)
    return args


def gemm_source_sha(workload):
    h = hashlib.sha256()
    for name in KERNEL_SRCS[WORKLOAD_KERNEL[workload]]:
        p = os.path.join(CSRC, name)
        if not os.path.exists(p):
            return None
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload):
    """HBM bytes per GEMM launch from committed rocprofv3 counters, valid only
    for the GEMM source they were taken on."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    e = d.get(workload)
    if not e or e.get("gemm_source_sha") != gemm_source_sha(workload):
        return None
    return e.get("hbm_bytes_per_launch")


class Prepared:
    """Device-resident operands of one GEMM of the workload."""

    def __init__(self, nv, torch, lin, rotate=1):
        dev = torch.device("cuda:0")
        self.m, self.k = lin.a.shape
        self.n = lin.n
        to_dev = (lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)) if lin.a_dtype == "f32" \
            else (lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev).to(torch.bfloat16))
        self.a = to_dev(lin.a)
        # static activation scale: calibrated on a separate draw of the same distribution
        self.ga = torch.zeros(1, dtype=torch.float32, device=dev)
        nv.nvfp4_quantize(to_dev(lin.a_calib), self.ga, "dynamic")
        # weights: each module quantised with its own dynamic scale into its rows of one buffer
        self.wc = torch.empty((self.n, self.k // 2), dtype=torch.uint8, device=dev)
        self.ws = torch.empty((self.n, self.k // 16), dtype=torch.uint8, device=dev)
        gs, rows, r0 = [], [], 0
        for _, w in lin.modules:
            g = torch.zeros(1, dtype=torch.float32, device=dev)
            nv.nvfp4_quantize(to_dev(w), g, "dynamic", codes=self.wc[r0:r0 + w.shape[0]],
                              scales=self.ws[r0:r0 + w.shape[0]])
            gs.append(float(g.item()))
            rows.append(w.shape[0])
            r0 += w.shape[0]
        g_star, self.lossy = nv.nvfp4_fuse_rescale(self.ws, self.k, rows, gs) if len(rows) > 1 else (gs[0], None)
        self.gw = torch.tensor([g_star], dtype=torch.float32, device=dev)
        self.module_gscales = gs
        self.module_rows = rows
        self.copies = [(self.wc, self.ws)] + [(self.wc.clone(), self.ws.clone()) for _ in range(rotate - 1)]
        self.ac = torch.empty((self.m, self.k // 2), dtype=torch.uint8, device=dev)
        self.asc = torch.empty((self.m, self.k // 16), dtype=torch.uint8, device=dev)
        self.c = torch.empty((self.m, self.n), dtype=torch.bfloat16, device=dev)

    def flops(self):
        return 2.0 * self.m * self.n * self.k

    def gemm_bytes(self):
        """Algorithmic HBM bytes of one GEMM: both operands' codes + scales once, C once."""
        return (self.m + self.n) * (self.k // 2 + self.k // 16) + self.m * self.n * 2

    def quant_bytes(self):
        return self.m * self.k * self.a.element_size() + self.m * (self.k // 2 + self.k // 16)


def fp8_decode_scale(x):
    """Per-tensor E4M3 decode scale amax / 448 (a 1-element fp32 tensor)."""
    return (x.float().abs().max() / 448.0).reshape(1).float()


def fp8_weight(torch, w, sw):
    """E4M3 weight bytes: fp32(w / sw) cast to float8_e4m3fn."""
    return (w.float() / sw).to(torch.float8_e4m3fn)


def fp8_activation(torch, a, inv_sa):
    """E4M3 activation bytes: (a * 1/sa) in the activation's dtype, cast to
    float8_e4m3fn (what the comparison times every step)."""
    return (a * inv_sa).to(torch.float8_e4m3fn)


def fp8_gemm(torch, a8, w8, sa, sw):
    """bf16 C = (a8 * sa) @ (w8 * sw)^T by hipBLASLt through torch._scaled_mm."""
    return torch._scaled_mm(a8, w8.t(), scale_a=sa, scale_b=sw, out_dtype=torch.bfloat16)


def fp8_compare(torch, preps, lins, steps, warmup, rotate=1):
    """The recipes the pages compare against keep these GEMMs in FP8 (the news
    article, section 04).  Same shapes and inputs: per-tensor E4M3 scales
    (448 / amax), activation cast to E4M3 every step, weights cast once, bf16
    output, one hipBLASLt GEMM.  A library baseline, not part of the path."""
    f8 = getattr(torch, "float8_e4m3fn", None)
    if f8 is None or not hasattr(torch, "_scaled_mm"):
        return {"error": "torch has no float8_e4m3fn / _scaled_mm"}
    res = []
    try:
        for lin, p in zip(lins, preps):
            dev = p.a.device
            w = torch.cat([torch.from_numpy(np.ascontiguousarray(wi, dtype=np.float32)) for _, wi in lin.modules]).to(dev)
            sa = fp8_decode_scale(p.a)
            sw = fp8_decode_scale(w)
            w8s = [fp8_weight(torch, w, sw) for _ in range(rotate)]  # copies rotated like the W4A4 weights
            a_bf = p.a
            inv_sa = (1.0 / sa).to(a_bf.dtype)
            del w

            def one(i):
                return fp8_gemm(torch, fp8_activation(torch, a_bf, inv_sa), w8s[i % rotate], sa, sw)

            for i in range(warmup):
                c = one(i)
            torch.cuda.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            for i in range(steps):
                c = one(i)
            t1.record()
            torch.cuda.synchronize()
            ms = t0.elapsed_time(t1) / steps
            a8 = fp8_activation(torch, a_bf, inv_sa)
            torch.cuda.synchronize()
            t0.record()
            for i in range(steps):
                c = fp8_gemm(torch, a8, w8s[i % rotate], sa, sw)
            t1.record()
            torch.cuda.synchronize()
            ms_gemm = t0.elapsed_time(t1) / steps
            fp8_bytes = p.n * p.k + p.m * p.k + p.m * p.n * 2
            res.append({"name": lin.name, "ms_step": round(ms, 5), "ms_gemm": round(ms_gemm, 5),
                        "tflops_step": round(p.flops() / (ms * 1e-3) / 1e12, 2),
                        "tflops_gemm": round(p.flops() / (ms_gemm * 1e-3) / 1e12, 2),
                        "weight_bytes": p.n * p.k, "gemm_gbs": round(fp8_bytes / (ms_gemm * 1e-3) / 1e9, 1),
                        "weight_copies_rotated": rotate})
            del w8s, a8, c
    except Exception as e:  # a missing FP8 path is reported, not fatal
        return {"error": f"{type(e).__name__}: {e}"[:300], "done": res}
    return {"kind": "FP8 E4M3 W8A8, per-tensor scales, hipBLASLt via torch._scaled_mm (library baseline)",
            "gemms": res, "fp8_mfma_peak_tflops": 5000.0}


def copy_calibration(torch):
    """A plain 1 GiB device-to-device copy: the known size that HBM byte
    counters are scaled against."""
    nbytes = 1 << 30
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    return nbytes


def _probes(torch):
    """The measurement probes (an MFMA-only loop and a streaming read) of
    bench_probes.hip, built beside this file; None when they are not built."""
    import ctypes

    path = os.path.join(ROOT, "libnvfp4_probes.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.probe_mfma_f16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return lib


def _time_launches(torch, fn, reps):
    fn()
    fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        fn()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / reps


def measured_mfma_peak(torch):
    """fp16 MFMA rate of waves doing nothing but v_mfma_f32_32x32x16_f16
    (4 waves per SIMD, four independent chains each), TFLOP/s."""
    lib = _probes(torch)
    if lib is None:
        return None
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    wg, iters = 2048, 4096
    ms = _time_launches(torch, lambda: lib.probe_mfma_f16(wg, iters, sink.data_ptr(), st), 5)
    return wg * 4 * iters * 4 * 32768 / (ms * 1e-3) / 1e12


def measured_stream_read(torch):
    """HBM read rate of a 1 GiB streaming read with 16-byte non-temporal
    loads (512 workgroups: the best of a sweep on this chip), GB/s."""
    lib = _probes(torch)
    if lib is None:
        return None
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    buf = torch.ones(1 << 28, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    ms = _time_launches(torch, lambda: lib.probe_stream_read(buf.data_ptr(), buf.numel() * 4, 512, sink.data_ptr(), st), 10)
    return buf.numel() * 4 / (ms * 1e-3) / 1e9


def run_kv8(args):
    """Static FP8 KV-cache quantisation: K and V of a 32K-token context, 8 KV
    heads x 128 (bf16 in, E4M3 out), four layers' worth rotated so the 256 MB
    Infinity Cache cannot hold them; bytes = 2 read + 1 written per element."""
    import torch

    import nvfp4_w4a4_block_quantize_amd as nv
    from nvfp4_w4a4_block_quantize_amd import synth

    nv.load_library()
    rows, cols, layers = 32768, 1024, 4
    ins, outs = [], []
    for i in range(2 * layers):
        x, _ = synth.activations(args.seed, "long", 800 + i, rows, cols, dist="t3")
        ins.append(torch.from_numpy(x).cuda().to(torch.bfloat16))
        outs.append(torch.empty((rows, cols), dtype=torch.uint8, device="cuda:0"))
        del x
    state = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    nv.nvfp4_amax_observe(ins[0], state)
    s = nv.nvfp4_kv_scale_from_amax(state)
    steps = args.steps if args.steps is not None else 50

    def step(i):
        j = 2 * (i % layers)
        nv.nvfp4_kv_quantize_fp8(ins[j], s, out=outs[j])
        nv.nvfp4_kv_quantize_fp8(ins[j + 1], s, out=outs[j + 1])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    byts = 2 * rows * cols * 3
    gbs = byts / (ms * 1e-3) / 1e9
    out = {"metric": "static FP8 KV-cache quantisation GB/s (K and V, 32K tokens), % of HBM roofline",
           "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16 in, e4m3 out", "data": "synthetic (seeded; no dataset)",
           "config": {"workload": "kv_fp8_32k_x_8x128", "k_and_v": [rows, cols], "layers_rotated": layers,
                      "kernel_source_sha": gemm_source_sha("kv8")},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": load_traffic("kv8"),
                        "kernel": "kv_quantize_kernel", "avg_ms": round(ms / 2, 5)}}
    if args.copy_calibration:
        out["copy_calibration_bytes"] = copy_calibration(torch)
    print(json.dumps(out), flush=True)


def run_calib(args):
    """Calibration observer: max|x| of one 32K-token batch of hidden size 5120
    (bf16, 335.5 MB) folded into a device word per step; bytes = the batch."""
    import torch

    import nvfp4_w4a4_block_quantize_amd as nv
    from nvfp4_w4a4_block_quantize_amd import synth

    nv.load_library()
    rows, cols = 32768, synth.HIDDEN
    batches = []
    for i in range(2):  # two resident batches, alternated, 671 MB > the 256 MB Infinity Cache
        x, _ = synth.activations(args.seed, "long", 500 + i, rows, cols, dist="t3")
        batches.append(torch.from_numpy(x).cuda().to(torch.bfloat16))
        del x
    state = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    steps = args.steps if args.steps is not None else 50
    for i in range(args.warmup):
        nv.nvfp4_amax_observe(batches[i % 2], state)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        nv.nvfp4_amax_observe(batches[i % 2], state)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    byts = rows * cols * 2
    gbs = byts / (ms * 1e-3) / 1e9
    g = nv.nvfp4_gscale_from_amax(state)
    out = {"metric": "calibration observer GB/s (max|x| over 32K-token batches), % of HBM roofline",
           "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16 in, f32 max", "data": "synthetic (seeded; no dataset)",
           "config": {"workload": "calib_observer_32k_x_5120", "batch": [rows, cols], "gscale": float(g.item()),
                      "kernel_source_sha": gemm_source_sha("calib")},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": load_traffic("calib"),
                        "kernel": "amax_kernel (observer)", "avg_ms": round(ms, 5)}}
    if args.copy_calibration:
        out["copy_calibration_bytes"] = copy_calibration(torch)
    print(json.dumps(out), flush=True)


WORKLOAD_NAMES = {"gdn": "gdn_fused_in_proj_prefill_8k", "mlp": "mlp_gate_up_down_prefill_8k",
                  "decode": "decode_gate_up_m32", "long": "attn_qkv_o_prefill_32k"}


def measure(nv, torch, workload, seed, steps, warmup, fp8=False, copy_cal=False):
    """One workload's step throughput, per-kernel split and dominant-GEMM
    roofline.  Returns (result dict, lins) with the device buffers released."""
    from nvfp4_w4a4_block_quantize_amd import synth

    lins = synth.make_workload(workload, seed=seed)
    rotate = 4 if workload == "decode" else 1
    preps = [Prepared(nv, torch, lin, rotate=rotate) for lin in lins]
    torch.cuda.synchronize()

    def step(i, ev=None):
        for j, p in enumerate(preps):
            wc, ws = p.copies[i % len(p.copies)]
            if ev is not None:
                ev[j][0].record()
            nv.nvfp4_quantize(p.a, p.ga, "static", codes=p.ac, scales=p.asc)
            if ev is not None:
                ev[j][1].record()
            nv.nvfp4_gemm(p.ac, p.asc, p.ga, wc, ws, p.gw, out=p.c)
            if ev is not None:
                ev[j][2].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region 1: the whole step, back to back (this is `value`)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps

    # timed region 2: the same steps with events between the kernels (per-kernel durations)
    n_ev = min(steps, 200)
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in preps] for _ in range(n_ev)]
    torch.cuda.synchronize()
    for i in range(n_ev):
        step(i, evs[i])
    torch.cuda.synchronize()
    q_ms = [float(np.mean([evs[i][j][0].elapsed_time(evs[i][j][1]) for i in range(n_ev)])) for j in range(len(preps))]
    g_ms = [float(np.mean([evs[i][j][1].elapsed_time(evs[i][j][2]) for i in range(n_ev)])) for j in range(len(preps))]

    # timed region 3: the dominant GEMM alone, back to back (the roofline's
    # kernel duration; events between kernels add their own overhead to a
    # decode-sized launch)
    jd = int(np.argmax([p.flops() for p in preps]))
    pd = preps[jd]
    reps = min(max(steps, 20), 200)
    state = {"i": 0}

    def gemm_only():
        wc, ws = pd.copies[state["i"] % len(pd.copies)]
        state["i"] += 1
        nv.nvfp4_gemm(pd.ac, pd.asc, pd.ga, wc, ws, pd.gw, out=pd.c)

    dom_ms = _time_launches(torch, gemm_only, reps)

    flops = sum(p.flops() for p in preps)
    if workload == "decode":
        p = preps[0]
        step_bytes = p.gemm_bytes() + p.quant_bytes() + p.m * (p.k // 2 + p.k // 16)
        value, unit = step_bytes / (ms_step * 1e-3) / 1e9, "GB/s"
        gb = p.gemm_bytes() / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gb, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gb / PEAK_HBM_GBS, 4), "traffic": load_traffic(workload),
                "kernel": "nvfp4 gemm (decode shape)", "avg_ms": round(dom_ms, 5),
                "bytes_per_launch": p.gemm_bytes()}
        stream = measured_stream_read(torch)
        if stream is not None:
            roof["measured_stream_read_gbs"] = round(stream, 1)
            roof["frac_of_measured_stream"] = round(gb / stream, 4)
        # the same call on one weight copy, which then sits in the 256 MB Infinity Cache
        wc0, ws0 = p.copies[0]
        ms1 = _time_launches(torch, lambda: nv.nvfp4_gemm(p.ac, p.asc, p.ga, wc0, ws0, p.gw, out=p.c), 200)
        roof["single_copy_cache_resident_gbs"] = round(p.gemm_bytes() / (ms1 * 1e-3) / 1e9, 1)
        metric = "W4A4 decode-shaped GEMM GB/s incl. act-quant (M=32), % of HBM roofline"
    else:
        value, unit = flops / (ms_step * 1e-3) / 1e12, "TFLOP/s"
        # dominant kernel: the largest GEMM of the step
        ach = pd.flops() / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_F16_MFMA_TFLOPS, 4), "traffic": load_traffic(workload),
                "kernel": f"nvfp4 gemm {pd.m}x{pd.n}x{pd.k}", "avg_ms": round(dom_ms, 5),
                "frac_of_fp4_peak": round(ach / PEAK_FP4_MFMA_TFLOPS, 4)}
        loop = measured_mfma_peak(torch)
        if loop is not None:
            roof["measured_mfma_f16_loop_tflops"] = round(loop, 1)
            roof["frac_of_measured_loop"] = round(ach / loop, 4)
        metric = METRIC

    res = {
        "metric": metric, "value": round(value, 3), "unit": unit, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "config": {
            "workload": WORKLOAD_NAMES[workload],
            "gemms": [{"name": lin.name, "M": p.m, "N": p.n, "K": p.k, "modules": p.module_rows,
                       "quant_ms": round(q, 5), "gemm_ms": round(g, 5),
                       "gemm_tflops": round(p.flops() / (g * 1e-3) / 1e12, 2),
                       "quant_gbs": round(p.quant_bytes() / (q * 1e-3) / 1e9, 1),
                       "quant_frac_of_hbm": round(p.quant_bytes() / (q * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
                      for lin, p, q, g in zip(lins, preps, q_ms, g_ms)],
            "a_dtype": lins[0].a_dtype, "c_dtype": "bf16", "act_gscale": "static (calibrated on a separate draw)",
            "weights": "pre-quantised per module, fuse-rescaled, not timed",
            "weight_copies_rotated": rotate, "gemm_kernel": WORKLOAD_KERNEL[workload],
            "gemm_source_sha": gemm_source_sha(workload),
        },
        "roofline": roof,
    }
    if fp8:
        res["fp8_w8a8_compare"] = fp8_compare(torch, preps, lins, min(max(steps, 20), 200), max(warmup, 5),
                                              rotate=rotate)
        r0 = res["fp8_w8a8_compare"].get("gemms", [])
        if r0:
            res["fp8_w8a8_compare"]["fp8_over_w4a4_gemm_time"] = round(
                r0[jd]["ms_gemm"] / dom_ms, 4) if jd < len(r0) else None
    if copy_cal:
        res["copy_calibration_bytes"] = copy_calibration(torch)
    del preps
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, lins


def secondary_line(res):
    """The fields of a secondary workload's result kept in the headline line."""
    keep = {k: res[k] for k in ("metric", "value", "unit", "steps", "warmup", "ms_per_step")}
    keep["workload"] = res["config"]["workload"]
    keep["gemms"] = [{k: g[k] for k in ("name", "M", "N", "K", "quant_ms", "gemm_ms", "gemm_tflops")}
                     for g in res["config"]["gemms"]]
    keep["roofline"] = res["roofline"]
    keep["weight_copies_rotated"] = res["config"]["weight_copies_rotated"]
    return keep


def run(args):
    import torch

    import nvfp4_w4a4_block_quantize_amd as nv

    nv.load_library()
    torch.cuda.init()
    steps = args.steps if args.steps is not None else (1000 if args.workload == "decode" else 50)

    # the decode-shaped and MLP workloads, each with its own warm-up and steps,
    # run before the headline (the chip's clock has then settled for it)
    secondary = {}
    if args.workload == "gdn" and not args.no_secondary:
        dres, _ = measure(nv, torch, "decode", args.seed, 1000, 1000)
        secondary["decode"] = secondary_line(dres)
        mres, _ = measure(nv, torch, "mlp", args.seed, 20, 10)
        secondary["mlp"] = secondary_line(mres)

    res, lins = measure(nv, torch, args.workload, args.seed, steps, args.warmup,
                        fp8=args.fp8_compare or (args.workload == "gdn" and not args.no_secondary),
                        copy_cal=args.copy_calibration)
    out = {
        "metric": res["metric"], "value": res["value"], "unit": res["unit"], "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "e2m1xe2m1 decoded exactly to f16, f16 MFMA, f32 accumulate",
        "data": "synthetic (seeded; no dataset or trained weights)",
        "config": res["config"],
        "roofline": res["roofline"],
    }
    for k in ("fp8_w8a8_compare", "copy_calibration_bytes"):
        if k in res:
            out[k] = res[k]
    if secondary:
        out["secondary"] = secondary
    out["timing_order"] = (("secondary workloads (decode, then MLP) with their own warm-up, then " if secondary else "")
                           + "the headline: --warmup untimed steps, the --steps timed steps (value), a per-kernel "
                             "event pass, the dominant GEMM alone back to back (roofline), the probes"
                           + (", the FP8 comparison" if "fp8_w8a8_compare" in res else "")
                           + ("; then the CPU oracle" if not args.no_cpu_baseline else ""))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(lins, args.cpu_rows, args.workload)
    print(json.dumps(out), flush=True)


def cpu_baseline(lins, rows, workload):
    """The oracle, as it stands, on a bounded row sample of the same workload:
    quantise `rows` activation rows and multiply them (float64) against the
    oracle's own quantised, fuse-rescaled weights.  Weight preparation is not
    timed, as on the GPU side."""
    from oracle import nvfp4_oracle as O

    lin = max(lins, key=lambda l: l.m * l.n * l.k)
    rows = min(rows, lin.m)
    a = lin.a[:rows]
    _, _, g_a = O.quantize_ref(lin.a_calib)
    qs = [O.quantize_ref(w) for _, w in lin.modules]
    wc = np.concatenate([q[0] for q in qs])
    if len(qs) > 1:
        ws, g_w, _ = O.fuse_rescale_ref(np.concatenate([q[1] for q in qs]), [q[0].shape[0] for q in qs],
                                        [q[2] for q in qs])
    else:
        ws, g_w = qs[0][1], qs[0][2]
    t0 = time.perf_counter()
    ac, asc, _ = O.quantize_ref(a, g_a)
    O.gemm_ref(ac, asc, g_a, wc, ws, g_w)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * lin.n * lin.k
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    host = host_description()
    if workload == "decode":
        byts = rows * lin.k * 2 + lin.n * (lin.k // 2 + lin.k // 16)
        return {"value": round(byts / dt / 1e9, 4), "unit": "GB/s", "cores": min(cores, threads), "kind": "oracle",
                "seconds": round(dt, 2),
                "sample": f"{rows} of {lin.m} rows of {lin.name}: quantise + float64 dequantise-matmul vs full W",
                **host}
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": min(cores, threads), "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"{rows} of {lin.m} activation rows of {lin.name} (N={lin.n}, K={lin.k}): quantise + "
                      f"float64 dequantise-matmul (plus its |a||w| bound) against the full weight",
            **host}


def host_description():
    """CPU model and numpy's BLAS build, for the oracle timing."""
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        dep = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{dep.get('name')} {dep.get('version')}".strip()
    except Exception:
        pass
    return {"cpu": cpu, "blas": blas}


def time_shape(nv, torch, m, n, k, reps=100, min_rotated_bytes=512 << 20, seed=3):
    """GPU time of one nvfp4_gemm call on MxNxK: `reps` calls captured in one
    HIP graph, replayed three times after one untimed replay.  A and the
    weight copies hold random codes and E4M3 scale bytes 0x28-0x47 (scales
    2^-2 .. 2^1.9); enough weight copies are rotated from call to call that
    the rotated set reaches `min_rotated_bytes` (at least 2 copies), so the
    weight streams from HBM rather than the 256 MB Infinity Cache.  Timing
    only: the parity tests check the outputs."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(seed)

    def rnd(rows, cols, lo, hi):
        return torch.randint(lo, hi, (rows, cols), dtype=torch.uint8, generator=g).to(dev)

    wbytes = n * (k // 2 + k // 16)
    copies = int(max(2, -(-min_rotated_bytes // wbytes)))
    ac, asc = rnd(m, k // 2, 0, 256), rnd(m, k // 16, 0x28, 0x48)
    ws = [(rnd(n, k // 2, 0, 256), rnd(n, k // 16, 0x28, 0x48)) for _ in range(copies)]
    ga = torch.full((1,), 0.5, device=dev)
    gw = torch.full((1,), 2.0, device=dev)
    c = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    for i in range(2 * copies):
        nv.nvfp4_gemm(ac, asc, ga, ws[i % copies][0], ws[i % copies][1], gw, out=c)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for i in range(reps):
                nv.nvfp4_gemm(ac, asc, ga, ws[i % copies][0], ws[i % copies][1], gw, out=c)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / (3 * reps) * 1000.0
    nbytes = (m + n) * (k // 2 + k // 16) + m * n * 2
    return {"M": m, "N": n, "K": k, "us_per_call": round(us, 3), "weight_copies_rotated": copies,
            "rotated_weight_mb": round(copies * wbytes / 1e6, 1),
            "gbs": round(nbytes / (us * 1e-6) / 1e9, 1), "tflops": round(2.0 * m * n * k / (us * 1e-6) / 1e12, 2)}


def run_shapes(args):
    import torch

    import nvfp4_w4a4_block_quantize_amd as nv

    nv.load_library()
    shapes = []
    for sh in args.shapes.split(","):
        m, n, k = (int(v) for v in sh.lower().strip().split("x"))
        if m < 1 or n < 1 or k < 16 or k % 16:
            raise SystemExit(f"bad shape {sh}: M, N >= 1 and K a positive multiple of 16")
        shapes.append(time_shape(nv, torch, m, n, k))
        print(f"[shape] {shapes[-1]}", file=sys.stderr, flush=True)
    print(json.dumps({"metric": "nvfp4_gemm GPU time per call (HIP graph replays of 100 calls)", "n_gpus": 1,
                      "data": "synthetic (random codes and scale bytes)", "c_dtype": "bf16", "shapes": shapes}),
          flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py measures one GPU; --gpus must be 1",
                          "n_gpus_requested": args.gpus}), flush=True)
        sys.exit(2)
    if args.shapes:
        run_shapes(args)
    elif args.workload == "calib":
        run_calib(args)
    elif args.workload == "kv8":
        run_kv8(args)
    else:
        run(args)


if __name__ == "__main__":
    main()
