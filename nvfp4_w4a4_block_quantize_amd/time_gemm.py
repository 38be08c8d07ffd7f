"""GPU time of nvfp4_gemm on given shapes, from HIP graph replays.

    python -m nvfp4_w4a4_block_quantize_amd.time_gemm 32x14336x5120 1x4352x5120 [--reps 100] [--copies 4]

For each MxNxK: random codes and E4M3 scale bytes (values 0x28-0x47, i.e.
scales 2^-2 .. 2^1.9) for A and for `copies` weight copies, rotated from call
to call so that the weight is streamed from HBM when the copies outgrow the
256 MB Infinity Cache.  `reps` calls are captured in one graph, which is
replayed three times; the line printed per shape gives the mean GPU time per
call and the rate over the call's algorithmic bytes (codes and scales of both
operands once, and C in bf16).  Timing only: the outputs are not checked
here (the parity tests do that).
"""
import argparse

import torch

from . import load_library, nvfp4_gemm


def time_shape(m, n, k, reps=100, copies=4, seed=3):
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(seed)
    rnd = lambda rows, cols, lo, hi: torch.randint(lo, hi, (rows, cols), dtype=torch.uint8, generator=g).to(dev)
    ac, asc = rnd(m, k // 2, 0, 256), rnd(m, k // 16, 0x28, 0x48)
    ws = [(rnd(n, k // 2, 0, 256), rnd(n, k // 16, 0x28, 0x48)) for _ in range(copies)]
    ga = torch.full((1,), 0.5, device=dev)
    gw = torch.full((1,), 2.0, device=dev)
    c = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    for i in range(2 * copies):
        nvfp4_gemm(ac, asc, ga, ws[i % copies][0], ws[i % copies][1], gw, out=c)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            for i in range(reps):
                nvfp4_gemm(ac, asc, ga, ws[i % copies][0], ws[i % copies][1], gw, out=c)
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
    return us, nbytes / (us * 1e-6) / 1e9, 2.0 * m * n * k / (us * 1e-6) / 1e12


def main():
    p = argparse.ArgumentParser()
    p.add_argument("shapes", nargs="+", help="MxNxK")
    p.add_argument("--reps", type=int, default=100)
    p.add_argument("--copies", type=int, default=4)
    args = p.parse_args()
    load_library()
    for sh in args.shapes:
        m, n, k = (int(v) for v in sh.lower().split("x"))
        us, gbs, tflops = time_shape(m, n, k, args.reps, args.copies)
        print(f"{m}x{n}x{k}: {us:.2f} us per call, {gbs:.0f} GB/s, {tflops:.1f} TFLOP/s", flush=True)


if __name__ == "__main__":
    main()
