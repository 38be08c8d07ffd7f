"""Serving-style use of the library on the GPU: the quantise -> GEMM step
captured in a HIP graph and replayed (every replay checked against the eager
result, with eager work and synchronisation in between), and two independent
layers running concurrently on two streams.  Nothing in the library allocates,
synchronises or memsets, so both must give the eager results exactly."""
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


def prepared(nv, m, n, k, seed):
    x, oc = synth.activations(seed, "gdn", 900, m, k)
    xc, _ = synth.activations(seed, "gdn", 901, m, k, outlier_cols=oc)
    w = synth.weights(seed, "gdn", 902, n, k)
    dev = torch.device("cuda:0")
    a = torch.from_numpy(x).to(dev).to(torch.bfloat16)
    ga = torch.zeros(1, dtype=torch.float32, device=dev)
    nv.nvfp4_quantize(torch.from_numpy(xc).to(dev).to(torch.bfloat16), ga, "dynamic")
    gw = torch.zeros(1, dtype=torch.float32, device=dev)
    wc, ws = nv.nvfp4_quantize(torch.from_numpy(w).to(dev).to(torch.bfloat16), gw, "dynamic")
    ac = torch.empty((m, k // 2), dtype=torch.uint8, device=dev)
    asc = torch.empty((m, k // 16), dtype=torch.uint8, device=dev)
    c = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    return a, ga, wc, ws, gw, ac, asc, c


# decode kernel; prefill kernel; prefill tiles then a 64-column strip on the decode kernel (two launches, 256 CUs)
@pytest.mark.parametrize("shape", [(32, 4352, 5120), (512, 1024, 1024), (512, 32832, 1024)])
def test_graph_replays_match_eager(gpu_lib, shape):
    nv = gpu_lib
    m, n, k = shape
    a, ga, wc, ws, gw, ac, asc, c = prepared(nv, m, n, k, 1)

    def step():
        nv.nvfp4_quantize(a, ga, "static", codes=ac, scales=asc)
        nv.nvfp4_gemm(ac, asc, ga, wc, ws, gw, out=c)

    step()
    torch.cuda.synchronize()
    ref_c, ref_ac = c.clone(), ac.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(4):
        log("graph replay", shape, r)
        c.zero_()
        ac.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ac, ref_ac), f"replay {r}: activation codes"
        assert torch.equal(c, ref_c), f"replay {r}: GEMM output"
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(c, ref_c)


def test_two_streams_concurrently(gpu_lib):
    nv = gpu_lib
    layers = [prepared(nv, 256, 2048, 2048, 2), prepared(nv, 32, 4096, 2048, 3)]
    refs = []
    for a, ga, wc, ws, gw, ac, asc, c in layers:
        nv.nvfp4_quantize(a, ga, "static", codes=ac, scales=asc)
        nv.nvfp4_gemm(ac, asc, ga, wc, ws, gw, out=c)
        torch.cuda.synchronize()
        refs.append(c.clone())
        c.zero_()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for it in range(3):
        log("two streams", it)
        for (a, ga, wc, ws, gw, ac, asc, c), st in zip(layers, streams):
            with torch.cuda.stream(st):
                for _ in range(5):
                    nv.nvfp4_quantize(a, ga, "static", codes=ac, scales=asc, stream=st)
                    nv.nvfp4_gemm(ac, asc, ga, wc, ws, gw, out=c, stream=st)
        torch.cuda.synchronize()
        for (a, ga, wc, ws, gw, ac, asc, c), ref in zip(layers, refs):
            assert torch.equal(c, ref)
            c.zero_()
        torch.cuda.synchronize()
