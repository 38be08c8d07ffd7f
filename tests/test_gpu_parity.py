"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Codes and scale bytes must match bit for bit; the GEMM must satisfy
|C_gpu - C_ref| <= 1e-5 * sum_k |a_k w_k| per element (fp32 output), with
bf16 / f16 outputs allowed one extra unit in the last place of the narrow
type.  Inputs are seeded (nvfp4_w4a4_block_quantize_amd.synth) or
hand-built edge cases.
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


def dev_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def dev_bf16(x):
    bits = synth.bf16_bits(x).view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(bits)).cuda().view(torch.bfloat16)


def dev_f16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float16)).cuda()


def gscale_tensor(g):
    return torch.tensor([float(np.float32(g))], dtype=torch.float32, device="cuda")


def quantize_gpu(nv, x, dtype, g=None):
    """x: float32 array holding values of `dtype`; g None = dynamic."""
    t = {"f32": dev_f32, "bf16": dev_bf16, "f16": dev_f16}[dtype](x)
    gs = gscale_tensor(0.0 if g is None else g)
    codes, scales = nv.nvfp4_quantize(t, gs, "dynamic" if g is None else "static")
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), np.float32(gs.cpu().numpy()[0])


def assert_quant_equal(nv, x, dtype, g=None, label=""):
    log("quantize", label, dtype, x.shape, "dynamic" if g is None else f"g={g}")
    c, s, gg = quantize_gpu(nv, x, dtype, g)
    rc, rs, rg = O.quantize_ref(x, g)
    assert gg == rg, (gg, rg)
    assert np.array_equal(s, rs), f"scale mismatch at {np.argwhere(s != rs)[:5]}"
    assert np.array_equal(c, rc), f"code mismatch at {np.argwhere(c != rc)[:5]}"


# ------------------------------------------------------------------ quantiser
def test_quantize_tiny_fp32_dynamic(gpu_lib):
    (lin,) = synth.make_workload("tiny")
    assert_quant_equal(gpu_lib, lin.a, "f32", None, "tiny A")
    assert_quant_equal(gpu_lib, lin.modules[0][1], "f32", None, "tiny W")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_quantize_random_static_and_dynamic(gpu_lib, dtype):
    rng = np.random.default_rng(21)
    for rows, cols in ((1, 16), (3, 48), (37, 272), (129, 1040)):
        x = (rng.standard_t(3, (rows, cols)) * 2).astype(np.float32)
        x[:, rng.integers(0, cols)] *= 50
        x = synth.round_to_bf16(x) if dtype == "bf16" else (np.clip(x, -6e4, 6e4).astype(np.float16).astype(np.float32) if dtype == "f16" else x)
        assert_quant_equal(gpu_lib, x, dtype, None, f"random {rows}x{cols}")
        assert_quant_equal(gpu_lib, x, dtype, np.float32(37.5), f"random {rows}x{cols}")


def test_quantize_adversarial_blocks(gpu_lib):
    """Ties of E2M1 after scaling, zero blocks, underflowing blocks, static-g
    saturation and negative zeros."""
    g = np.float32(1.0)
    grid = np.array([0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 6], np.float32)
    rows = [grid, -grid, np.zeros(16, np.float32), np.full(16, -0.0, np.float32),
            np.array([1e-30] + [0] * 15, np.float32), np.array([100, -80, 3, 0.1] + [0] * 12, np.float32),
            np.nextafter(grid, np.float32(10)), np.nextafter(grid, np.float32(-10))]
    x = np.stack(rows).astype(np.float32)
    x[:, -1] = 6.0  # block amax 6 so that scale = 1 and y = x exactly
    assert_quant_equal(gpu_lib, x, "f32", g, "ties and edges")
    assert_quant_equal(gpu_lib, x, "f32", np.float32(1e-7), "underflow")
    assert_quant_equal(gpu_lib, x, "f32", np.float32(1e4), "saturation")
    assert_quant_equal(gpu_lib, x, "f32", None, "dynamic")
    assert_quant_equal(gpu_lib, np.zeros((4, 64), np.float32), "f32", None, "all zero")


def test_quantize_strided_rows(gpu_lib):
    rng = np.random.default_rng(22)
    x = synth.round_to_bf16(rng.standard_normal((20, 96)).astype(np.float32))
    full = np.zeros((20, 128), np.float32)
    full[:, :96] = x
    t = dev_bf16(full)[:, :96]
    gs = gscale_tensor(0)
    codes, scales = gpu_lib.nvfp4_quantize(t, gs, "dynamic")
    rc, rs, rg = O.quantize_ref(x)
    assert np.array_equal(codes.cpu().numpy(), rc) and np.array_equal(scales.cpu().numpy(), rs)
    assert np.float32(gs.item()) == rg


def test_quantize_deterministic(gpu_lib):
    rng = np.random.default_rng(23)
    x = synth.round_to_bf16(rng.standard_normal((512, 5120)).astype(np.float32))
    a = quantize_gpu(gpu_lib, x, "bf16", None)
    b = quantize_gpu(gpu_lib, x, "bf16", None)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))


def _random_quant_cases(n, seed):
    """Seeded random quantiser cases: rows 1-600, cols any multiple of 16 up to
    6384, each input dtype, padded row strides, static or dynamic global scale,
    and value sets from normal to wide-range (x 2^-20..2^20), tiny, mostly zero
    and outlier columns."""
    rng = np.random.default_rng(seed)
    return [(int(rng.choice([rng.integers(1, 8), rng.integers(8, 600)])), int(16 * rng.integers(1, 400)),
             str(rng.choice(["f32", "bf16", "f16"])), int(rng.choice([0, 0, 8, 24])),
             str(rng.choice(["normal", "wide", "tiny", "zeros", "outliers"])), str(rng.choice(["dynamic", "static"])))
            for _ in range(n)]


@pytest.mark.parametrize("case", _random_quant_cases(24, 2027))
def test_quantize_seeded_random_cases(gpu_lib, case):
    rows, cols, dt, pad, dist, mode = case
    rng = np.random.default_rng([32, rows, cols, pad])
    if dist == "normal":
        x = rng.standard_normal((rows, cols))
    elif dist == "wide":
        x = rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-20, 20, (rows, cols)))
    elif dist == "tiny":
        x = rng.standard_normal((rows, cols)) * 1e-6
    elif dist == "zeros":
        x = np.where(rng.random((rows, cols)) < 0.7, 0.0, rng.standard_normal((rows, cols)))
    else:
        x = rng.standard_normal((rows, cols))
        x[:, rng.integers(0, cols, 3)] *= 1000
    x = x.astype(np.float32)
    if dt == "f16":
        x = np.clip(x, -60000, 60000).astype(np.float16).astype(np.float32)
    elif dt == "bf16":
        x = synth.round_to_bf16(x).astype(np.float32)
    g = None if mode == "dynamic" else np.float32(rng.uniform(0.1, 1e4))
    log("quantize random", case)
    full = np.zeros((rows, cols + pad), np.float32)
    full[:, :cols] = x
    t = {"f32": dev_f32, "bf16": dev_bf16, "f16": dev_f16}[dt](full)[:, :cols]
    gs = gscale_tensor(0.0 if g is None else g)
    codes, scales = gpu_lib.nvfp4_quantize(t, gs, mode)
    torch.cuda.synchronize()
    rc, rs, rg = O.quantize_ref(x, g)
    assert np.float32(gs.item()) == rg
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


# ------------------------------------------------------------------ fuse-rescale
def test_fuse_rescale_matches_oracle(gpu_lib):
    rng = np.random.default_rng(24)
    rows = [96, 64, 3, 5]
    K = 256
    qs = []
    for i, r in enumerate(rows):
        w = (rng.standard_normal((r, K)) * [0.021, 0.017, 0.005, 0.09][i]).astype(np.float32)
        qs.append(quantize_gpu(gpu_lib, synth.round_to_bf16(w), "bf16", None))
    scales = np.concatenate([q[1] for q in qs])
    gs = [q[2] for q in qs]
    log("fuse", rows, gs)
    t = torch.from_numpy(scales.copy()).cuda()
    g_star, lossy = gpu_lib.nvfp4_fuse_rescale(t, K, rows, gs)
    torch.cuda.synchronize()
    ref, ref_g, ref_lossy = O.fuse_rescale_ref(scales, rows, gs)
    assert np.float32(g_star) == ref_g
    assert np.array_equal(t.cpu().numpy(), ref)
    assert int(lossy.item()) == ref_lossy


def test_fuse_rescale_single_module_is_identity(gpu_lib):
    s = np.random.default_rng(25).integers(0, 0x7F, (7, 4)).astype(np.uint8)
    t = torch.from_numpy(s.copy()).cuda()
    g, lossy = gpu_lib.nvfp4_fuse_rescale(t, 64, [7], [3.0])
    torch.cuda.synchronize()
    assert g == 3.0 and np.array_equal(t.cpu().numpy(), s) and int(lossy.item()) == 0


# ------------------------------------------------------------------ GEMM
def rand_operand(rng, rows, K, scale_lo=0x20, scale_hi=0x58):
    codes = rng.integers(0, 256, (rows, K // 2)).astype(np.uint8)
    scales = rng.integers(scale_lo, scale_hi, (rows, K // 16)).astype(np.uint8)
    return codes, scales


def gemm_gpu(nv, ac, asc, ga, wc, wsc, gw, out_dtype):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    c = nv.nvfp4_gemm(t(ac), t(asc), gscale_tensor(ga), t(wc), t(wsc), gscale_tensor(gw),
                      out_dtype={"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out_dtype])
    torch.cuda.synchronize()
    return c.float().cpu().numpy()


def check_gemm(C, ref, bound, out_dtype):
    err = np.abs(C.astype(np.float64) - ref)
    lim = 1e-5 * bound
    if out_dtype == "bf16":
        lim = lim + 2.0 ** -8 * np.abs(ref)
    elif out_dtype == "f16":
        lim = lim + 2.0 ** -11 * np.abs(ref) + 2.0 ** -24
    bad = err > lim
    assert not bad.any(), f"{int(bad.sum())} elements out of tolerance, worst at {np.argwhere(bad)[:3]}, " \
                          f"err {err[bad][:3]}, lim {lim[bad][:3]}"
    zero_rows = bound == 0
    assert np.all(C[zero_rows] == 0)


# with k % 128 == 0, m <= 64 takes the decode-shaped (weight-streaming) path, m > 256 the main
# prefill (direct-to-LDS) path and 64 < m <= 256 whichever is estimated faster; other shapes the
# generic one
GEMM_SHAPES = [(64, 128, 256), (300, 520, 384), (1, 1, 16), (33, 257, 400), (256, 256, 128), (513, 300, 1056),
               (32, 1000, 640), (7, 333, 48), (64, 96, 4096),
               (16, 4352, 5120), (48, 777, 1024), (1, 300, 192), (32, 129, 64), (64, 33, 128), (32, 4096, 320),
               (33, 520, 2048), (32, 1000, 768), (17, 300, 256), (1, 4099, 1280), (32, 4352, 5120), (31, 100, 2048),
               (32, 520, 17408), (8, 2000, 5120), (32, 700, 6144),
               (64, 4352, 5120), (57, 300, 8192), (40, 130, 7424), (64, 70, 7680),  # 64-row decode block
               (9, 200, 9216), (5, 130, 17408), (24, 1100, 6144), (3, 9000, 4096), (12, 37000, 512),  # LDS-resident A or not
               (32, 30000, 5888), (16, 25000, 5632),  # LDS-resident A near the size of the LDS
               (2, 1, 256), (32, 5, 512), (4, 36864, 256), (4, 36865, 256),  # fewer rows than a tile; one round or not
               (32, 30000, 512), (16, 26000, 1024), (20, 24576, 512), (20, 24577, 512), (40, 17000, 256),  # kernel choice by grid
               (2048, 8256, 512),  # 264 tiles, a 64-column ragged edge at scale
               (100, 100, 128), (300, 1000, 640), (1024, 2000, 896), (520, 600, 2176), (2048, 1536, 2176),  # K % 512 != 0
               (32, 600, 2176), (9, 1000, 384), (64, 300, 640), (1, 130, 128), (20, 24577, 384), (48, 5000, 1152),  # K % 256 == 128
               (96, 5000, 5120), (160, 4352, 2176), (250, 1024, 4096), (200, 700, 2176),  # 65-256 rows in 64-row decode blocks
               (65, 64, 256), (300, 520, 512), (513, 777, 1024), (257, 300, 256), (1000, 1000, 2560), (256, 512, 5120),
               (512, 32832, 1024), (700, 21800, 640), (6000, 8288, 256),  # a ragged last column strip on the decode-shaped kernel (256 CUs)
               (100, 5120, 1024), (40, 10000, 512), (200, 3000, 4096),  # 64-row decode blocks with 3 weight tiles: one workgroup per CU (256 CUs)
               (32, 10240, 512), (9, 9000, 256), (32, 4352, 1024), (5, 640, 768),
               (32, 17408, 512), (12, 20000, 256),  # activations in LDS, 2 quads of 1, 2 or 3 weight tiles
               (32, 65536, 256),  # activations in LDS, 144-row workgroups over two rounds
               # weight streaming (up to 32 rows, k 4096 or 5120, 80-144 weight rows per CU on 256 CUs):
               # the decode benchmark's shape, ragged slabs, a last workgroup of one row, 1 and 2 activation tiles
               (32, 34816, 5120), (1, 20488, 4096), (17, 36864, 4096), (16, 30001, 5120), (32, 25000, 4096),
               (5, 36863, 5120),
               # a part-empty last round of 256x256 tiles whose columns go to 256x128 tiles (256 CUs: 320 tiles
               # -> 256 + 128 columns of 16 row tiles), K a whole number of four-stage groups or not, ragged M
               (4096, 5120, 1024), (4000, 5120, 1152)]


@pytest.mark.parametrize("shape", GEMM_SHAPES)
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gemm_random_codes(gpu_lib, shape, out_dtype):
    M, N, K = shape
    rng = np.random.default_rng([26, M, N, K])
    ac, asc = rand_operand(rng, M, K)
    wc, wsc = rand_operand(rng, N, K)
    ga, gw = np.float32(rng.uniform(0.5, 300)), np.float32(rng.uniform(100, 3e4))
    log("gemm", shape, out_dtype)
    C = gemm_gpu(gpu_lib, ac, asc, ga, wc, wsc, gw, out_dtype)
    ref, bound = O.gemm_ref(ac, asc, ga, wc, wsc, gw)
    check_gemm(C, ref, bound, out_dtype)


# the persistent form of the prefill kernel (whole 256x256 tiles, at least three per CU, K a multiple of
# 512; on 256 CUs): the fewest stages (K = 512, the last group of four the only one) at exactly three
# tiles per workgroup, and tile counts that are not a whole number of rounds (some workgroups take one
# tile more); a single row of 769 tiles (a count that is not a multiple of the 8 XCDs); the ragged
# shape has as many tiles but runs the one-tile kernel
PERSISTENT_SHAPES = [(4096, 12288, 512), (6144, 8448, 1024), (3072, 16640, 1536), (256, 196864, 512),
                     (4000, 8400, 1024)]


@pytest.mark.parametrize("shape", PERSISTENT_SHAPES)
@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
def test_gemm_persistent_prefill(gpu_lib, shape, out_dtype):
    M, N, K = shape
    rng = np.random.default_rng([33, M, N, K])
    ac, asc = rand_operand(rng, M, K)
    wc, wsc = rand_operand(rng, N, K)
    ga, gw = np.float32(rng.uniform(0.5, 300)), np.float32(rng.uniform(100, 3e4))
    log("gemm persistent", shape, out_dtype)
    C = gemm_gpu(gpu_lib, ac, asc, ga, wc, wsc, gw, out_dtype)
    ref, bound = O.gemm_ref(ac, asc, ga, wc, wsc, gw)
    check_gemm(C, ref, bound, out_dtype)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
def test_gemm_persistent_prefill_strided_output(gpu_lib, out_dtype):
    """The persistent prefill kernel writing every output dtype into rows of an
    odd stride (no 16-byte stores): the columns past n stay untouched."""
    M, N, K = 4096, 12288, 1024
    rng = np.random.default_rng([34, M, N, K])
    ac, asc = rand_operand(rng, M, K)
    wc, wsc = rand_operand(rng, N, K)
    ga, gw = np.float32(rng.uniform(0.5, 300)), np.float32(rng.uniform(100, 3e4))
    log("gemm persistent strided", (M, N, K), out_dtype)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out_dtype]
    ldc = N + 37
    big = torch.full((M, ldc), 7.0, dtype=tdt, device="cuda")
    out = big[:, :N]
    gpu_lib.nvfp4_gemm(t(ac), t(asc), gscale_tensor(ga), t(wc), t(wsc), gscale_tensor(gw), out=out)
    torch.cuda.synchronize()
    ref, bound = O.gemm_ref(ac, asc, ga, wc, wsc, gw)
    check_gemm(out.float().cpu().numpy(), ref, bound, out_dtype)
    assert torch.all(big[:, N:] == 7.0).item(), "columns past n were written"


def _random_gemm_cases(n, seed):
    """Seeded random shapes over every GEMM path: 1-64, 65-256 and more rows,
    N from a handful to the LDS-resident kernel's range, K any multiple of 16
    up to 8192 (biased to multiples of 128, 256 and 512), scale operands at a
    byte offset of 0, 4 or 1, and each output dtype."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        m = int(rng.choice([rng.integers(1, 33), rng.integers(1, 65), rng.integers(65, 257), rng.integers(257, 1200)]))
        big_n = rng.integers(20000, 40000) if m <= 64 else rng.integers(300, 3000)
        nn = int(rng.choice([rng.integers(1, 300), rng.integers(300, 5000), big_n]))
        kb = int(rng.choice([16, 128, 256, 512]))
        k = min(int(kb * rng.integers(1, max(2, 8192 // kb))), 8192)
        cases.append((m, nn, k, int(rng.choice([0, 0, 0, 4, 1])), str(rng.choice(["f32", "bf16", "f16"]))))
    return cases


@pytest.mark.parametrize("case", _random_gemm_cases(40, 2026))
def test_gemm_seeded_random_shapes(gpu_lib, case):
    M, N, K, off, out_dtype = case
    rng = np.random.default_rng([31, M, N, K, off])
    ac, asc = rand_operand(rng, M, K)
    wc, wsc = rand_operand(rng, N, K)
    ga, gw = np.float32(rng.uniform(0.5, 300)), np.float32(rng.uniform(100, 3e4))
    log("gemm random", case)

    def dev_at(a, o):
        flat = torch.zeros(a.size + 64, dtype=torch.uint8, device="cuda")
        flat[o:o + a.size] = torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).cuda()
        return flat[o:o + a.size].view(a.shape)

    c = gpu_lib.nvfp4_gemm(dev_at(ac, 0), dev_at(asc, off), gscale_tensor(ga), dev_at(wc, 0), dev_at(wsc, off),
                           gscale_tensor(gw),
                           out_dtype={"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out_dtype])
    torch.cuda.synchronize()
    ref, bound = O.gemm_ref(ac, asc, ga, wc, wsc, gw)
    check_gemm(c.float().cpu().numpy(), ref, bound, out_dtype)


@pytest.mark.parametrize("shape", [(20, 700, 1024), (9, 300, 2048), (32, 500, 5120), (50, 260, 1536), (100, 300, 1024),
                                   (512, 32832, 512), (32, 30000, 5120), (4096, 5120, 1024), (4000, 8400, 1024),
                                   (6144, 8448, 1024)])
@pytest.mark.parametrize("scale_offset", [0, 4, 1])
def test_gemm_offset_scales_strided_output(gpu_lib, shape, scale_offset):
    """Scale operands off a 16-byte boundary (legal: the ABI puts no alignment
    on scales) take the paths that load scales from memory, or the generic
    kernel at a byte offset; outputs go to an odd row stride, and the columns
    past n stay untouched."""
    M, N, K = shape
    rng = np.random.default_rng([28, M, N, K, scale_offset])
    ac, asc = rand_operand(rng, M, K)
    wc, wsc = rand_operand(rng, N, K)
    ga, gw = np.float32(rng.uniform(0.5, 300)), np.float32(rng.uniform(100, 3e4))
    log("gemm offset/strided", shape, scale_offset)

    def dev_at(a, off):
        flat = torch.zeros(a.size + 64, dtype=torch.uint8, device="cuda")
        flat[off:off + a.size] = torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).cuda()
        return flat[off:off + a.size].view(a.shape)

    ldc = N + 37
    big = torch.full((M, ldc), 7.0, dtype=torch.float32, device="cuda")
    out = big[:, :N]
    gpu_lib.nvfp4_gemm(dev_at(ac, 0), dev_at(asc, scale_offset), gscale_tensor(ga), dev_at(wc, 0),
                       dev_at(wsc, scale_offset), gscale_tensor(gw), out=out)
    torch.cuda.synchronize()
    ref, bound = O.gemm_ref(ac, asc, ga, wc, wsc, gw)
    check_gemm(out.cpu().numpy(), ref, bound, "f32")
    assert torch.all(big[:, N:] == 7.0).item(), "columns past n were written"


# the second shape ends in a 40-column strip on the decode-shaped kernel (256 CUs); the third streams the weight
@pytest.mark.parametrize("shape", [(70, 90, 512), (700, 21800, 640), (24, 30000, 4096)])
def test_gemm_f16_output(gpu_lib, shape):
    M, N, K = shape
    rng = np.random.default_rng(27)
    ac, asc = rand_operand(rng, M, K, 0x30, 0x40)
    wc, wsc = rand_operand(rng, N, K, 0x30, 0x40)
    C = gemm_gpu(gpu_lib, ac, asc, np.float32(64), wc, wsc, np.float32(64), "f16")
    ref, bound = O.gemm_ref(ac, asc, np.float32(64), wc, wsc, np.float32(64))
    check_gemm(C, ref, bound, "f16")


@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", [(20, 24000, 5120), (9, 33001, 4096)])
def test_gemm_stream_strided_output(gpu_lib, shape, out_dtype):
    """The weight-streaming kernel writing every output dtype into rows of an
    odd stride (no 16-byte stores): the columns past n stay untouched."""
    M, N, K = shape
    rng = np.random.default_rng([29, M, N, K])
    ac, asc = rand_operand(rng, M, K)
    wc, wsc = rand_operand(rng, N, K)
    ga, gw = np.float32(rng.uniform(0.5, 300)), np.float32(rng.uniform(100, 3e4))
    log("gemm stream strided", shape, out_dtype)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out_dtype]
    ldc = N + 37
    big = torch.full((M, ldc), 7.0, dtype=tdt, device="cuda")
    out = big[:, :N]
    gpu_lib.nvfp4_gemm(t(ac), t(asc), gscale_tensor(ga), t(wc), t(wsc), gscale_tensor(gw), out=out)
    torch.cuda.synchronize()
    ref, bound = O.gemm_ref(ac, asc, ga, wc, wsc, gw)
    check_gemm(out.float().cpu().numpy(), ref, bound, out_dtype)
    assert torch.all(big[:, N:] == 7.0).item(), "columns past n were written"


def test_gemm_extreme_scales(gpu_lib):
    """Smallest and largest decoded magnitudes (E4M3 subnormal 2^-9 and 448 with
    codes 0.5 and 6) stay exact through the fp16 decode."""
    K = 256
    for sc in (0x01, 0x07, 0x08, 0x7E):
        ac = np.full((40, K // 2), 0x71, np.uint8)  # elements 0.5, 6, 0.5, 6, ...
        asc = np.full((40, K // 16), sc, np.uint8)
        wc = np.full((50, K // 2), 0x9F, np.uint8)  # -6, -0.5, ...
        wsc = np.full((50, K // 16), 0x38, np.uint8)
        C = gemm_gpu(gpu_lib, ac, asc, np.float32(1), wc, wsc, np.float32(1), "f32")
        ref, bound = O.gemm_ref(ac, asc, np.float32(1), wc, wsc, np.float32(1))
        assert np.array_equal(C.astype(np.float64), ref), sc


def test_gemm_zero_operand_gives_exact_zeros(gpu_lib):
    rng = np.random.default_rng(28)
    ac = np.zeros((65, 128), np.uint8)
    asc = rng.integers(0, 0x7F, (65, 16)).astype(np.uint8)
    wc, wsc = rand_operand(rng, 70, 256)
    C = gemm_gpu(gpu_lib, ac, asc, np.float32(1), wc, wsc, np.float32(1), "f32")
    assert np.all(C == 0)


@pytest.mark.parametrize("shape", [(300, 600, 1024), (512, 32832, 1024), (32, 34816, 5120), (3072, 16640, 1536)])
def test_gemm_deterministic(gpu_lib, shape):
    M, N, K = shape
    rng = np.random.default_rng(29)
    ac, asc = rand_operand(rng, M, K)
    wc, wsc = rand_operand(rng, N, K)
    a = gemm_gpu(gpu_lib, ac, asc, np.float32(3), wc, wsc, np.float32(5), "f32")
    b = gemm_gpu(gpu_lib, ac, asc, np.float32(3), wc, wsc, np.float32(5), "f32")
    assert np.array_equal(a, b)


# ------------------------------------------------------------------ end to end, tiny workload
def test_tiny_end_to_end(gpu_lib):
    (lin,) = synth.make_workload("tiny")
    a, w = lin.a, lin.modules[0][1]
    ga_t = gscale_tensor(0)
    gw_t = gscale_tensor(0)
    ac, asc = gpu_lib.nvfp4_quantize(dev_f32(a), ga_t, "dynamic")
    wc, wsc = gpu_lib.nvfp4_quantize(dev_f32(w), gw_t, "dynamic")
    C = gpu_lib.nvfp4_gemm(ac, asc, ga_t, wc, wsc, gw_t, torch.float32).cpu().numpy()
    rac, rasc, rga = O.quantize_ref(a)
    rwc, rwsc, rgw = O.quantize_ref(w)
    assert np.array_equal(ac.cpu().numpy(), rac) and np.array_equal(wc.cpu().numpy(), rwc)
    ref, bound = O.gemm_ref(rac, rasc, rga, rwc, rwsc, rgw)
    check_gemm(C, ref, bound, "f32")
