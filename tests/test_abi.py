"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and rejects invalid arguments before touching HIP (a rejected call
returns its status without any device work, so these run without a GPU)."""
import ctypes
import os
import re

import pytest

import nvfp4_w4a4_block_quantize_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:nvfp4_status|const char\s*\*|int32_t)\s*(nvfp4_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(os.environ.get("NVFP4_ABI_LIB") or nv.LIB_PATH):
        pytest.skip("libnvfp4.so not built")
    # NVFP4_ABI_LIB: another build of the C-ABI layer (the sanitized host build)
    return nv.load_library(os.environ.get("NVFP4_ABI_LIB"))


def test_header_declares_the_three_operations():
    fns = declared_functions()
    for name in ("nvfp4_quantize", "nvfp4_fuse_rescale", "nvfp4_gemm", "nvfp4_status_str", "nvfp4_abi_version"):
        assert name in fns


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(nv.SIGNATURES)


def test_abi_version_and_status_strings(lib):
    assert lib.nvfp4_abi_version() == 1
    for s in range(7):
        assert len(lib.nvfp4_status_str(s)) > 0
    assert lib.nvfp4_status_str(99) == b"unknown status"


# a fake, 256-byte-aligned "device" address: validation never dereferences it
P = 1 << 20


def q(lib, **kw):
    a = dict(x=P, x_dtype=1, rows=4, cols=32, ldx=32, gscale=P, mode=0, codes=P, scales=P, stream=None)
    a.update(kw)
    return lib.nvfp4_quantize(a["x"], a["x_dtype"], a["rows"], a["cols"], a["ldx"], a["gscale"], a["mode"],
                              a["codes"], a["scales"], a["stream"])


def test_quantize_validation(lib):
    assert q(lib, x=None) == 1
    assert q(lib, codes=None) == 1
    assert q(lib, x_dtype=7) == 4
    assert q(lib, mode=3) == 4
    assert q(lib, rows=0) == 2
    assert q(lib, cols=24) == 2
    assert q(lib, ldx=16) == 2
    assert q(lib, cols=-16) == 2
    assert q(lib, x=P + 8) == 3
    assert q(lib, x_dtype=1, ldx=36) == 3  # 36 bf16 = 72 bytes, not a multiple of 16
    assert q(lib, codes=P + 2) == 3


def g(lib, **kw):
    a = dict(m=8, n=8, k=32, ac=P, asc=P, ag=P, wc=P, wsc=P, wg=P, c=P, dt=0, ldc=8)
    a.update(kw)
    return lib.nvfp4_gemm(a["m"], a["n"], a["k"], a["ac"], a["asc"], a["ag"], a["wc"], a["wsc"], a["wg"], a["c"],
                          a["dt"], a["ldc"], None)


def test_gemm_validation(lib):
    assert g(lib, ac=None) == 1
    assert g(lib, wg=None) == 1
    assert g(lib, c=None) == 1
    assert g(lib, dt=5) == 4
    assert g(lib, m=0) == 2
    assert g(lib, k=40) == 2
    assert g(lib, ldc=4) == 2
    assert g(lib, ac=P + 8) == 3
    assert g(lib, c=P + 2, dt=0) == 3


def f(lib, rows=(4, 4), gs=(1.0, 2.0), k=32, scales=P, out=True):
    n = len(rows)
    r = (ctypes.c_int64 * max(n, 1))(*rows)
    gg = (ctypes.c_float * max(n, 1))(*gs)
    o = ctypes.c_float(-1.0)
    st = lib.nvfp4_fuse_rescale(scales, k, n, ctypes.cast(r, ctypes.c_void_p), ctypes.cast(gg, ctypes.c_void_p),
                                ctypes.addressof(o) if out else None, None, None)
    return st, o.value


def test_fuse_rescale_validation_writes_nothing_on_error(lib):
    assert f(lib, scales=None) == (1, -1.0)
    assert f(lib, out=False)[0] == 1
    assert f(lib, k=24) == (2, -1.0)
    assert f(lib, rows=(4, 0)) == (2, -1.0)
    assert f(lib, gs=(1.0, 0.0)) == (5, -1.0)
    assert f(lib, gs=(1.0, float("inf"))) == (5, -1.0)
    assert f(lib, gs=(float("nan"), 1.0)) == (5, -1.0)
    assert f(lib, rows=(), gs=()) == (5, -1.0)
    assert f(lib, rows=(1,) * 65, gs=(1.0,) * 65) == (5, -1.0)


def test_amax_observe_validation(lib):
    obs = lib.nvfp4_amax_observe
    assert obs(None, 1, 4, 32, 32, P, None) == 1
    assert obs(P, 1, 4, 32, 32, None, None) == 1
    assert obs(P, 7, 4, 32, 32, P, None) == 4
    assert obs(P, 1, 0, 32, 32, P, None) == 2
    assert obs(P, 1, 4, 12, 12, P, None) == 2   # cols not a multiple of 8
    assert obs(P, 1, 4, 32, 16, P, None) == 2   # ldx < cols
    assert obs(P + 8, 1, 4, 32, 32, P, None) == 3
    assert obs(P, 1, 4, 32, 36, P, None) == 3   # row pitch not a multiple of 16 bytes
    assert lib.nvfp4_gscale_from_amax(None, P, None) == 1
    assert lib.nvfp4_gscale_from_amax(P, None, None) == 1
    assert lib.nvfp4_gscale_from_amax(P + 2, P, None) == 3


def test_kv_quantize_validation(lib):
    kv = lib.nvfp4_kv_quantize_fp8
    assert kv(None, 1, 4, 32, 32, P, P, None) == 1
    assert kv(P, 1, 4, 32, 32, None, P, None) == 1
    assert kv(P, 1, 4, 32, 32, P, None, None) == 1
    assert kv(P, 9, 4, 32, 32, P, P, None) == 4
    assert kv(P, 1, 4, 12, 12, P, P, None) == 2
    assert kv(P, 1, 4, 32, 16, P, P, None) == 2
    assert kv(P, 1, 4, 32, 32, P, P + 4, None) == 3
    assert lib.nvfp4_kv_scale_from_amax(None, P, None) == 1
    assert lib.nvfp4_kv_scale_from_amax(P, P + 1, None) == 3


def test_valid_calls_without_a_gpu_return_device_error(lib):
    """Every launching entry point validates its arguments, then finds no
    usable GPU and returns NVFP4_ERR_DEVICE without writing anything (the
    host output of nvfp4_fuse_rescale keeps its value)."""
    if os.environ.get("NVFP4_NO_GPU") != "1":
        torch = pytest.importorskip("torch")
        if torch.cuda.device_count() > 0:
            pytest.skip("a GPU is visible: valid calls would launch kernels on these placeholder addresses")
    assert q(lib) == 6
    assert q(lib, mode=1) == 6
    assert g(lib) == 6
    assert g(lib, m=32, n=34816, k=5120, ldc=34816, dt=1) == 6
    assert f(lib) == (6, -1.0)
    assert lib.nvfp4_amax_observe(P, 1, 4, 32, 32, P, None) == 6
    assert lib.nvfp4_gscale_from_amax(P, P, None) == 6
    assert lib.nvfp4_kv_quantize_fp8(P, 1, 4, 32, 32, P, P, None) == 6
    assert lib.nvfp4_kv_scale_from_amax(P, P, None) == 6


def test_binding_rejects_bad_buffers_before_the_call():
    """The Python binding checks caller-supplied outputs and scale tensors
    (dtype, shape, contiguity, one fp32 element) before the C call; a wrong
    buffer is rejected, never passed on to be written out of bounds."""
    torch = pytest.importorskip("torch")
    x = torch.zeros((4, 32), dtype=torch.bfloat16)
    g1 = torch.zeros(1, dtype=torch.float32)
    codes, scales = torch.zeros((4, 16), dtype=torch.uint8), torch.zeros((4, 2), dtype=torch.uint8)
    with pytest.raises(ValueError, match="codes must have shape"):
        nv.nvfp4_quantize(x, g1, codes=torch.zeros((4, 8), dtype=torch.uint8), scales=scales)
    with pytest.raises(ValueError, match="scales must be uint8"):
        nv.nvfp4_quantize(x, g1, codes=codes, scales=torch.zeros((4, 2), dtype=torch.int16))
    with pytest.raises(ValueError, match="codes must be contiguous"):
        nv.nvfp4_quantize(x, g1, codes=torch.zeros((16, 4), dtype=torch.uint8).t(), scales=scales)
    with pytest.raises(ValueError, match="gscale must be a float32 tensor with one element"):
        nv.nvfp4_quantize(x, torch.zeros(1, dtype=torch.bfloat16), codes=codes, scales=scales)
    with pytest.raises(ValueError, match="gscale must be a float32 tensor with one element"):
        nv.nvfp4_quantize(x, torch.zeros(2, dtype=torch.float32), codes=codes, scales=scales)
    with pytest.raises(ValueError, match="mode must be"):
        nv.nvfp4_quantize(x, g1, mode="Static", codes=codes, scales=scales)
    with pytest.raises(ValueError, match="must be a GPU tensor"):  # every buffer right, but on the host
        nv.nvfp4_quantize(x, g1, codes=codes, scales=scales)
    ac, asc = torch.zeros((2, 16), dtype=torch.uint8), torch.zeros((2, 2), dtype=torch.uint8)
    wc, wsc = torch.zeros((3, 16), dtype=torch.uint8), torch.zeros((3, 2), dtype=torch.uint8)
    with pytest.raises(ValueError, match="w_codes must have shape"):
        nv.nvfp4_gemm(ac, asc, g1, torch.zeros((3, 8), dtype=torch.uint8), wsc, g1)
    with pytest.raises(ValueError, match="a_scales must have shape"):
        nv.nvfp4_gemm(ac, torch.zeros((2, 4), dtype=torch.uint8), g1, wc, wsc, g1)
    with pytest.raises(ValueError, match="w_gscale must be a float32"):
        nv.nvfp4_gemm(ac, asc, g1, wc, wsc, torch.zeros(1, dtype=torch.float64))
    with pytest.raises(ValueError, match="scales must have shape"):
        nv.nvfp4_fuse_rescale(torch.zeros((5, 2), dtype=torch.uint8), 32, [2, 2], [1.0, 2.0])
    with pytest.raises(ValueError, match="out must have shape"):
        nv.nvfp4_kv_quantize_fp8(x, g1, out=torch.zeros((4, 16), dtype=torch.uint8))
    with pytest.raises(ValueError, match="amax_state must be a float32"):
        nv.nvfp4_amax_observe(x, torch.zeros(1, dtype=torch.int32))
