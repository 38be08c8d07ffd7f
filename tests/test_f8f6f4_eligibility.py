"""When could gfx950's block-scaled f8f6f4 MFMA take NVFP4 operands exactly?

That instruction scales raw E2M1 codes by one power-of-two (E8M0) factor per
32 elements of a row.  NVFP4 gives every 16 elements their own E4M3 scale
(news article "Qwen3.8-27B最激进4bit量化开源，权重显存暴降2.9倍！", section 02), so
a 32-element group maps onto it exactly only when its two 16-block scales are
equal and a power of two; one MFMA tile step needs that for all 32 rows of
both operands.  This measures the eligible fraction on the seeded workloads
(sampled rows, through the CPU oracle's quantiser) and checks that the test
does detect eligibility where it exists."""
import numpy as np

from nvfp4_w4a4_block_quantize_amd import synth
from oracle import nvfp4_oracle as O


def eligible(scales):
    """Per (row, 32-element group): both E4M3 block scales equal and a power of two."""
    s = scales.reshape(scales.shape[0], -1, 2).astype(np.int64)
    e, m = (s[:, :, 0] >> 3) & 15, s[:, :, 0] & 7
    pow2 = np.where(e == 0, (m & (m - 1)) == 0, m == 0)  # normal: no mantissa bits; subnormal: one bit
    return (s[:, :, 0] == s[:, :, 1]) & pow2


def tile_steps(ok):
    """Per (32-row tile, 32-element group): every row of the tile eligible."""
    rows = ok.shape[0] // 32 * 32
    return ok[:rows].reshape(-1, 32, ok.shape[1]).all(axis=1)


def test_detects_eligible_data():
    # a block of all +1 with g = 1: S = E4M3(1/6) is not a power of two; with
    # amax 6 per block the scale is exactly 1.0 = 2^0 in both blocks of a group
    x = np.ones((64, 256), dtype=np.float32)
    x[:, ::16] = 6.0
    _, s, _ = O.quantize_ref(x, np.float32(1.0))
    ok = eligible(s)
    assert ok.all() and tile_steps(ok).all()


def test_workloads_are_essentially_never_eligible():
    report = []
    for cfg, rows in (("gdn", 128), ("decode", 32), ("mlp", 128)):
        for lin in synth.make_workload(cfg, m_override=rows):
            _, sa, _ = O.quantize_ref(lin.a[:rows], O.global_scale(lin.a_calib))
            w = lin.modules[0][1][:256]
            _, sw, _ = O.quantize_ref(w)
            fa, fw = eligible(sa).mean(), eligible(sw).mean()
            ta, tw = tile_steps(eligible(sa)).mean(), tile_steps(eligible(sw)).mean()
            report.append((lin.name, fa, fw, ta, tw))
            # a few percent of groups at most, and no whole tile step
            assert fa < 0.05 and fw < 0.05, report[-1]
            assert ta == 0.0 and tw == 0.0, report[-1]
    print(report)
