"""Reusable pin checks for the oracle.

Each check takes the implementation under test as an argument and returns a
count of violations, so the same checks run against the oracle (expecting 0)
and against deliberately broken copies of it (expecting > 0, see
test_oracle_mutations.py).  The references used here are independent of the
oracle's own code: exact rationals (fractions.Fraction), torch's float8 cast,
brute-force argmin over the value grid, and closed forms.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# E2M1 grid written from the bit layout s|e1e0|m, bias 1 (independent of the oracle's decoder)
E2M1_FRACTIONS = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def e4m3_fraction_table():
    """All 127 finite non-negative E4M3FN values as (byte, Fraction)."""
    out = []
    for b in range(0x7F):
        e, m = b >> 3, b & 7
        v = Fraction(m, 8) * Fraction(1, 2 ** 6) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        out.append((b, v))
    return out


E4M3_TABLE = e4m3_fraction_table()


def count_changed_dequant_factors(old_scales, new_scales, module_rows, module_gscales, g_star):
    """Blocks of a fused group whose dequantisation factor changed: exact
    rationals, per block, e4m3(S') / g* against e4m3(S) / g_i (the news
    article, section 03: the repair folds g*/g_i into the block scales, so a
    block is reproduced exactly when the two factors are equal)."""
    val = dict(E4M3_TABLE)
    old_scales, new_scales = np.asarray(old_scales), np.asarray(new_scales)
    gs = Fraction(float(np.float32(g_star)))
    n, r0 = 0, 0
    for rows, g in zip(module_rows, module_gscales):
        gi = Fraction(float(np.float32(g)))
        for b_old, b_new in zip(old_scales[r0:r0 + rows].ravel(), new_scales[r0:r0 + rows].ravel()):
            if val[int(b_new)] / gs != val[int(b_old)] / gi:
                n += 1
        r0 += rows
    return n


def e2m1_exact(y: float) -> int:
    """Nearest E2M1 code by exact rational distance, ties to the even code, saturating."""
    a = abs(Fraction(float(y)))
    if a > 6:
        mag = 7
    else:
        best = None
        for c, v in enumerate(E2M1_FRACTIONS):
            d = abs(a - v)
            key = (d, c % 2)  # smaller distance first, then the even code
            if best is None or key < best[0]:
                best = (key, c)
        mag = best[1]
    return (8 if math.copysign(1.0, float(y)) < 0 else 0) | mag


def e4m3_exact(s: float) -> int:
    """Nearest E4M3FN byte by exact rational distance, ties to even mantissa, saturating at 448."""
    a = Fraction(float(s))
    if a >= 448:
        return 0x7E
    best = None
    for b, v in E4M3_TABLE:
        key = (abs(a - v), b % 2)
        if best is None or key < best[0]:
            best = (key, b)
    return best[1]


def fp32_neighbourhood(points, ulps=48):
    """All float32 values within +-ulps of each point (and the points themselves)."""
    out = []
    for p in points:
        u = np.float32(p).view(np.uint32).astype(np.int64)
        lo = max(u - ulps, 0)
        out.append(np.arange(lo, u + ulps + 1, dtype=np.int64).astype(np.uint32).view(np.float32))
    return np.concatenate(out)


# --------------------------------------------------------------------- E2M1
def check_e2m1_roundtrip(decode, encode):
    """encode(decode(c)) == c for all 16 codes (brute force over the code space)."""
    codes = np.arange(16)
    vals = np.asarray(decode(codes), dtype=np.float64)
    bad = 0
    for c, v in zip(codes, vals):
        if float(v) != float(E2M1_FRACTIONS[c & 7]) * (-1 if c & 8 else 1):
            bad += 1
    back = np.asarray(encode(vals.astype(np.float32)))
    # -0.0 decodes from code 8 and must come back as 8 (sign bit kept)
    bad += int(np.count_nonzero(back != codes))
    return bad


def check_e2m1_vs_fractions(encode, n_random=20000, seed=1):
    pts = [0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0, 6.5, 7.0, 1e-30, 1e30]
    ys = fp32_neighbourhood(pts)
    rng = np.random.default_rng(seed)
    ys = np.concatenate([ys, rng.uniform(0, 8, n_random).astype(np.float32),
                         (rng.standard_normal(n_random) * 3).astype(np.float32)])
    ys = np.concatenate([ys, -ys, np.array([np.float32(-0.0)])])
    got = np.asarray(encode(ys))
    want = np.array([e2m1_exact(float(y)) for y in ys])
    return int(np.count_nonzero(got != want))


def check_e2m1_dense_sweep(encode, lo_exp=-3, hi_exp=3, stride=1, chunk=1 << 22):
    """Every stride-th float32 in [2^lo_exp, 2^hi_exp): compare against a brute
    force argmin over the grid (float64 distances, exact in this range)."""
    grid = np.array([float(v) for v in E2M1_FRACTIONS])
    start = np.uint32(np.float32(2.0 ** lo_exp).view(np.uint32))
    stop = np.uint32(np.float32(2.0 ** hi_exp).view(np.uint32))
    bad = 0
    for base in range(int(start), int(stop), chunk * stride):
        u = np.arange(base, min(base + chunk * stride, int(stop)), stride, dtype=np.uint64).astype(np.uint32)
        y = u.view(np.float32)
        a = y.astype(np.float64)
        d = np.abs(a[:, None] - grid[None, :])
        dmin = d.min(axis=1, keepdims=True)
        nearest = d == dmin  # one candidate, or two on an exact tie
        idx = np.arange(8)[None, :]
        even_pick = np.where(nearest & (idx % 2 == 0), idx, 99).min(axis=1)
        any_pick = np.where(nearest, idx, 99).min(axis=1)
        best = np.where(even_pick != 99, even_pick, any_pick)
        best = np.where(a > 6.0, 7, best)
        bad += int(np.count_nonzero(np.asarray(encode(y)) != best))
    return bad


# --------------------------------------------------------------------- E4M3
def check_e4m3_decode(decode):
    bad = 0
    for b, v in E4M3_TABLE:
        if float(decode(b)) != float(v) or float(decode(b | 0x80)) != -float(v):
            bad += 1
    if not (math.isnan(float(decode(0x7F))) and math.isnan(float(decode(0xFF)))):
        bad += 1
    return bad


def check_e4m3_roundtrip(decode, encode):
    bytes_ = np.arange(0x7F)
    vals = np.asarray(decode(bytes_), dtype=np.float64).astype(np.float32)
    return int(np.count_nonzero(np.asarray(encode(vals)) != bytes_))


def _e4m3_equivalence_class_inputs():
    """float32 patterns covering every rounding situation of a 3-bit mantissa:
    every exponent that can reach E4M3 (plus a margin), every top-8 mantissa
    pattern, and low bits {0, 1, half, all}."""
    exps = np.arange(127 - 30, 127 + 12, dtype=np.uint32)
    tops = np.arange(256, dtype=np.uint32)
    lows = np.array([0, 1, 0x4000, 0x7FFF], dtype=np.uint32)
    u = (exps[:, None, None] << 23) | (tops[None, :, None] << 15) | lows[None, None, :]
    return u.reshape(-1).view(np.float32)


def check_e4m3_vs_torch(encode, n_random=200000, seed=2):
    """Against torch's float8_e4m3fn cast (round to nearest even) after clamping to 448."""
    import torch

    rng = np.random.default_rng(seed)
    s = np.concatenate([_e4m3_equivalence_class_inputs(), rng.uniform(0, 500, n_random).astype(np.float32),
                        np.exp2(rng.uniform(-14, 9, n_random)).astype(np.float32),
                        np.array([0.0, 448.0, 448.5, 464.0, 1e9, 2.0 ** -9, 2.0 ** -10, 2.0 ** -6], dtype=np.float32)])
    ref = torch.from_numpy(np.minimum(s, np.float32(448.0))).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    return int(np.count_nonzero(np.asarray(encode(s)) != ref))


def check_e4m3_vs_fractions(encode, seed=3):
    pts = [float(v) for _, v in E4M3_TABLE] + [float((E4M3_TABLE[i][1] + E4M3_TABLE[i + 1][1]) / 2) for i in range(126)]
    s = fp32_neighbourhood([p for p in pts if p >= 0], ulps=3)
    s = s[s >= 0]
    rng = np.random.default_rng(seed)
    s = np.concatenate([s, np.exp2(rng.uniform(-12, 9, 3000)).astype(np.float32)])
    got = np.asarray(encode(s))
    want = np.array([e4m3_exact(float(v)) for v in s])
    return int(np.count_nonzero(got != want))


# --------------------------------------------------------------------- quantiser
def load_worked_examples():
    with open(os.path.join(GOLDEN, "hand_worked_examples.json")) as f:
        return json.load(f)["examples"]


def check_worked_examples(quantize):
    bad = 0
    for ex in load_worked_examples():
        g = np.array([int(ex["g_bits"], 16)], dtype=np.uint32).view(np.float32)[0]
        x = np.array([ex["x"]], dtype=np.float32)
        codes, scales, _ = quantize(x, g)
        if bytes(np.asarray(codes, dtype=np.uint8).reshape(-1)).hex() != ex["packed"]:
            bad += 1
        if int(np.asarray(scales).reshape(-1)[0]) != int(ex["scale"], 16):
            bad += 1
    return bad


def check_dynamic_scale_maps_amax_to_top(quantize, seed=4):
    """With the dynamic global scale, the block holding the tensor's largest
    magnitude gets the largest E4M3 scale (448) and that element the largest
    E2M1 code (6): the global scale's purpose in the format."""
    rng = np.random.default_rng(seed)
    bad = 0
    for _ in range(20):
        x = (rng.standard_normal((4, 64)) * rng.uniform(1e-3, 1e3)).astype(np.float32)
        codes, scales, g = quantize(x, None)
        r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
        byte = int(np.asarray(codes)[r, c // 2])
        code = (byte >> 4) if c % 2 else (byte & 0xF)
        if int(np.asarray(scales)[r, c // 16]) != 0x7E or (code & 7) != 7:
            bad += 1
        if np.float32(g) != np.float32(np.float32(2688.0) / np.float32(np.max(np.abs(x)))):
            bad += 1
    return bad


def check_quantize_exact_steps(quantize, n_blocks=3000, seed=5):
    """Block-by-block re-derivation with exact rationals: S = E4M3 of the
    correctly rounded fp32 s_b, codes = E2M1 of the correctly rounded fp32 y.
    Inputs put elements close to E2M1 ties and scales close to E4M3 ties."""
    rng = np.random.default_rng(seed)
    g = np.float32(rng.uniform(50, 500))
    x = rng.standard_normal((n_blocks, 16)).astype(np.float32)
    # push some elements onto the neighbourhood of ties after scaling
    x[::7, 3] = np.float32(0.75) * x[::7, 0]
    x[::11, 5] = -x[::11, 0] * np.float32(2.5 / 6)
    x[::13, :] *= np.float32(1e-6)
    x = x.reshape(-1, 64)
    codes, scales, _ = quantize(x, g)
    codes = np.asarray(codes)
    scales = np.asarray(scales)
    bad = 0
    xb = x.reshape(-1, 16)
    sb = scales.reshape(-1)
    cb = codes.reshape(-1, 8)
    def f32(q):  # exact rational of the correctly rounded float32 of an exact rational
        return Fraction(_round_fraction_to_f32(Fraction(q)))
    for i in range(0, xb.shape[0], 3):
        blk = xb[i]
        a = max(abs(Fraction(float(v))) for v in blk)
        s = f32(f32(a / 6) * Fraction(float(g)))
        S = e4m3_exact(float(s))
        if S != int(sb[i]):
            bad += 1
            continue
        dS = dict(E4M3_TABLE)[S]
        r = Fraction(0) if S == 0 else f32(Fraction(float(g)) / dS)
        for j in range(16):
            y = np.float32(float(f32(Fraction(float(blk[j])) * r)))
            if blk[j] < 0 or (blk[j] == 0 and math.copysign(1, float(blk[j])) < 0):
                y = -abs(y) if y != 0 else np.float32(-0.0)
            want = e2m1_exact(float(y))
            byte = int(cb[i, j // 2])
            got = (byte >> 4) if j % 2 else (byte & 0xF)
            if got != want:
                bad += 1
    return bad


def _round_fraction_to_f32(q: Fraction) -> float:
    """Correctly rounded (nearest even) float32 value of an exact rational, as a float."""
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    # q in [2^e, 2^(e+1)); float32 keeps 24 significant bits (normal range only here)
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    n = q / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(fl * ulp)


def check_block_locality(quantize, seed=6):
    """With a fixed global scale, changing elements of one block changes only
    that block's scale byte and code bytes (outlier damage stays in its block)."""
    rng = np.random.default_rng(seed)
    bad = 0
    for _ in range(30):
        x = rng.standard_normal((3, 96)).astype(np.float32)
        g = np.float32(268.8)
        c0, s0, _ = quantize(x, g)
        r, b = rng.integers(0, 3), rng.integers(0, 6)
        y = x.copy()
        y[r, b * 16 + rng.integers(0, 16)] = np.float32(rng.choice([100.0, -1e3, 1e-7, 0.0]))
        c1, s1, _ = quantize(y, g)
        c0, s0, c1, s1 = map(np.asarray, (c0, s0, c1, s1))
        dc = np.argwhere(c0 != c1)
        ds = np.argwhere(s0 != s1)
        for rr, cc in dc:
            if rr != r or cc // 8 != b:
                bad += 1
        for rr, bb in ds:
            if rr != r or bb != b:
                bad += 1
    return bad


def check_error_bound(quantize, dequant, seed=7):
    """Per element |x - x_hat| <= (1 + 2^-4) * amax_b / 6 (plus fp32 slack)
    whenever the block scale is normal and unsaturated; the bound depends on the
    element's own block amax only."""
    rng = np.random.default_rng(seed)
    bad = 0
    for _ in range(20):
        x = (rng.standard_t(3, (8, 128)) * rng.uniform(0.01, 10)).astype(np.float32)
        x[:, 5] *= 100
        codes, scales, g = quantize(x, None)
        xh = np.asarray(dequant(codes, scales, g))
        amax_b = np.repeat(np.max(np.abs(x.reshape(8, 8, 16)), axis=2), 16, axis=1)
        S = np.repeat(np.asarray(scales).astype(np.int64), 16, axis=1)
        normal = (S >= 0x08) & (S < 0x7E)
        lim = (1 + 2.0 ** -4) * amax_b / 6 * (1 + 1e-6)
        bad += int(np.count_nonzero((np.abs(x - xh) > lim) & normal))
    return bad


def check_max_code_in_normal_blocks(quantize, seed=8):
    """Every block whose scale is a normal E4M3 value has an element at |code| = 6."""
    rng = np.random.default_rng(seed)
    bad = 0
    for _ in range(20):
        x = (rng.standard_normal((16, 64)) * rng.uniform(1e-4, 1e4)).astype(np.float32)
        g = np.float32(rng.uniform(1, 1e4))
        codes, scales, _ = quantize(x, g)
        cod = np.asarray(codes)
        full = np.empty((16, 64), dtype=np.int64)
        full[:, 0::2] = cod & 0xF
        full[:, 1::2] = cod >> 4
        has6 = np.any((full.reshape(16, 4, 16) & 7) == 7, axis=2)
        bad += int(np.count_nonzero((np.asarray(scales) >= 0x08) & ~has6))
    return bad


def check_pow2_equivariance(quantize, seed=9):
    """quantize(2^k x, 2^-k g) is byte-identical to quantize(x, g)."""
    rng = np.random.default_rng(seed)
    bad = 0
    for k in (-6, -3, 1, 4, 9):
        x = rng.standard_normal((4, 64)).astype(np.float32)
        g = np.float32(100.0)
        a = quantize(x, g)
        b = quantize((x * np.float32(2.0 ** k)).astype(np.float32), np.float32(g * np.float32(2.0 ** -k)))
        bad += int(np.count_nonzero(np.asarray(a[0]) != np.asarray(b[0]))) + int(np.count_nonzero(np.asarray(a[1]) != np.asarray(b[1])))
    return bad


def check_sign_symmetry(quantize, seed=10):
    """quantize(-x) flips every code's sign bit and leaves the scales alone."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((4, 64)).astype(np.float32)
    x[0, :16] = 0.0
    a = quantize(x, np.float32(77.0))
    b = quantize(-x, np.float32(77.0))
    return int(np.count_nonzero((np.asarray(a[0]) ^ 0x88) != np.asarray(b[0]))) + int(np.count_nonzero(np.asarray(a[1]) != np.asarray(b[1])))


def check_idempotence(quantize, dequant, seed=11):
    """With a power-of-two global scale, quantising the dequantised tensor
    again gives back the same bytes on every block whose E4M3 scale is a
    normal value.  Such a block holds a code of magnitude 6, so its amax is
    6 dec(S)/g exactly and the scale comes back unchanged, and every element
    already sits on the E2M1 grid (saturated blocks included)."""
    rng = np.random.default_rng(seed)
    bad = 0
    for g in (np.float32(1.0), np.float32(64.0), np.float32(0.125)):
        x = (rng.standard_normal((16, 128)) * rng.uniform(0.01, 50.0, (16, 1))).astype(np.float32)
        x[3, 16:32] = -0.0
        codes, scales, _ = quantize(x, g)
        codes, scales = np.asarray(codes), np.asarray(scales)
        xh = np.asarray(dequant(codes, scales, g), dtype=np.float64).astype(np.float32)
        c2, s2, _ = quantize(xh, g)
        c2, s2 = np.asarray(c2), np.asarray(s2)
        normal = (scales & 0x7F) >= 0x08  # [rows, blocks]
        bad += int(np.count_nonzero(normal & (s2 != scales)))
        same_codes = (c2 == codes).reshape(codes.shape[0], -1, 8).all(axis=2)  # 8 bytes per block
        bad += int(np.count_nonzero(normal & ~same_codes))
    return bad


def check_underflowed_blocks_are_zero(quantize, seed=17):
    """A block whose scale underflows to E4M3 zero encodes every element as a
    signed zero, whatever the element magnitudes are (tiny global scale)."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((4, 64)) * 10).astype(np.float32)
    codes, scales, _ = quantize(x, np.float32(1e-6))
    bad = int(np.count_nonzero(np.asarray(scales) != 0))
    bad += int(np.count_nonzero((np.asarray(codes) & 0x77) != 0))
    return bad
