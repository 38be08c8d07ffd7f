"""CPU oracle for the NVFP4 W4A4 linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant generator with the HIP library, and it never imports that package.

What it computes, and where the pages define it
------------------------------------------------
Pages: arXiv 2609.04098 "Why Gated DeltaNet Survives 4-Bit Quantization:
NVFP4 W4A4 for the Recurrent Half of a Hybrid 27B LLM" as reported by

* [NEWS]  the 智猩猩 article "Qwen3.8-27B最激进4bit量化开源，权重显存暴降2.9倍！",
  section 02 (NVFP4 量化格式) and section 03 (Minima 模型构建);
* [READ]  the MessageDaily paper reading of the same paper, section 一
  (论文背景), section 四 4.1/4.2 and section 六;
* [ABS]   the paper's English abstract (arxivdaily listing).

The format ([NEWS] §02, [READ] §一): values are stored as 4-bit E2M1; every 16
consecutive elements share one E4M3 block scale; each tensor additionally
carries one FP32 global scale.  W4A4 means both the weights and the
activations are quantised this way, so the product is a 4-bit x 4-bit GEMM.
The fused-module repair ([NEWS] §03, [ABS]): modules calibrated one by one are
served as one GEMM; all tensors of a fused group are brought to one global
scale and the ratio is folded into their E4M3 block scales (checkpoint side).

Readings where the pages leave a step open (each is also listed in the
design notes):

* global scale: the stored value is the ENCODE scale g; a tensor whose
  largest magnitude is amax gets g = fp32(2688 / amax) (2688 = 448 * 6, the
  largest E4M3 scale times the largest E2M1 value), and g = 1 for an all-zero
  tensor.  Dequantisation divides by g.
* blocks run along the reduction axis K (16 contiguous elements of a row).
* block scale s_b = fp32(fp32(amax_b / 6) * g), encoded to E4M3 (OCP "FN"
  flavour: bias 7, max 448, no infinities) with round-to-nearest-even and
  saturation to 448.
* element code: y = fp32(x * r_b) with r_b = fp32(g / dec(S_b)) (r_b = 0 when
  S_b encodes 0), then E2M1 round-to-nearest-even (ties to the even code),
  saturating at 6, with the sign bit taken from y (so -0.0 and negatives that
  round to 0 give code 0x8).
* packing: element 2j in the low nibble of byte j; scales row-major.
* fused group: g* = min_i g_i (the largest DEcode scale, so no folded scale
  can exceed 448); rho_i = fp32(g* / g_i); S' = E4M3(fp32(dec(S) * rho_i));
  codes are left unchanged.
* GEMM: C = A_hat @ W_hat^T with both operands dequantised exactly and the
  matmul in float64.

Every function below is vectorised numpy written for clarity, not speed.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

BLOCK = 16  # elements per block scale ([NEWS] §02: one E4M3 scale per 16 elements)
E2M1_MAX = 6.0  # largest E2M1 magnitude
E4M3_MAX = 448.0  # largest finite OCP E4M3FN value
GLOBAL_SCALE_NUMERATOR = np.float32(E4M3_MAX * E2M1_MAX)  # 2688


# ---------------------------------------------------------------------------
# E2M1: 1 sign bit, 2 exponent bits, 1 mantissa bit, exponent bias 1.
# ---------------------------------------------------------------------------
def e2m1_decode(code):
    """Value of 4-bit E2M1 codes ([NEWS] §02 names E2M1 as the element format).

    Bit layout s|e1 e0|m with bias 1: e = 0 is subnormal (m * 2^-1), otherwise
    2^(e-1) * (1 + m/2).  Returns float64.
    """
    code = np.asarray(code, dtype=np.int64)
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m * 0.5, (e - 1).astype(np.int32)))
    return np.where(s == 1, -mag, mag)


def _e2m1_grid():
    """The 8 non-negative E2M1 values, in code order (from e2m1_decode)."""
    return [float(v) for v in e2m1_decode(np.arange(8))]


def e2m1_encode(y):
    """Round float32 values to E2M1 codes: nearest grid value, ties to the even
    code, magnitudes beyond 6 saturate to 6, sign bit from signbit(y).

    Implemented literally: find the two grid neighbours lo <= |y| <= hi and keep
    the nearer one (distances in float64, which is exact for |y| <= 6 in the
    region where a tie is possible); on a tie keep the one whose code is even.
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)
    grid = _e2m1_grid()
    mag_code = np.full(a.shape, 7, dtype=np.int64)  # |y| > 6 saturates to 6 (code 7)
    assigned = np.zeros(a.shape, dtype=bool)
    for lo_code in range(7):
        hi_code = lo_code + 1
        lo, hi = grid[lo_code], grid[hi_code]
        inside = (a >= lo) & (a <= hi) & ~assigned
        d_lo = a - lo
        d_hi = hi - a
        pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi_code % 2 == 0))
        mag_code = np.where(inside, np.where(pick_hi, hi_code, lo_code), mag_code)
        assigned |= inside
    sign = np.signbit(y).astype(np.int64)
    return (sign << 3) | mag_code


# ---------------------------------------------------------------------------
# E4M3 (OCP FN flavour): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits.
# ---------------------------------------------------------------------------
def e4m3_decode(byte):
    """Value of E4M3FN bytes as float64 ([NEWS] §02: block scales are E4M3).

    e = 0: subnormal m * 2^-9; else 2^(e-7) * (1 + m/8).  0x7F / 0xFF are NaN
    (never produced by the quantiser).
    """
    byte = np.asarray(byte, dtype=np.int64)
    s = (byte >> 7) & 1
    e = (byte >> 3) & 15
    m = byte & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32)))
    mag = np.where((byte & 0x7F) == 0x7F, np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e4m3_encode(s):
    """Encode non-negative float32 block scales to E4M3FN bytes, round to
    nearest even, saturating to 448 (0x7E).

    Written from the format definition: split |s| into exponent and
    significand with frexp (exact), quantise the significand to 3 fraction
    bits (normal range) or to multiples of 2^-9 (subnormal range) with
    round-half-even, then carry and saturate.
    """
    s = np.asarray(s, dtype=np.float32).astype(np.float64)
    if np.any(s < 0) or np.any(np.isnan(s)):
        raise ValueError("block scales are non-negative")
    out = np.zeros(s.shape, dtype=np.int64)
    sat = s >= E4M3_MAX
    out[sat] = 0x7E
    rest = ~sat & (s > 0)
    v = s[rest]
    mant, ex = np.frexp(v)  # v = mant * 2^ex, mant in [0.5, 1)
    exp_unb = ex - 1  # v = (2*mant) * 2^exp_unb, 2*mant in [1, 2)
    normal = exp_unb >= -6
    # normal: significand 1.f -> f * 8 rounded half-even
    sig = np.where(normal, (2.0 * mant - 1.0) * 8.0, 0.0)
    q_norm = np.round(sig)  # numpy rounds half to even; sig is exact in float64
    e_field = np.where(normal, exp_unb + 7, 0)
    carry = q_norm == 8
    e_field = np.where(carry, e_field + 1, e_field)
    q_norm = np.where(carry, 0, q_norm)
    # subnormal: v / 2^-9 rounded half-even (8 becomes the smallest normal 0x08)
    q_sub = np.round(np.ldexp(v, 9))
    code_norm = (e_field.astype(np.int64) << 3) | q_norm.astype(np.int64)
    code_sub = q_sub.astype(np.int64)  # 0..8; 8 == 0x08 == 2^-6
    code = np.where(normal, code_norm, code_sub)
    code = np.minimum(code, 0x7E)  # values just below 448 never round past it
    out[rest] = code
    return out


# ---------------------------------------------------------------------------
# Quantiser ([NEWS] §02; readings in the module docstring)
# ---------------------------------------------------------------------------
def global_scale(x):
    """Dynamic encode global scale g = fp32(2688 / amax(x)); 1.0 for amax = 0."""
    amax = np.float32(np.max(np.abs(np.asarray(x, dtype=np.float32)))) if np.size(x) else np.float32(0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(GLOBAL_SCALE_NUMERATOR / amax)


def calibrate_ref(batches):
    """Static activation global scale from a calibration set: the encode scale
    of everything the observer saw, g = fp32(2688 / max_i max|batch_i|), 1.0
    when every value is zero (the paper reading, section 四 4.1, and the news
    article, section 03: activations are calibrated once, on 128 samples of
    32K tokens).  The largest magnitude is folded batch by batch, as the
    observer does; max is exact, so the fold equals the maximum over the
    concatenation."""
    amax = np.float32(0.0)
    for b in batches:
        b = np.asarray(b, dtype=np.float32)
        if b.size:
            amax = max(amax, np.float32(np.max(np.abs(b))))
    if amax == 0:
        return amax, np.float32(1.0)
    return amax, np.float32(GLOBAL_SCALE_NUMERATOR / amax)


def kv_scale_ref(amax):
    """Encode scale of a static FP8 KV cache: fp32(448 / amax), 1.0 for amax = 0
    (the news article, section 03: statically calibrated FP8 KV-cache scales;
    448 is the largest finite E4M3 value)."""
    amax = np.float32(amax)
    return np.float32(1.0) if amax == 0 else np.float32(np.float32(448.0) / amax)


def kv_quantize_ref(x, s):
    """E4M3FN bytes of y = fp32(x * s): sign bit from y, magnitude rounded to
    nearest even and saturated at 448 by the same encoder as the block scales."""
    x = np.asarray(x, dtype=np.float32)
    y = (x * np.float32(s)).astype(np.float32)
    mag = e4m3_encode(np.abs(y))
    return (mag | (np.signbit(y).astype(np.int64) << 7)).astype(np.uint8)


def quantize_ref(x, g=None):
    """NVFP4 quantisation of a [rows, cols] array (cols % 16 == 0).

    ``x`` holds float32 values (bf16/fp16 inputs are first widened exactly);
    ``g`` is the encode global scale (float32) or None for the dynamic one.
    Returns (codes uint8 [rows, cols/2], scales uint8 [rows, cols/16], g).
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % BLOCK:
        raise ValueError("expected [rows, cols] with cols a multiple of 16")
    g = global_scale(x) if g is None else np.float32(g)
    rows, cols = x.shape
    xb = x.reshape(rows, cols // BLOCK, BLOCK)
    amax_b = np.max(np.abs(xb), axis=2)  # exact
    s_b = (amax_b / np.float32(6.0)).astype(np.float32) * g  # two IEEE float32 roundings
    s_b = s_b.astype(np.float32)
    S_b = e4m3_encode(s_b)
    dec_S = e4m3_decode(S_b).astype(np.float32)  # exact
    with np.errstate(divide="ignore", invalid="ignore"):
        r_b = np.where(S_b == 0, np.float32(0.0), (g / dec_S).astype(np.float32)).astype(np.float32)
    y = (xb * r_b[:, :, None]).astype(np.float32)
    codes = e2m1_encode(y).reshape(rows, cols)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, S_b.astype(np.uint8), np.float32(g)


def unpack_codes(packed):
    """[rows, cols/2] bytes -> [rows, cols] 4-bit codes (element 2j = low nibble)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.int64)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def dequant_ref(packed, scales, g):
    """x_hat = e2m1(code) * dec(S_b) / g in float64 (exact up to the division)."""
    codes = unpack_codes(packed)
    rows, cols = codes.shape
    vals = e2m1_decode(codes).reshape(rows, cols // BLOCK, BLOCK)
    sc = e4m3_decode(np.asarray(scales)).reshape(rows, cols // BLOCK, 1)
    return (vals * sc).reshape(rows, cols) / np.float64(np.float32(g))


# ---------------------------------------------------------------------------
# Fused-group repair ([NEWS] §03; [ABS])
# ---------------------------------------------------------------------------
def fuse_rescale_ref(scales, module_rows, module_gscales):
    """Unify the global scales of a fused group and fold the ratios into the
    E4M3 block scales.

    ``scales``: uint8 [sum(module_rows), K/16], the modules' block scales
    stacked in module order; ``module_gscales``: each module's encode scale.
    Returns (new_scales, g_star, lossy_blocks) where lossy_blocks counts the
    blocks whose dequantisation factor dec(S')/g* differs from dec(S)/g_i.
    """
    scales = np.asarray(scales, dtype=np.uint8)
    gs = [np.float32(v) for v in module_gscales]
    if len(gs) != len(module_rows) or sum(module_rows) != scales.shape[0]:
        raise ValueError("module_rows / module_gscales do not match scales")
    if any(not (math.isfinite(float(v)) and v > 0) for v in gs):
        raise ValueError("global scales must be finite and > 0")
    g_star = min(gs)
    out = scales.copy()
    lossy = 0
    r0 = 0
    for n_i, g_i in zip(module_rows, gs):
        blk = scales[r0:r0 + n_i]
        rho = np.float32(g_star / g_i)
        folded = (e4m3_decode(blk).astype(np.float32) * rho).astype(np.float32)
        new = e4m3_encode(folded).astype(np.uint8)
        out[r0:r0 + n_i] = new
        # exact comparison of dec(S')/g* and dec(S)/g_i (cross-multiplied in float64:
        # 4-bit by 24-bit significands, so both products are exact)
        lossy += int(np.count_nonzero(e4m3_decode(new) * np.float64(g_i) != e4m3_decode(blk) * np.float64(g_star)))
        r0 += n_i
    return out, np.float32(g_star), lossy


# ---------------------------------------------------------------------------
# GEMM on the encoded operands
# ---------------------------------------------------------------------------
def gemm_ref(a_codes, a_scales, g_a, w_codes, w_scales, g_w):
    """C = A_hat @ W_hat^T in float64, plus the tolerance basis |A_hat| @ |W_hat|^T.

    Both operands are dequantised exactly (dequant_ref) and multiplied with a
    float64 matmul; the second result is the per-element sum of |a_k * w_k|.
    """
    a = dequant_ref(a_codes, a_scales, g_a)
    w = dequant_ref(w_codes, w_scales, g_w)
    return a @ w.T, np.abs(a) @ np.abs(w).T


# ---------------------------------------------------------------------------
# Exact helpers for self-tests (rational arithmetic, no rounding at all)
# ---------------------------------------------------------------------------
def exact_value_fraction(packed, scales, g, row, col):
    """Dequantised element as an exact Fraction: e2m1 * dec(S) / g."""
    byte = int(np.asarray(packed)[row, col // 2])
    code = (byte >> 4) if (col % 2) else (byte & 0xF)
    return Fraction(float(e2m1_decode(code))) * Fraction(float(e4m3_decode(int(np.asarray(scales)[row, col // BLOCK])))) / Fraction(float(np.float32(g)))
