"""Pins of the CPU oracle against what the pages and the mathematics fix.

The format (E2M1 elements, one E4M3 scale per 16 elements, an FP32 global
scale) is the one described in the news article 'Qwen3.8-27B最激进4bit量化开源，
权重显存暴降2.9倍！', section 02; outlier locality is stated there and in the
MessageDaily paper reading, sections 4.2 (i) and 六; the fused-group repair
is section 03 of the news article.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import nvfp4_oracle as O
from tests import oracle_pins as P


# ------------------------------------------------------------------ element format
def test_e2m1_roundtrip_all_codes():
    assert P.check_e2m1_roundtrip(O.e2m1_decode, O.e2m1_encode) == 0


def test_e2m1_vs_exact_rationals():
    assert P.check_e2m1_vs_fractions(O.e2m1_encode) == 0


def test_e2m1_dense_sweep_all_fp32_in_decision_range():
    # every float32 in [1/8, 8): all 7 decision points and the saturation edge
    assert P.check_e2m1_dense_sweep(O.e2m1_encode, -3, 3, stride=1) == 0


def test_e2m1_dense_sweep_small_and_large():
    assert P.check_e2m1_dense_sweep(O.e2m1_encode, -40, -3, stride=997) == 0
    assert P.check_e2m1_dense_sweep(O.e2m1_encode, 3, 40, stride=997) == 0


def test_e4m3_decode_table():
    assert P.check_e4m3_decode(O.e4m3_decode) == 0
    assert O.e4m3_decode(0x7E) == 448.0 and O.e4m3_decode(0x08) == 2.0 ** -6 and O.e4m3_decode(0x01) == 2.0 ** -9
    finite = [b for b in range(128) if not np.isnan(O.e4m3_decode(b))]
    assert len(finite) == 127


def test_e4m3_roundtrip():
    assert P.check_e4m3_roundtrip(O.e4m3_decode, O.e4m3_encode) == 0


def test_e4m3_vs_torch_float8_cast():
    assert P.check_e4m3_vs_torch(O.e4m3_encode) == 0


def test_e4m3_vs_exact_rationals():
    assert P.check_e4m3_vs_fractions(O.e4m3_encode) == 0


# ------------------------------------------------------------------ quantiser
def test_hand_worked_examples():
    assert P.check_worked_examples(O.quantize_ref) == 0


def test_dynamic_global_scale_maps_tensor_amax_to_top_codes():
    assert P.check_dynamic_scale_maps_amax_to_top(O.quantize_ref) == 0


def test_zero_tensor_dynamic_scale_is_one():
    codes, scales, g = O.quantize_ref(np.zeros((2, 32), np.float32))
    assert g == np.float32(1.0) and not codes.any() and not scales.any()


def test_quantize_matches_exact_step_by_step_derivation():
    assert P.check_quantize_exact_steps(O.quantize_ref) == 0


def test_block_locality_of_outliers():
    assert P.check_block_locality(O.quantize_ref) == 0


def test_error_bound_depends_on_own_block_only():
    assert P.check_error_bound(O.quantize_ref, O.dequant_ref) == 0


def test_outlier_contrast_with_per_tensor_scaling():
    """Block scaling keeps an outlier's damage inside its block; one scale for
    the whole tensor (the contrast the paper reading draws in section 六) lets
    the same outlier wipe out every other element."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((1, 256)).astype(np.float32)
    x[0, 7] = 1000.0
    codes, scales, g = O.quantize_ref(x)
    err_block = np.abs(O.dequant_ref(codes, scales, g) - x)[0, 16:]
    # per-tensor 4-bit: one scale amax/6 for all elements, E2M1 rounding
    step = np.float32(np.max(np.abs(x)) / 6)
    pt = O.e2m1_decode(O.e2m1_encode((x / step).astype(np.float32))) * step
    err_tensor = np.abs(pt - x)[0, 16:]
    assert err_block.max() < 0.5 and err_tensor.mean() > 10 * err_block.mean()
    assert np.all(pt[0, 16:] == 0)  # every non-outlier element is flushed


def test_underflowed_blocks_encode_zeros():
    assert P.check_underflowed_blocks_are_zero(O.quantize_ref) == 0


def test_max_code_present_in_every_normal_block():
    assert P.check_max_code_in_normal_blocks(O.quantize_ref) == 0


def test_power_of_two_equivariance():
    assert P.check_pow2_equivariance(O.quantize_ref) == 0


def test_requantising_the_dequantised_tensor_is_idempotent():
    assert P.check_idempotence(O.quantize_ref, O.dequant_ref) == 0


def test_sign_symmetry():
    assert P.check_sign_symmetry(O.quantize_ref) == 0


def test_negative_zero_and_nibble_order():
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = -0.0
    x[0, 1] = 1.0
    codes, scales, _ = O.quantize_ref(x, np.float32(1.0))
    # element 0 (-0.0) in the low nibble keeps its sign: code 8; element 1 = 1/(1/6)... S = fp32(1/6)
    assert codes[0, 0] & 0xF == 8
    assert codes[0, 0] >> 4 == 7  # the block amax maps to code 6 (0b111)


def test_bits_per_element():
    """4-bit codes plus one 8-bit scale per 16 elements: 4.5 bits per element."""
    x = np.ones((8, 512), np.float32)
    codes, scales, _ = O.quantize_ref(x)
    assert (codes.nbytes + scales.nbytes) * 8 / x.size == 4.5


# ------------------------------------------------------------------ GEMM
def _rand_q(rng, rows, cols):
    codes = rng.integers(0, 256, (rows, cols // 2)).astype(np.uint8)
    scales = rng.integers(0, 0x7F, (rows, cols // 16)).astype(np.uint8)
    return codes, scales


def test_gemm_vs_exact_rationals():
    rng = np.random.default_rng(12)
    M, N, K = 3, 4, 48
    ac, asc = _rand_q(rng, M, K)
    wc, wsc = _rand_q(rng, N, K)
    ga, gw = np.float32(3.7), np.float32(123.25)
    C, B = O.gemm_ref(ac, asc, ga, wc, wsc, gw)
    for m in range(M):
        for n in range(N):
            exact = sum(P_exact(ac, asc, ga, m, k) * P_exact(wc, wsc, gw, n, k) for k in range(K))
            absum = sum(abs(P_exact(ac, asc, ga, m, k) * P_exact(wc, wsc, gw, n, k)) for k in range(K))
            assert abs(Fraction(float(C[m, n])) - exact) <= Fraction(1, 2 ** 48) * max(absum, Fraction(1, 2 ** 200))
            assert abs(Fraction(float(B[m, n])) - absum) <= Fraction(1, 2 ** 48) * max(absum, Fraction(1, 2 ** 200))


def P_exact(codes, scales, g, r, k):
    """Exact dequantised value, written from the format definition independently of the oracle."""
    byte = int(codes[r, k // 2])
    c = (byte >> 4) if k % 2 else (byte & 0xF)
    v = P.E2M1_FRACTIONS[c & 7] * (-1 if c & 8 else 1)
    s = dict(P.E4M3_TABLE)[int(scales[r, k // 16])]
    return v * s / Fraction(float(g))


def test_gemm_closed_form_all_ones():
    # all codes 0x2 (value 1), scale 0x38 (1.0), g = 1  ->  C = K everywhere
    K = 256
    a = np.full((5, K // 2), 0x22, np.uint8)
    s = np.full((5, K // 16), 0x38, np.uint8)
    C, B = O.gemm_ref(a, s, np.float32(1), a[:3], s[:3], np.float32(1))
    assert np.all(C == K) and np.all(B == K)


def test_gemm_one_hot_block():
    K = 64
    a = np.zeros((2, K // 2), np.uint8)
    w = np.zeros((3, K // 2), np.uint8)
    sa = np.full((2, K // 16), 0x38, np.uint8)
    sw = np.full((3, K // 16), 0x38, np.uint8)
    a[1, 20] = 0x07  # element 40 of row 1 = 6 (low nibble)
    sa[1, 2] = 0x48  # block 2 scale = 2^(9-7) = 4
    w[2, 20] = 0x0D  # element 40 of row 2 = -3
    sw[2, 2] = 0x30  # 0.5
    C, _ = O.gemm_ref(a, sa, np.float32(2), w, sw, np.float32(4))
    expect = np.zeros((2, 3))
    expect[1, 2] = (6 * 4 / 2) * (-3 * 0.5 / 4)
    assert np.array_equal(C, expect)


# ------------------------------------------------------------------ fused-group repair
def _modules(rng, rows, K, amaxes):
    out = []
    for r, am in zip(rows, amaxes):
        w = rng.standard_normal((r, K)).astype(np.float32)
        w *= np.float32(am / np.max(np.abs(w)))
        out.append(O.quantize_ref(w))
    return out


def test_fuse_owner_module_unchanged_and_gstar_is_min():
    rng = np.random.default_rng(13)
    qs = _modules(rng, [8, 6, 2, 2], 64, [0.21, 0.17, 0.05, 0.9])
    scales = np.concatenate([q[1] for q in qs])
    gs = [q[2] for q in qs]
    new, gstar, _ = O.fuse_rescale_ref(scales, [8, 6, 2, 2], gs)
    assert gstar == min(gs)
    i = int(np.argmin(gs))
    r0 = sum([8, 6, 2, 2][:i])
    n_i = [8, 6, 2, 2][i]
    assert np.array_equal(new[r0:r0 + n_i], scales[r0:r0 + n_i])
    # no folded scale ever exceeds the largest E4M3 value (rho <= 1)
    assert new.max() <= 0x7E


def test_fuse_power_of_two_ratios_are_exact():
    rng = np.random.default_rng(14)
    K = 128
    w = [rng.standard_normal((4, K)).astype(np.float32) for _ in range(3)]
    q0 = O.quantize_ref(w[0], np.float32(64.0))
    q1 = O.quantize_ref(w[1], np.float32(256.0))
    q2 = O.quantize_ref(w[2], np.float32(1024.0))
    scales = np.concatenate([q0[1], q1[1], q2[1]])
    new, gstar, lossy = O.fuse_rescale_ref(scales, [4, 4, 4], [q0[2], q1[2], q2[2]])
    assert gstar == np.float32(64.0)
    before = np.concatenate([O.dequant_ref(q[0], q[1], q[2]) for q in (q0, q1, q2)])
    after = O.dequant_ref(np.concatenate([q0[0], q1[0], q2[0]]), new, gstar)
    normal = np.repeat(new >= 0x08, 16, axis=1)
    assert np.array_equal(after[normal], before[normal])
    # the count of changed dequantisation factors, from exact rationals: with
    # power-of-two ratios every folded block here stays normal, so none changes
    assert lossy == P.count_changed_dequant_factors(scales, new, [4, 4, 4], [q0[2], q1[2], q2[2]], gstar) == 0


def test_fuse_general_ratio_within_one_e4m3_half_ulp():
    rng = np.random.default_rng(15)
    rows = [8, 6, 2, 2]
    qs = _modules(rng, rows, 128, [0.21, 0.17, 0.05, 0.9])
    scales = np.concatenate([q[1] for q in qs])
    codes = np.concatenate([q[0] for q in qs])
    new, gstar, lossy = O.fuse_rescale_ref(scales, rows, [q[2] for q in qs])
    before = np.concatenate([O.dequant_ref(q[0], q[1], q[2]) for q in qs])
    after = O.dequant_ref(codes, new, gstar)
    normal = np.repeat(new >= 0x08, 16, axis=1)
    rel = np.abs(after - before)[normal] <= 2.0 ** -4 * np.abs(before[normal]) * (1 + 1e-6)
    assert rel.all()
    exact = P.count_changed_dequant_factors(scales, new, rows, [q[2] for q in qs], gstar)
    assert lossy == exact and exact > 0
    # the bug: one shared scale without folding distorts by g_i / g* (3x-18x here)
    buggy = O.dequant_ref(codes, scales, gstar)
    ratios = [float(q[2] / gstar) for q in qs]
    assert max(ratios) > 3
    r0 = 0
    for q, n_i in zip(qs, rows):
        blk_b, blk_t = buggy[r0:r0 + n_i], before[r0:r0 + n_i]
        nz = blk_t != 0
        np.testing.assert_allclose(blk_b[nz] / blk_t[nz], float(q[2] / gstar), rtol=1e-6)
        r0 += n_i


def test_fused_gemm_equals_per_module_gemms_within_fold_bound():
    rng = np.random.default_rng(16)
    rows = [16, 8, 3]
    K = 64
    qs = _modules(rng, rows, K, [0.3, 0.08, 1.5])
    a = rng.standard_normal((5, K)).astype(np.float32)
    ac, asc, ga = O.quantize_ref(a)
    new, gstar, _ = O.fuse_rescale_ref(np.concatenate([q[1] for q in qs]), rows, [q[2] for q in qs])
    Cf, Bf = O.gemm_ref(ac, asc, ga, np.concatenate([q[0] for q in qs]), new, gstar)
    Cs = np.concatenate([O.gemm_ref(ac, asc, ga, q[0], q[1], q[2])[0] for q in qs], axis=1)
    assert np.all(np.abs(Cf - Cs) <= 2.0 ** -4 * Bf * (1 + 1e-6) + 1e-300)


def test_fuse_rejects_bad_global_scales():
    with pytest.raises(ValueError):
        O.fuse_rescale_ref(np.zeros((2, 1), np.uint8), [1, 1], [1.0, 0.0])
    with pytest.raises(ValueError):
        O.fuse_rescale_ref(np.zeros((2, 1), np.uint8), [1, 1], [1.0, float("nan")])


# ---- calibration observer (static activation global scale)

def test_calibration_hand_example():
    # largest magnitude 7 over three batches: g = 2688 / 7 = 384 exactly
    amax, g = O.calibrate_ref([np.array([[1.0, -3.0]]), np.array([[2.5, 0.5]]), np.array([[-7.0, 0.0]])])
    assert amax == np.float32(7.0) and g == np.float32(384.0)


def test_calibration_all_zero_and_empty_give_unit_scale():
    assert O.calibrate_ref([np.zeros((2, 16))])[1] == np.float32(1.0)
    assert O.calibrate_ref([])[1] == np.float32(1.0)


def test_calibration_is_order_free_and_equals_the_concatenation():
    rng = np.random.default_rng(11)
    batches = [rng.standard_t(3, size=(int(rng.integers(1, 9)), 32)).astype(np.float32) for _ in range(7)]
    _, g = O.calibrate_ref(batches)
    assert g == O.calibrate_ref(batches[::-1])[1]
    assert g == O.global_scale(np.concatenate(batches))
    # and it is the dynamic scale the quantiser would pick for the whole set
    assert g == np.float32(2688.0) / np.float32(np.abs(np.concatenate(batches)).max())


# ---- static FP8 KV-cache quantisation

def test_kv_fp8_hand_values():
    # s = 1: exact values, the largest finite value, saturation, signed zero,
    # subnormal ties (2^-10 -> 0, 3*2^-10 -> the even neighbour 2*2^-9) and a
    # normal tie (17 lies halfway between 16 = 0x58 and 18 = 0x59 -> 16)
    x = np.array([1.0, -1.5, 448.0, 500.0, -1e6, -0.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 17.0],
                 dtype=np.float32)
    q = O.kv_quantize_ref(x, np.float32(1.0))
    assert list(q) == [0x38, 0xBC, 0x7E, 0x7E, 0xFE, 0x80, 0x01, 0x00, 0x02, 0x58]


def test_kv_fp8_matches_torch_cast_in_range():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch has no float8_e4m3fn")
    rng = np.random.default_rng(41)
    x = (rng.standard_t(3, 200000) * 20).astype(np.float32)
    s = O.kv_scale_ref(np.abs(x).max())
    q = O.kv_quantize_ref(x, s)
    y = (x * s).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)  # every |y| <= 448 here: torch's cast is an independent encoder


def test_kv_fp8_scale_maps_amax_to_448():
    assert O.kv_scale_ref(np.float32(7.0)) == np.float32(64.0)
    assert O.kv_scale_ref(np.float32(0.0)) == np.float32(1.0)
    x = np.array([-7.0, 3.0], dtype=np.float32)
    assert O.kv_quantize_ref(x, O.kv_scale_ref(7.0))[0] == 0xFE  # -448
