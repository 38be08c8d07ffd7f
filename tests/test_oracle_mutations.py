"""Plant plausible mistakes in a copy of the oracle and check that the pins
catch every one of them.  The copy is built from the oracle's source text with
one textual edit, executed into a fresh namespace; the real oracle is never
modified.  If a mutation's anchor text is no longer in the oracle, the test
fails, so the list stays in step with the code."""
import inspect
import types

import numpy as np
import pytest

from oracle import nvfp4_oracle as O
from tests import oracle_pins as P

SRC = inspect.getsource(O)


def mutant(old, new):
    assert old in SRC, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def quant_pins(m):
    try:
        return _quant_pins(m)
    except Exception:  # a mutant that crashes is caught too
        return 1


def _quant_pins(m):
    return (P.check_worked_examples(m.quantize_ref) + P.check_quantize_exact_steps(m.quantize_ref, n_blocks=600)
            + P.check_dynamic_scale_maps_amax_to_top(m.quantize_ref) + P.check_sign_symmetry(m.quantize_ref)
            + P.check_e2m1_roundtrip(m.e2m1_decode, m.e2m1_encode) + P.check_e4m3_roundtrip(m.e4m3_decode, m.e4m3_encode)
            + P.check_e2m1_vs_fractions(m.e2m1_encode, n_random=2000) + P.check_e4m3_vs_fractions(m.e4m3_encode)
            + P.check_underflowed_blocks_are_zero(m.quantize_ref) + P.check_idempotence(m.quantize_ref, m.dequant_ref))


QUANT_MUTANTS = {
    "e2m1 ties away from zero": ("(d_hi == d_lo) & (hi_code % 2 == 0)", "(d_hi == d_lo)"),
    "e2m1 drops the sign of zero": ("sign = np.signbit(y).astype(np.int64)", "sign = (y < 0).astype(np.int64)"),
    "e2m1 no saturation": ("mag_code = np.full(a.shape, 7, dtype=np.int64)", "mag_code = np.full(a.shape, 0, dtype=np.int64)"),
    "e2m1 wrong subnormal value": ("np.where(e == 0, m * 0.5,", "np.where(e == 0, m * 0.25,"),
    "e4m3 truncates": ("q_norm = np.round(sig)", "q_norm = np.floor(sig)"),
    "e4m3 wrong bias": ("exp_unb + 7", "exp_unb + 8"),
    "e4m3 subnormal step": ("q_sub = np.round(np.ldexp(v, 9))", "q_sub = np.round(np.ldexp(v, 8))"),
    "block amax/4 instead of /6": ("s_b = (amax_b / np.float32(6.0))", "s_b = (amax_b / np.float32(4.0))"),
    "scale not applied to elements": ("y = (xb * r_b[:, :, None])", "y = (xb * g)"),
    "nibbles swapped": ("packed = (codes[:, 0::2] | (codes[:, 1::2] << 4))", "packed = (codes[:, 1::2] | (codes[:, 0::2] << 4))"),
    "global scale 448/amax": ("GLOBAL_SCALE_NUMERATOR / amax", "np.float32(448.0) / amax"),
    "element divided by the reciprocal": ("y = (xb * r_b[:, :, None])", "y = (xb / np.maximum(r_b[:, :, None], np.float32(1e-30)))"),
    "zero block not flushed": ("np.where(S_b == 0, np.float32(0.0),", "np.where(S_b == 0, np.float32(1.0),"),
}


@pytest.mark.parametrize("name", sorted(QUANT_MUTANTS))
def test_quantiser_mutants_are_caught(name):
    m = mutant(*QUANT_MUTANTS[name])
    assert quant_pins(m) > 0, f"no pin caught: {name}"


def test_unmutated_copy_passes_the_same_pins():
    m = mutant("BLOCK = 16", "BLOCK = 16")
    assert quant_pins(m) == 0


def _fuse_pins(m):
    """The fuse-rescale pins from test_oracle, returning a violation count."""
    rng = np.random.default_rng(15)
    rows = [8, 6, 2, 2]
    qs = []
    for r, am in zip(rows, [0.21, 0.17, 0.05, 0.9]):
        w = rng.standard_normal((r, 128)).astype(np.float32)
        w *= np.float32(am / np.max(np.abs(w)))
        qs.append(O.quantize_ref(w))
    scales = np.concatenate([q[1] for q in qs])
    codes = np.concatenate([q[0] for q in qs])
    new, gstar, lossy = m.fuse_rescale_ref(scales, rows, [q[2] for q in qs])
    before = np.concatenate([O.dequant_ref(q[0], q[1], q[2]) for q in qs])
    after = O.dequant_ref(codes, new, gstar)
    big = np.repeat(new >= 0x08, 16, axis=1)
    bad = int(np.count_nonzero(np.abs(after - before)[big] > 2.0 ** -4 * np.abs(before[big]) * (1 + 1e-6)))
    # the module that owns g* keeps its bytes
    i = int(np.argmin([q[2] for q in qs]))
    r0 = sum(rows[:i])
    bad += int(np.count_nonzero(new[r0:r0 + rows[i]] != scales[r0:r0 + rows[i]]))
    # the lossy-block count against exact rationals
    bad += abs(lossy - P.count_changed_dequant_factors(scales, new, rows, [q[2] for q in qs], gstar))
    # power-of-two ratios: the folded bytes change, the dequantisation factors do not
    w = [rng.standard_normal((4, 128)).astype(np.float32) for _ in range(3)]
    q2 = [O.quantize_ref(wi, np.float32(g)) for wi, g in zip(w, (64.0, 256.0, 1024.0))]
    s2 = np.concatenate([q[1] for q in q2])
    new2, g2, lossy2 = m.fuse_rescale_ref(s2, [4, 4, 4], [q[2] for q in q2])
    bad += int(np.count_nonzero(new2 != s2) == 0)  # the non-owner modules' bytes must change
    bad += abs(lossy2 - P.count_changed_dequant_factors(s2, new2, [4, 4, 4], [q[2] for q in q2], g2))
    return bad


FUSE_MUTANTS = {
    "shared scale is the max encode scale": ("g_star = min(gs)", "g_star = max(gs)"),
    "ratio inverted": ("rho = np.float32(g_star / g_i)", "rho = np.float32(g_i / g_star)"),
    "ratio not folded": ("folded = (e4m3_decode(blk).astype(np.float32) * rho)", "folded = (e4m3_decode(blk).astype(np.float32))"),
    "lossy count counts changed bytes": (
        "lossy += int(np.count_nonzero(e4m3_decode(new) * np.float64(g_i) != e4m3_decode(blk) * np.float64(g_star)))",
        "lossy += int(np.count_nonzero(new != blk))"),
    "lossy count compares against the module's own scale": (
        "lossy += int(np.count_nonzero(e4m3_decode(new) * np.float64(g_i) != e4m3_decode(blk) * np.float64(g_star)))",
        "lossy += int(np.count_nonzero(e4m3_decode(new) * np.float64(g_i) != e4m3_decode(blk) * np.float64(g_i)))"),
}


@pytest.mark.parametrize("name", sorted(FUSE_MUTANTS))
def test_fuse_mutants_are_caught(name):
    assert _fuse_pins(O) == 0
    assert _fuse_pins(mutant(*FUSE_MUTANTS[name])) > 0


GEMM_MUTANTS = {
    "weights not transposed": ("return a @ w.T, np.abs(a) @ np.abs(w).T", "return a @ w[:, :a.shape[1]].T[::-1], np.abs(a) @ np.abs(w).T"),
    "scales dropped": ("return (vals * sc).reshape(rows, cols)", "return (vals).reshape(rows, cols)"),
    "global scale multiplied": ("/ np.float64(np.float32(g))", "* np.float64(np.float32(g))"),
}


@pytest.mark.parametrize("name", sorted(GEMM_MUTANTS))
def test_gemm_mutants_are_caught(name):
    from tests.test_oracle import P_exact

    rng = np.random.default_rng(12)
    M, N, K = 4, 4, 32
    ac = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    asc = rng.integers(0x20, 0x50, (M, K // 16)).astype(np.uint8)
    wc = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    wsc = rng.integers(0x20, 0x50, (N, K // 16)).astype(np.uint8)
    m = mutant(*GEMM_MUTANTS[name])
    C, _ = m.gemm_ref(ac, asc, np.float32(3.5), wc, wsc, np.float32(7.25))
    exact = np.array([[float(sum(P_exact(ac, asc, np.float32(3.5), i, k) * P_exact(wc, wsc, np.float32(7.25), j, k) for k in range(K)))
                       for j in range(N)] for i in range(M)])
    assert not np.allclose(C, exact, rtol=1e-12, atol=0)
