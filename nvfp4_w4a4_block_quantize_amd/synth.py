"""Seeded synthetic inputs for the NVFP4 W4A4 linear layer workloads.

This module only draws random numbers and rounds them to the input dtype
(bf16 / fp32).  It holds none of the quantisation or GEMM arithmetic, so both
the HIP path and the CPU oracle can be fed from it.

The shapes follow the hybrid 27B model the pages quantise (hidden size 5120,
GDN input projections qkv 8192 + z 6144 + a 48 + b 48, MLP intermediate
17408, attention q/k/v 14336 and o_proj 6144); the pages' own workloads are
8K- and 32K-token prompts, for which these seeded tensors stand in.  No
dataset, checkpoint or trained weight is used.

Every tensor is drawn from ``numpy.random.default_rng([seed, config_id,
tensor_id])``; values are drawn in float32, outliers are applied in float32,
and the result is rounded to bf16 (round to nearest even) unless the config
keeps float32.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

CONFIG_IDS = {"tiny": 0, "gdn": 1, "mlp": 2, "decode": 3, "long": 4}

HIDDEN = 5120
GDN_MODULES = (("qkv", 8192), ("z", 6144), ("a", 48), ("b", 48))
MLP_INTER = 17408
ATTN_QKV = 14336
ATTN_O_IN = 6144


def rng_for(seed: int, config: str, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([seed, CONFIG_IDS[config], tensor_id])


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest-even bf16, returned as float32 holding the bf16 value."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    return (r.astype(np.uint32) << 16).view(np.float32).reshape(x.shape)


def bf16_bits(x_bf16_valued: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are exactly bf16 (uint16 array)."""
    return (np.ascontiguousarray(x_bf16_valued, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _outlier_columns(rng: np.random.Generator, cols: int, fraction: float) -> np.ndarray:
    n = max(1, int(round(fraction * cols)))
    return np.sort(rng.choice(cols, size=n, replace=False))


def activations(seed, config, tensor_id, rows, cols, dist="normal", outlier_fraction=0.001,
                outlier_scale=100.0, bf16=True, outlier_cols=None):
    """[rows, cols] activations with a few outlier channels (whole columns scaled)."""
    rng = rng_for(seed, config, tensor_id)
    if dist == "normal":
        x = rng.standard_normal((rows, cols), dtype=np.float32)
    elif dist == "t3":
        x = rng.standard_t(3, size=(rows, cols)).astype(np.float32)
    else:
        raise ValueError(dist)
    if outlier_fraction > 0:
        if outlier_cols is None:
            outlier_cols = _outlier_columns(rng_for(seed, config, 1000 + tensor_id), cols, outlier_fraction)
        x[:, outlier_cols] *= np.float32(outlier_scale)
    return (round_to_bf16(x) if bf16 else x), outlier_cols


def weights(seed, config, tensor_id, rows, cols, std=0.02, row_outlier_fraction=0.0,
            row_outlier_scale=8.0, bf16=True):
    """[rows, cols] weights ~N(0, std) with an optional fraction of rows scaled up."""
    rng = rng_for(seed, config, tensor_id)
    w = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)
    if row_outlier_fraction > 0:
        n = max(1, int(round(row_outlier_fraction * rows)))
        sel = np.sort(rng_for(seed, config, 2000 + tensor_id).choice(rows, size=n, replace=False))
        w[sel] *= np.float32(row_outlier_scale)
    return round_to_bf16(w) if bf16 else w


@dataclass
class Linear:
    """One GEMM of a workload: activations A[M,K] against a (possibly fused)
    weight W[N,K] given as a list of per-module blocks of rows."""

    name: str
    a: np.ndarray
    a_calib: np.ndarray  # separate draw used to calibrate the static activation scale
    modules: list = field(default_factory=list)  # [(name, W_i)]
    a_dtype: str = "bf16"

    @property
    def m(self):
        return self.a.shape[0]

    @property
    def k(self):
        return self.a.shape[1]

    @property
    def n(self):
        return sum(w.shape[0] for _, w in self.modules)


def make_workload(config: str, seed: int = 0, m_override: int | None = None):
    """The GEMMs of one named workload, as host arrays.

    tiny   : A[64x256] fp32 ~N(0,1); W[128x256] fp32 ~N(0,0.02)
    gdn    : A[8192x5120] bf16 ~N(0,1), 0.1% outlier channels x100; fused
             qkv|z|a|b weights ~N(0,0.02), one module each
    mlp    : gate_up: A[8192x5120] t(3) + outlier channels -> gate|up
             [2x17408x5120]; down: A[8192x17408] t(3) -> W[5120x17408];
             weights ~N(0,0.02) with 1% of rows x8
    decode : A[32x5120] ~N(0,1) + outlier channels; W[34816x5120] ~N(0,0.02)
    long   : A[32768x5120] t(3) + outlier channels -> W_qkv[14336x5120];
             A2[32768x6144] t(3) -> W_o[5120x6144]
    """
    if config == "tiny":
        m = m_override or 64
        a, oc = activations(seed, config, 0, m, 256, outlier_fraction=0.0, bf16=False)
        ac, _ = activations(seed, config, 100, m, 256, outlier_fraction=0.0, bf16=False)
        w = weights(seed, config, 1, 128, 256, bf16=False)
        return [Linear("tiny", a, ac, [("w", w)], a_dtype="f32")]
    if config == "gdn":
        m = m_override or 8192
        a, oc = activations(seed, config, 0, m, HIDDEN)
        ac, _ = activations(seed, config, 100, m, HIDDEN, outlier_cols=oc)
        mods = [(nm, weights(seed, config, 1 + i, rows, HIDDEN)) for i, (nm, rows) in enumerate(GDN_MODULES)]
        return [Linear("gdn_in_proj", a, ac, mods)]
    if config == "mlp":
        m = m_override or 8192
        a1, oc1 = activations(seed, config, 0, m, HIDDEN, dist="t3")
        a1c, _ = activations(seed, config, 100, m, HIDDEN, dist="t3", outlier_cols=oc1)
        gate = weights(seed, config, 1, MLP_INTER, HIDDEN, row_outlier_fraction=0.01)
        up = weights(seed, config, 2, MLP_INTER, HIDDEN, row_outlier_fraction=0.01)
        a2, oc2 = activations(seed, config, 3, m, MLP_INTER, dist="t3")
        a2c, _ = activations(seed, config, 103, m, MLP_INTER, dist="t3", outlier_cols=oc2)
        down = weights(seed, config, 4, HIDDEN, MLP_INTER, row_outlier_fraction=0.01)
        return [Linear("mlp_gate_up", a1, a1c, [("gate", gate), ("up", up)]),
                Linear("mlp_down", a2, a2c, [("down", down)])]
    if config == "decode":
        m = m_override or 32
        a, oc = activations(seed, config, 0, m, HIDDEN)
        ac, _ = activations(seed, config, 100, m, HIDDEN, outlier_cols=oc)
        w = weights(seed, config, 1, 2 * MLP_INTER, HIDDEN)
        return [Linear("decode_gate_up", a, ac, [("w", w)])]
    if config == "long":
        m = m_override or 32768
        a, oc = activations(seed, config, 0, m, HIDDEN, dist="t3")
        ac, _ = activations(seed, config, 100, m, HIDDEN, dist="t3", outlier_cols=oc)
        wq = weights(seed, config, 1, ATTN_QKV, HIDDEN)
        a2, oc2 = activations(seed, config, 2, m, ATTN_O_IN, dist="t3")
        a2c, _ = activations(seed, config, 102, m, ATTN_O_IN, dist="t3", outlier_cols=oc2)
        wo = weights(seed, config, 3, HIDDEN, ATTN_O_IN)
        return [Linear("attn_qkv", a, ac, [("qkv", wq)]), Linear("attn_o", a2, a2c, [("o", wo)])]
    raise ValueError(f"unknown workload {config!r}")
