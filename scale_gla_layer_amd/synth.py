"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module holds no arithmetic of the layer itself: it only draws numbers and
rounds them to the storage precision, so both sides consume identical values.

Recipe (the workloads of the MS-GLA notes are trained-model runs on FineWeb-Edu;
the layer's cost does not depend on data values, so Gaussian inputs of the
same shapes stand in for them):

* ``numpy.random.default_rng(seed)`` (PCG64) draws float64 in this fixed order:
  X [B, L, d] ~ N(0, 1); then for every branch, in configuration order,
  W_q [d, h*d_k], W_k [d, h*d_k], W_v [d, h*d_v], W_g1 [d, r], W_g2 [r, h*d_k],
  all ~ N(0, 0.02) (0.02 is a standard deviation), then b_g [h*d_k] drawn
  ~ U(lo, hi) only when the workload asks for a random gate bias (else 0),
  then W_o [h*d_v, d] ~ N(0, 0.02); finally W_f [d, m] ~ N(0, 0.02) and
  b_f [m] = 0.
* Values are rounded to the storage type with round-to-nearest-even: float32
  for the fp32 path, bfloat16 (via float32) for the bf16 path.  Biases stay
  float32 in both paths.
* Weights use the notes' row-vector convention ``x @ W`` with ``W`` stored
  [in][out] row-major.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

from .config import BF16, F32, MsglaConfig

STD = 0.02


def round_f32(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def f32_to_bf16_bits(a32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(a32)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(a: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f64(f32_to_bf16_bits(np.asarray(a, dtype=np.float64).astype(np.float32)))


def round_to(a: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16(a) if dtype == BF16 else round_f32(a)


@dataclasses.dataclass
class BranchWeights:
    W_q: np.ndarray   # [d, h*d_k]
    W_k: np.ndarray   # [d, h*d_k]
    W_v: np.ndarray   # [d, h*d_v]
    W_g1: np.ndarray  # [d, r]
    W_g2: np.ndarray  # [r, h*d_k]
    b_g: np.ndarray   # [h*d_k]  (float32 values)
    W_o: np.ndarray   # [h*d_v, d]
    g_norm: Optional[np.ndarray] = None  # [h*d_v] (float32 values), configs with norm only


@dataclasses.dataclass
class LayerWeights:
    branches: List[BranchWeights]
    W_f: np.ndarray   # [d, m]
    b_f: np.ndarray   # [m]  (float32 values)


def make_weights(cfg: MsglaConfig, rng: np.random.Generator,
                 gate_bias: Optional[Tuple[float, float]] = None) -> LayerWeights:
    d, dk, dv, r = cfg.d_model, cfg.d_k, cfg.d_v, cfg.gate_rank
    rt = lambda a: round_to(a, cfg.dtype)
    brs = []
    for h in cfg.heads:
        W_q = rt(rng.normal(0.0, STD, (d, h * dk)))
        W_k = rt(rng.normal(0.0, STD, (d, h * dk)))
        W_v = rt(rng.normal(0.0, STD, (d, h * dv)))
        W_g1 = rt(rng.normal(0.0, STD, (d, r)))
        W_g2 = rt(rng.normal(0.0, STD, (r, h * dk)))
        if gate_bias is None:
            b_g = np.zeros(h * dk)
        else:
            b_g = round_f32(rng.uniform(gate_bias[0], gate_bias[1], h * dk))
        W_o = rt(rng.normal(0.0, STD, (h * dv, d)))
        brs.append(BranchWeights(W_q, W_k, W_v, W_g1, W_g2, b_g, W_o))
    m = cfg.n_branches
    W_f = rt(rng.normal(0.0, STD, (d, m)))
    b_f = np.zeros(m)
    if cfg.norm:  # drawn last, so configurations without it keep their streams
        for br, h in zip(brs, cfg.heads):
            br.g_norm = round_f32(1.0 + 0.1 * rng.normal(0.0, 1.0, h * dv))
    return LayerWeights(brs, W_f, b_f)


def make_inputs(cfg: MsglaConfig, batch: int, seq_len: int, seed: int = 0,
                gate_bias: Optional[Tuple[float, float]] = None):
    """Returns (X [B, L, d] float64 rounded to cfg.dtype, LayerWeights)."""
    rng = np.random.default_rng(seed)
    X = round_to(rng.normal(0.0, 1.0, (batch, seq_len, cfg.d_model)), cfg.dtype)
    W = make_weights(cfg, rng, gate_bias)
    return X, W


def make_tokens(cfg: MsglaConfig, batch: int, n: int, seed: int) -> np.ndarray:
    """Extra N(0,1) tokens [B, n, d] (decode inputs), from their own stream."""
    rng = np.random.default_rng(seed)
    return round_to(rng.normal(0.0, 1.0, (batch, n, cfg.d_model)), cfg.dtype)


def make_mask(batch: int, seq_len: int, seed: int, min_keep: float = 0.5,
              hole_prob: float = 0.05, hole_start: int = 0) -> np.ndarray:
    """Token mask [B, L] uint8 of a padded batch: sequence b keeps its first
    len_b tokens, len_b uniform in [ceil(min_keep L), L], and each kept token
    from position hole_start on is also dropped with probability hole_prob;
    1 = token, 0 = padding."""
    rng = np.random.default_rng(seed)
    lo = int(np.ceil(min_keep * seq_len))
    lens = rng.integers(lo, seq_len + 1, size=batch)
    keep = np.arange(seq_len)[None, :] < lens[:, None]
    holes = rng.random((batch, seq_len)) < hole_prob
    holes[:, :hole_start] = False
    return (keep & ~holes).astype(np.uint8)


def storage_array(a: np.ndarray, dtype: str) -> np.ndarray:
    """Host buffer in the storage type: uint16 bf16 bits or float32."""
    if dtype == BF16:
        return f32_to_bf16_bits(np.asarray(a, dtype=np.float64).astype(np.float32))
    return np.ascontiguousarray(a, dtype=np.float32)
