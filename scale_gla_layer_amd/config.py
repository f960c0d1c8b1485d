"""Layer configuration and the named synthetic workloads.

The layer is the MS-GLA token-mixing layer described in the reading notes
"MS-GLA：多时间尺度门控线性注意力研读笔记" (notes on arXiv:2609.35664,
"MS-GLA: Multi-Scale Gated Linear Attention ..."), Sec. 3 and Eqs. (8)-(11).

A configuration names a set of branches.  Branch i pools the sequence over
non-overlapping blocks of ``scales[i]`` tokens and owns ``heads[i]`` GLA heads
of width ``d_k`` x ``d_v`` (Sec. 3.2, Eq. (9): the head counts add up to the
layer's total H).  ``gate_rank`` is the rank r of the low-rank forget-gate
projection, ``gate_normalizer`` the divisor applied to logsigmoid, and
``chunk`` is only the GPU schedule's chunk length (Sec. 3.4 separates the
pooling block from the kernel chunk; results do not depend on it).
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class MsglaConfig:
    scales: Tuple[int, ...]
    heads: Tuple[int, ...]
    d_model: int
    d_k: int
    d_v: int
    gate_rank: int
    chunk: int = 64
    gate_normalizer: float = 16.0
    q_scale: float = 1.0
    dtype: str = BF16
    norm: bool = False  # per-head RMS normalisation of each branch's output before W_o

    def __post_init__(self):
        if len(self.scales) != len(self.heads) or not self.scales:
            raise ValueError("scales and heads must be non-empty and of equal length")
        if len(set(self.scales)) != len(self.scales):
            raise ValueError("scales must be distinct")
        if any(s <= 0 for s in self.scales) or any(h <= 0 for h in self.heads):
            raise ValueError("scales and heads must be positive")
        if self.dtype not in (F32, BF16):
            raise ValueError(f"dtype must be {F32!r} or {BF16!r}")

    @property
    def n_branches(self) -> int:
        return len(self.scales)

    @property
    def total_heads(self) -> int:
        return sum(self.heads)

    def state_elements(self) -> int:
        """Recurrent-state elements per sequence: sum_s h_s d_k d_v = H d_k d_v."""
        return sum(h * self.d_k * self.d_v for h in self.heads)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg: MsglaConfig
    batch: int
    seq_len: int
    gate_bias: Optional[Tuple[float, float]] = None  # U(lo, hi) per channel, else 0
    description: str = ""


def _layer(scales, heads, dtype=BF16, d=1024, dk=128, dv=256, r=16, chunk=64):
    return MsglaConfig(tuple(scales), tuple(heads), d, dk, dv, r, chunk, 16.0, 1.0, dtype)


WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", MsglaConfig((1, 2, 4), (2, 1, 1), 64, 16, 32, 4, 16, 16.0, 1.0, F32),
        batch=1, seq_len=64,
        description="tiny fp32 MS-GLA {1,2,4}/[2,1,1], d=64, d_k=16, d_v=32, r=4, chunk 16"),
    "gla_baseline": Workload(
        "gla_baseline", _layer((1,), (4,)), batch=8, seq_len=2048,
        description="single-scale GLA layer, 4 heads at scale 1, B=8, L=2048, d=1024, bf16"),
    "main": Workload(
        "main", _layer((1, 2, 4), (2, 1, 1)), batch=8, seq_len=2048,
        description="MS-GLA {1,2,4}/[2,1,1], B=8, L=2048, d=1024, bf16"),
    "long": Workload(
        "long", _layer((1, 2, 4), (2, 1, 1)), batch=1, seq_len=16384, gate_bias=(1.0, 4.0),
        description="MS-GLA {1,2,4}/[2,1,1], B=1, L=16384, gate bias U(1,4), bf16"),
    "sweep_1248": Workload(
        "sweep_1248", _layer((1, 2, 4, 8), (1, 1, 1, 1)), batch=16, seq_len=4096,
        description="MS-GLA {1,2,4,8}/[1,1,1,1], B=16, L=4096, bf16"),
    "sweep_24": Workload(
        "sweep_24", _layer((2, 4), (2, 2)), batch=16, seq_len=4096,
        description="MS-GLA {2,4}/[2,2] (no fine branch), B=16, L=4096, bf16"),
}
