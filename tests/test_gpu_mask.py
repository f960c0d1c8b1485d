"""GPU parity of the masked forward (Eq. (8) with a token mask M) against the
fp64 oracle, through the C ABI.

Masks come from ``synth.make_mask``: a padded batch (each sequence keeps a
prefix of random length) with random holes, plus the edge cases all ones,
all zeros, and whole blocks of padding.  Same bars as the unmasked parity
tests: row-relative error <= 1e-4 (fp32) and <= 2e-2 (bf16), rows the oracle
gives as exactly zero exactly zero on the device.

The bf16 cases put no holes in the first 8 positions of a sequence.  A hole
there can leave a row whose only term is a branch's first coarse output,
(q_0 . k_0) v_0 W_o, whose dot product cancels strongly; the bf16 path rounds
each pooled mean to bf16 before the projection, and that rounding alone moves
such a row by up to ~0.1 of its own (tiny) size.  The fp32 cases have holes
everywhere."""
import dataclasses

import numpy as np
import pytest

from scale_gla_layer_amd.config import BF16, F32, MsglaConfig, WORKLOADS
from scale_gla_layer_amd.runner import from_device
from scale_gla_layer_amd.synth import make_inputs, make_mask
from tests.gpu_cases import check_against_oracle, run_device, say

pytestmark = pytest.mark.gpu

TINY = WORKLOADS["tiny_f32"].cfg
MAIN = WORKLOADS["main"].cfg


def masked_case(cfg, B, L, seed, M=None, batches=None):
    say(f"masked scales={cfg.scales} heads={cfg.heads} d={cfg.d_model} dk={cfg.d_k} dv={cfg.d_v} "
        f"C={cfg.chunk} {cfg.dtype} B={B} L={L} seed={seed}")
    X, W = make_inputs(cfg, B, L, seed=seed)
    if M is None:
        M = make_mask(B, L, seed=seed + 1000, hole_prob=0.1, hole_start=8 if cfg.dtype == BF16 else 0)
    _, _, out, _ = run_device(cfg, X, W, M=M)
    O = from_device(out)
    check_against_oracle(cfg, X, W, O, batches=batches, M=M)
    return X, W, M, O


@pytest.mark.parametrize("L", [1, 3, 17, 64, 100, 257])
def test_tiny_fp32_masked(L):
    masked_case(TINY, 3, L, seed=L)


@pytest.mark.parametrize("scales,heads", [((1, 3, 4), (1, 1, 1)), ((2, 4), (1, 1)), ((1, 2, 4, 8), (1, 1, 1, 1))])
def test_fp32_masked_scale_sets(scales, heads):
    cfg = dataclasses.replace(TINY, scales=scales, heads=heads)
    masked_case(cfg, 2, 131, seed=7)


def test_fp32_all_padding_is_zero():
    masked_case(TINY, 2, 70, seed=3, M=np.zeros((2, 70), np.uint8))


def test_fp32_whole_padded_blocks():
    L = 96
    M = np.ones((2, L), np.uint8)
    M[0, 8:16] = 0      # two whole s = 4 blocks
    M[1, 1::4] = 0      # one token of every s = 4 block
    M[1, 40:64] = 0
    masked_case(TINY, 2, L, seed=4, M=M)


def test_mask_of_ones_at_scale_one_is_bit_exact():
    """With only a scale-1 branch the mask multiplies the projections by 1."""
    import torch
    cfg = dataclasses.replace(TINY, scales=(1,), heads=(2,))
    X, W = make_inputs(cfg, 2, 90, seed=5)
    _, _, out0, _ = run_device(cfg, X, W)
    _, _, out1, _ = run_device(cfg, X, W, M=np.ones((2, 90), np.uint8))
    assert torch.equal(out0, out1)


def test_bf16_masked_main_dims():
    cfg = dataclasses.replace(MAIN)
    masked_case(cfg, 2, 300, seed=11)


def test_bf16_masked_full_size():
    """The main workload's shape with a padded-batch mask: the device runs the
    whole batch, the oracle two sampled sequences."""
    wl = WORKLOADS["main"]
    masked_case(wl.cfg, wl.batch, wl.seq_len, seed=12, batches=[0, 5])
