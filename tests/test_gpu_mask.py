"""GPU parity of the masked forward (Eq. (8) with a token mask M) against the
fp64 oracle, through the C ABI.

Masks come from ``synth.make_mask``: a padded batch (each sequence keeps a
prefix of random length) with random holes, plus the edge cases all ones,
all zeros, and whole blocks of padding.  Same bars as the unmasked parity
tests: row-relative error <= 1e-4 (fp32) and <= 2e-2 (bf16), rows the oracle
gives as exactly zero exactly zero on the device.

Holes may fall anywhere, also in a sequence's first positions.  There a row's
only term can be a branch's first coarse output, (q_0 . k_0) v_0 W_o, whose
dot product may cancel strongly; the bf16 path therefore projects each block
mean's bf16 rounding residual as well (q and k see the mean at fp32
accuracy), which the bf16 cases here exercise."""
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
        M = make_mask(B, L, seed=seed + 1000, hole_prob=0.1)
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


@pytest.mark.parametrize("seed", [21, 22, 23])
def test_bf16_masked_holes_at_the_start(seed):
    """Dense holes in the first positions, where rows hold one coarse term:
    every sequence misses some of its first 8 tokens."""
    cfg = dataclasses.replace(MAIN)
    B, L = 4, 96
    M = make_mask(B, L, seed=seed, min_keep=1.0, hole_prob=0.05)
    rng = np.random.default_rng(seed)
    for b in range(B):
        M[b, rng.choice(8, size=1 + b, replace=False)] = 0
    masked_case(cfg, B, L, seed=seed, M=M)


def test_bf16_masked_no_fine_branch():
    """{2,4}: with holes at the start, early rows hold a single coarse term."""
    cfg = WORKLOADS["sweep_24"].cfg
    M = np.ones((3, 80), np.uint8)
    M[0, 0] = 0
    M[1, 1:3] = 0
    M[2, :4] = 0
    masked_case(cfg, 3, 80, seed=24, M=M)


def test_bf16_masked_full_size():
    """The main workload's shape with a padded-batch mask, every sequence
    against the oracle."""
    wl = WORKLOADS["main"]
    masked_case(wl.cfg, wl.batch, wl.seq_len, seed=12)


# ------------------------------------------------------------------ masked calls and the streaming state


def _masked_prefix(B, L0, L, seed):
    """A mask over L positions: holes in the first L0 (also in the last,
    incomplete blocks of the prefix), ones after them."""
    rng = np.random.default_rng(seed)
    M = np.ones((B, L), np.uint8)
    M[:, :L0] = rng.random((B, L0)) < 0.6
    M[0, L0 - 2: L0] = 0
    return M


@pytest.mark.parametrize("cfg_name,B,L0,n", [("tiny_f32", 2, 37, 12), ("tiny_f32", 3, 66, 9),
                                             ("main", 2, 45, 12)])
def test_masked_prefill_then_decode(cfg_name, B, L0, n):
    """A masked forward exporting its state, then decode steps: the outputs
    equal one masked forward whose mask is all ones over the decoded
    positions (the incomplete blocks' token counts carry over)."""
    import torch
    from oracle import msgla_oracle as orc
    from scale_gla_layer_amd.runner import read_state, to_device
    from tests.gpu_cases import TOL
    cfg = WORKLOADS[cfg_name].cfg
    say(f"masked prefill {cfg_name} B={B} L0={L0} then {n} decode steps")
    X, W = make_inputs(cfg, B, L0 + n, seed=40 + L0)
    M = _masked_prefix(B, L0, L0 + n, seed=41 + L0)
    layer, _, out, st = run_device(cfg, X[:, :L0], W, state_out=True, M=M[:, :L0])
    outs = [from_device(layer.decode_step(to_device(X[:, t], cfg.dtype), st)) for t in range(L0, L0 + n)]
    torch.cuda.synchronize()
    O = np.concatenate([from_device(out), np.stack(outs, axis=1)], axis=1)
    ref = orc.layer_forward(X, W, cfg, M=M)
    err, zeros = orc.row_relative_error(O, ref)
    say(f"row-relative error {err:.3e}")
    assert zeros and err <= TOL[cfg.dtype]
    assert read_state(cfg, st, B)["pos"] == L0 + n


def test_masked_state_export_matches_oracle():
    """fp32: the exported cache of a masked forward (S, masked pending sums,
    pending token counts, held outputs) against the oracle's."""
    from oracle import msgla_oracle as orc
    from scale_gla_layer_amd.runner import read_state
    cfg = TINY
    for L in (38, 64, 303):
        X, W = make_inputs(cfg, 2, L, seed=50 + L)
        M = _masked_prefix(2, L, L, seed=51 + L)
        say(f"masked state export tiny L={L}")
        _, _, _, st = run_device(cfg, X, W, state_out=True, M=M)
        dev = read_state(cfg, st, 2)
        _, ref = orc.layer_forward(X, W, cfg, return_state=True, M=M)
        for bd, br in zip(dev["branches"], ref["branches"]):
            assert np.array_equal(bd["tokens"], br["tokens"]), (L, bd["tokens"], br["tokens"])
            for key in ("S", "psum", "held"):
                a, b = bd[key], br[key]
                scale = max(1e-30, np.abs(b).max())
                assert np.abs(a - b).max() <= 1e-4 * scale + 1e-12, (L, key)


@pytest.mark.parametrize("cfg_name,B,L1,L2", [("tiny_f32", 2, 32, 50), ("main", 2, 128, 100),
                                               ("tiny_f32", 2, 31, 50), ("tiny_f32", 2, 6, 1),
                                               ("main", 2, 130, 99)])
def test_masked_forward_continues_from_a_state(cfg_name, B, L1, L2):
    """Two masked forwards, the second from the first's state (split at a
    block boundary of every scale, or inside blocks: then the second call's
    first block of a coarse branch completes the pending one, whose masked
    sum and token count the state holds), against one masked forward."""
    import torch
    from oracle import msgla_oracle as orc
    from scale_gla_layer_amd.runner import DeviceLayer, to_device
    from tests.gpu_cases import TOL, mask_to_device
    cfg = WORKLOADS[cfg_name].cfg
    say(f"masked continuation {cfg_name} B={B} L1={L1} L2={L2}")
    X, W = make_inputs(cfg, B, L1 + L2, seed=60)
    M = make_mask(B, L1 + L2, seed=61, min_keep=1.0, hole_prob=0.2)
    layer = DeviceLayer(cfg, W)
    st = layer.new_state(B)
    o1 = layer.forward(to_device(X[:, :L1], cfg.dtype), state_out=st, mask=mask_to_device(M[:, :L1]))
    o2 = layer.forward(to_device(X[:, L1:], cfg.dtype), state_in=st, state_out=st,
                       mask=mask_to_device(M[:, L1:]))
    torch.cuda.synchronize()
    O = np.concatenate([from_device(o1), from_device(o2)], axis=1)
    err, zeros = orc.row_relative_error(O, orc.layer_forward(X, W, cfg, M=M))
    say(f"row-relative error {err:.3e}")
    assert zeros and err <= TOL[cfg.dtype]
