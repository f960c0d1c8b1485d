"""GPU: the most general configurations the ABI accepts, against the fp64
oracle: eight branches with scales that are not powers of two (the generic
pooling path, blocks of different scales not nested), a gate rank above 16
(the 64-wide padded gate), q_scale != 1, several heads, both storage types;
each as a plain forward, a masked forward, and a forward split inside blocks
and continued from its state (the offsets of every branch differ), with
ragged lengths."""
import numpy as np
import pytest

from oracle import msgla_oracle as orc
from scale_gla_layer_amd.config import BF16, F32, MsglaConfig
from scale_gla_layer_amd.runner import DeviceLayer, from_device, to_device
from scale_gla_layer_amd.synth import make_inputs, make_mask
from tests.gpu_cases import TOL, check_against_oracle, mask_to_device, say

pytestmark = pytest.mark.gpu

SCALES = (1, 2, 3, 4, 5, 6, 7, 8)
HEADS = (2, 1, 1, 2, 1, 1, 1, 1)
WIDE = {
    F32: MsglaConfig(SCALES, HEADS, 128, 32, 64, 40, 32, 12.0, 0.75, F32),
    BF16: MsglaConfig(SCALES, HEADS, 128, 64, 128, 40, 64, 12.0, 0.75, BF16),
}


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("L", [1, 9, 211])
def test_eight_branches_odd_scales(dtype, L):
    import torch
    cfg = WIDE[dtype]
    B = 3
    say(f"wide config {dtype} B={B} L={L}")
    X, W = make_inputs(cfg, B, L, seed=70 + L)
    layer = DeviceLayer(cfg, W)
    out = layer.forward(to_device(X, cfg.dtype))
    torch.cuda.synchronize()
    check_against_oracle(cfg, X, W, from_device(out))


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_eight_branches_masked(dtype):
    import torch
    cfg = WIDE[dtype]
    B, L = 3, 173
    say(f"wide config masked {dtype} B={B} L={L}")
    X, W = make_inputs(cfg, B, L, seed=80)
    M = make_mask(B, L, seed=81, hole_prob=0.15)
    layer = DeviceLayer(cfg, W)
    out = layer.forward(to_device(X, cfg.dtype), mask=mask_to_device(M))
    torch.cuda.synchronize()
    check_against_oracle(cfg, X, W, from_device(out), M=M)


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("masked", [False, True])
def test_eight_branches_split_inside_blocks(dtype, masked):
    """Three calls over one sequence (117 + 1 + 95 tokens): the entry offsets
    of the second and third calls differ per branch (position mod s)."""
    import torch
    cfg = WIDE[dtype]
    B, parts = 2, (117, 1, 95)
    L = sum(parts)
    say(f"wide config split {parts} {dtype} masked={masked}")
    X, W = make_inputs(cfg, B, L, seed=90)
    M = make_mask(B, L, seed=91, min_keep=1.0, hole_prob=0.2) if masked else None
    layer = DeviceLayer(cfg, W)
    st = layer.new_state(B)
    outs, t0 = [], 0
    for k, n in enumerate(parts):
        m = mask_to_device(M[:, t0:t0 + n]) if masked else None
        o = layer.forward(to_device(X[:, t0:t0 + n], cfg.dtype), state_in=st if k else None,
                          state_out=st, mask=m)
        outs.append(from_device(o))
        t0 += n
    torch.cuda.synchronize()
    O = np.concatenate(outs, axis=1)
    err, zeros = orc.row_relative_error(O, orc.layer_forward(X, W, cfg, M=M))
    say(f"row-relative error {err:.3e}")
    assert np.all(np.isfinite(O)) and zeros and err <= TOL[cfg.dtype]


@pytest.mark.parametrize("dtype", [F32, BF16])
def test_eight_branches_prefill_decode_forward(dtype):
    """A prefill, 13 decode steps (every branch completes blocks at its own
    steps) and a forward over the rest from the same state."""
    import torch
    cfg = WIDE[dtype]
    B, L1, steps, L2 = 2, 50, 13, 40
    say(f"wide config prefill {L1} + {steps} decode steps + forward {L2}: {dtype}")
    L = L1 + steps + L2
    X, W = make_inputs(cfg, B, L, seed=95)
    layer = DeviceLayer(cfg, W)
    st = layer.new_state(B)
    outs = [from_device(layer.forward(to_device(X[:, :L1], cfg.dtype), state_out=st))]
    for t in range(L1, L1 + steps):
        o = layer.decode_step(to_device(np.ascontiguousarray(X[:, t]), cfg.dtype), st)
        outs.append(from_device(o)[:, None, :])
    outs.append(from_device(layer.forward(to_device(X[:, L1 + steps:], cfg.dtype), state_in=st,
                                          state_out=st)))
    torch.cuda.synchronize()
    check_against_oracle(cfg, X, W, np.concatenate(outs, axis=1))
