"""GPU: a forward that continues from a state (state_in) against the fp64
oracle run over the whole sequence in one pass.

Splitting a sequence at a position that is a multiple of every scale and
running the second part from the first part's state must give the outputs
(and the final state) of one forward over the whole sequence, to the same
bar as every other parity case.  Covers: coarse branches whose first
positions in the second part take the output held from the first part, a
second part shorter than a coarse scale (that branch then contributes only
its held output, and keeps its state), state_in equal to state_out, and the
errors for a position inside a block and for a header of another batch."""
import numpy as np
import pytest

from oracle import msgla_oracle as orc
from scale_gla_layer_amd import binding
from scale_gla_layer_amd.config import WORKLOADS
from scale_gla_layer_amd.runner import DeviceLayer, from_device, read_state, to_device
from scale_gla_layer_amd.synth import make_inputs
from tests.gpu_cases import TOL, check_against_oracle, say

pytestmark = pytest.mark.gpu

TINY = WORKLOADS["tiny_f32"].cfg
MAIN = WORKLOADS["main"].cfg


def _split_run(cfg, B, L1, L2, seed, same_buffer, gate_bias=None):
    import torch
    X, W = make_inputs(cfg, B, L1 + L2, seed=seed, gate_bias=gate_bias)
    layer = DeviceLayer(cfg, W)
    s1 = layer.new_state(B)
    s2 = s1 if same_buffer else layer.new_state(B)
    o1 = layer.forward(to_device(X[:, :L1], cfg.dtype), state_out=s1)
    o2 = layer.forward(to_device(X[:, L1:], cfg.dtype), state_in=s1, state_out=s2)
    torch.cuda.synchronize()
    O = np.concatenate([from_device(o1), from_device(o2)], axis=1)
    return X, W, O, s2


@pytest.mark.parametrize("cfg_name,B,L1,L2,same", [
    ("tiny_f32", 2, 32, 50, False),
    ("tiny_f32", 2, 16, 3, True),     # second part shorter than scale 4
    ("tiny_f32", 1, 4, 1, False),     # one token after one block of every scale
    ("main", 2, 128, 100, True),
    ("main", 1, 256, 2, False),       # scale 4 sees no block in the second part
    ("tiny_f32", 1, 512, 600, False), # both parts walk the chunk states in segments
    ("tiny_f32", 2, 400, 300, True),
])
def test_continue_matches_one_pass(cfg_name, B, L1, L2, same):
    cfg = WORKLOADS[cfg_name].cfg
    say(f"state_in {cfg_name} B={B} L1={L1} L2={L2} same_buffer={same}")
    X, W, O, st = _split_run(cfg, B, L1, L2, seed=11, same_buffer=same)
    check_against_oracle(cfg, X, W, O)
    if cfg.dtype == "f32":
        dev = read_state(cfg, st, B)
        _, ref = orc.layer_forward(X, W, cfg, return_state=True)
        assert dev["pos"] == L1 + L2
        for i, (bd, br) in enumerate(zip(dev["branches"], ref["branches"])):
            for key in ("S", "psum", "held"):
                a, b = bd[key], br[key]
                scale = max(1e-30, np.abs(b).max())
                assert np.abs(a - b).max() <= TOL["f32"] * scale + 1e-12, (i, key)


def test_sequence_shards_at_long_context_gates():
    """Two 2048-token shards of one sequence with the long workload's gates
    (alpha near 1, so the carried state dominates the second shard)."""
    wl = WORKLOADS["long"]
    say("state_in shards B=1 2 x 2048, gate bias U(1,4)")
    X, W, O, _ = _split_run(wl.cfg, 1, 2048, 2048, seed=14, same_buffer=True,
                            gate_bias=wl.gate_bias)
    check_against_oracle(wl.cfg, X, W, O)


def test_position_inside_a_block_is_unsupported():
    cfg = TINY
    X, W = make_inputs(cfg, 1, 40, seed=12)
    layer = DeviceLayer(cfg, W)
    st = layer.new_state(1)
    layer.forward(to_device(X[:, :6], cfg.dtype), state_out=st)  # 6 is not a multiple of 4
    say("state_in at position 6 (scale 4 has a block in progress)")
    with pytest.raises(binding.MsglaError) as e:
        layer.forward(to_device(X[:, 6:], cfg.dtype), state_in=st)
    assert e.value.status == 2


def test_state_of_another_batch_is_rejected():
    cfg = TINY
    X, W = make_inputs(cfg, 2, 16, seed=13)
    layer = DeviceLayer(cfg, W)
    st = layer.new_state(1)
    layer.state_init(st, 1)
    say("state_in written for B=1, used with B=2")
    with pytest.raises(binding.MsglaError) as e:
        layer.forward(to_device(X, cfg.dtype), state_in=st)
    assert e.value.status == 1
