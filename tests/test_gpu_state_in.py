"""GPU: a forward that continues from a state (state_in) against the fp64
oracle run over the whole sequence in one pass.

Splitting a sequence anywhere and running the second part from the first
part's state must give the outputs (and the final state) of one forward over
the whole sequence, to the same bar as every other parity case.  Covers:
splits at a block boundary of every scale and inside blocks (then each
coarse branch's first block in the second part completes the block the state
holds in progress), coarse branches whose first positions in the second part
take the output held from the first part, a second part shorter than a
coarse scale (that branch then contributes only its held output, and keeps
its state), decode steps between two forwards, state_in equal to state_out,
the device-side checks (a header of another batch, a state that records an
error), and graph capture of a continuing forward."""
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
    # splits inside blocks: block 0 of the second part completes the pending one
    ("tiny_f32", 2, 6, 50, False),    # r = 2 for scale 4
    ("tiny_f32", 2, 33, 47, True),    # r = 1 for scales 2 and 4
    ("tiny_f32", 1, 7, 1, False),     # the second part completes scale 4's block only
    ("tiny_f32", 2, 5, 2, False),     # scale 4's block stays pending across the call
    ("tiny_f32", 1, 513, 599, False), # segmented walks after an offset
    ("main", 2, 131, 101, True),
    ("main", 1, 258, 3, False),
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


def _all_nan(t) -> bool:
    import torch
    return bool(torch.isnan(t.float()).all())


@pytest.mark.parametrize("cfg_name,B,L1,steps,L2", [
    ("tiny_f32", 2, 30, 3, 40),   # 33: inside scale 2's and 4's blocks
    ("tiny_f32", 1, 8, 1, 5),
    ("main", 2, 128, 5, 70),
])
def test_forward_after_decode_steps(cfg_name, B, L1, steps, L2):
    """A prefill, a few decode steps (any number, so the position may fall
    inside a block), then a forward over the rest from the same state: the
    outputs of all three against one oracle pass."""
    import torch
    cfg = WORKLOADS[cfg_name].cfg
    say(f"prefill {L1} + {steps} decode steps + forward {L2}: {cfg_name} B={B}")
    L = L1 + steps + L2
    X, W = make_inputs(cfg, B, L, seed=16)
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
    assert binding.msgla_state_query(st)["position"] == L


def test_state_of_another_batch_is_rejected():
    """A state written for B = 1 given to a B = 2 call: only its header is read."""
    import torch
    cfg = TINY
    X, W = make_inputs(cfg, 2, 16, seed=13)
    layer = DeviceLayer(cfg, W)
    st = layer.new_state(1)
    layer.state_init(st, 1)
    say("state_in written for B=1, used with B=2")
    st2 = layer.new_state(2)
    out = layer.forward(to_device(X, cfg.dtype), state_in=st, state_out=st2)
    torch.cuda.synchronize()
    assert _all_nan(out)
    assert binding.msgla_state_query(st2)["status"] == 1


def test_error_state_propagates_and_decode_refuses_it():
    """A state that records an error (here: written by a forward whose entry
    state had another batch size) is refused by the next forward (status 1)
    and by the decode step (NaN output, the state unchanged)."""
    import torch
    cfg = TINY
    X, W = make_inputs(cfg, 2, 48, seed=15)
    layer = DeviceLayer(cfg, W)
    st = layer.new_state(2)
    layer.forward(to_device(X[:, :6], cfg.dtype), state_out=st)
    one = layer.new_state(1)
    layer.state_init(one, 1)
    bad = layer.new_state(2)
    layer.forward(to_device(X[:, 6:10], cfg.dtype), state_in=one, state_out=bad)
    torch.cuda.synchronize()
    assert binding.msgla_state_query(bad)["status"] == 1
    say("forward and decode from a state that records an error")
    bad2 = layer.new_state(2)
    out = layer.forward(to_device(X[:, 10:18], cfg.dtype), state_in=bad, state_out=bad2)
    torch.cuda.synchronize()
    assert _all_nan(out) and binding.msgla_state_query(bad2)["status"] == 1
    before = bad.clone()
    o = layer.decode_step(to_device(np.ascontiguousarray(X[:, 10]), cfg.dtype), bad)
    torch.cuda.synchronize()
    assert _all_nan(o) and torch.equal(bad, before)
    # the usable state still decodes
    o = layer.decode_step(to_device(np.ascontiguousarray(X[:, 6]), cfg.dtype), st)
    torch.cuda.synchronize()
    assert not torch.isnan(o.float()).any()
    assert binding.msgla_state_query(st)["position"] == 7


def test_continuing_forward_captured_in_a_graph():
    """msgla_forward with state_in and state_out captured once as a HIP graph
    and replayed with different entry states (eager work and a synchronisation
    between replays): every replay equals the eager call bit for bit."""
    import torch
    cfg = MAIN
    B, L1, L2 = 2, 128, 72
    X, W = make_inputs(cfg, B, L1 + L2, seed=16)
    X_alt = make_inputs(cfg, B, L1, seed=17)[0]
    layer = DeviceLayer(cfg, W)
    entry = {"a": layer.new_state(B), "b": layer.new_state(B)}
    layer.forward(to_device(X[:, :L1], cfg.dtype), state_out=entry["a"])
    layer.forward(to_device(X_alt, cfg.dtype), state_out=entry["b"])
    x2 = to_device(X[:, L1:], cfg.dtype)
    eager = {}
    for k, s0 in entry.items():
        s_out = layer.new_state(B)
        o = layer.forward(x2, state_in=s0, state_out=s_out)
        eager[k] = (o.clone(), s_out.clone())
    torch.cuda.synchronize()
    say(f"graph capture of a continuing forward main dims B={B} L={L2}")
    s_in = entry["a"].clone()
    s_out = layer.new_state(B)
    out = layer.new_output(B, L2)
    layer.ensure_workspace(B, L2)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x2, out=out, state_in=s_in, state_out=s_out)
    scratch = torch.zeros(1 << 20, device="cuda")
    def same_state(a, b):
        # the blob's contents (header fields, S, pending sums, held outputs);
        # its padding bytes are never written and hold whatever was there
        ra, rb = read_state(cfg, a, B), read_state(cfg, b, B)
        if any(ra[f] != rb[f] for f in ("magic", "version", "B", "m", "pos")):
            return False
        return all(np.array_equal(x[key], y[key]) for x, y in zip(ra["branches"], rb["branches"])
                   for key in ("S", "psum", "held"))

    for k in ("a", "b", "a", "b", "b", "a"):
        s_in.copy_(entry[k])
        g.replay()
        scratch.add_(1.0)  # the program's own eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager[k][0]), k
        assert same_state(s_out, eager[k][1]), k
    ref = orc.layer_forward(X, W, cfg)[:, L1:]
    err, zeros = orc.row_relative_error(from_device(out), ref)
    assert zeros and err <= TOL[cfg.dtype]
