"""GPU: msgla_forward_noalloc (the forward on the library's own per-device
workspace array, for callers that cannot allocate) against msgla_forward on
the same inputs: two calls in a row, the second with a smaller input, each
bit-identical to msgla_forward (same kernels), the smaller one also against
the fp64 oracle; sizes beyond the array are refused."""
import numpy as np
import pytest

from oracle import msgla_oracle as orc
from scale_gla_layer_amd import binding
from scale_gla_layer_amd.config import WORKLOADS
from scale_gla_layer_amd.runner import DeviceLayer, from_device, read_state, to_device
from scale_gla_layer_amd.synth import make_inputs
from tests.gpu_cases import TOL, say

pytestmark = pytest.mark.gpu


def _noalloc(layer, x, state_out=None, state_in=None):
    B, L, _ = x.shape
    out = layer.new_output(B, L)
    binding.msgla_forward_noalloc(layer.cfg, layer.packed, x, B, L, out, state_out=state_out,
                                  state_in=state_in)
    return out


def _same_state(cfg, a, b, B):
    ra, rb = read_state(cfg, a, B), read_state(cfg, b, B)
    return ra["pos"] == rb["pos"] and all(
        np.array_equal(x[k], y[k]) for x, y in zip(ra["branches"], rb["branches"])
        for k in ("S", "psum", "held"))


def test_noalloc_forward_matches_the_workspace_forward():
    import torch
    wl = WORKLOADS["main"]
    cfg = wl.cfg
    X, W = make_inputs(cfg, wl.batch, wl.seq_len, seed=31)
    layer = DeviceLayer(cfg, W)
    # first call: the full main workload (its workspace fits the array)
    say(f"noalloc main B={wl.batch} L={wl.seq_len}")
    x = to_device(X, cfg.dtype)
    ref = layer.forward(x)
    got = _noalloc(layer, x)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    # second call: a smaller input with a state export, then a continuation
    B, L1, L2 = 2, 300, 64
    X2 = X[:B, : L1 + L2]
    say(f"noalloc main dims B={B} L={L1} then {L2} from the state")
    s_ref, s_got = layer.new_state(B), layer.new_state(B)
    x1 = to_device(X2[:, :L1], cfg.dtype)
    ref1 = layer.forward(x1, state_out=s_ref)
    got1 = _noalloc(layer, x1, state_out=s_got)
    torch.cuda.synchronize()
    assert torch.equal(got1, ref1)
    assert _same_state(cfg, s_got, s_ref, B)
    x2 = to_device(X2[:, L1:], cfg.dtype)
    ref2 = layer.forward(x2, state_in=s_ref)
    got2 = _noalloc(layer, x2, state_in=s_got)
    torch.cuda.synchronize()
    assert torch.equal(got2, ref2)
    O = np.concatenate([from_device(got1), from_device(got2)], axis=1)
    err, zeros = orc.row_relative_error(O, orc.layer_forward(X2, W, cfg))
    say(f"noalloc row-relative error {err:.3e}")
    assert zeros and err <= TOL[cfg.dtype]


def test_noalloc_refuses_sizes_beyond_its_array():
    wl = WORKLOADS["sweep_1248"]
    assert binding.msgla_workspace_bytes(wl.cfg, wl.batch, wl.seq_len) > binding.NOALLOC_WORKSPACE_BYTES
    X, W = make_inputs(wl.cfg, 1, 64, seed=32)
    layer = DeviceLayer(wl.cfg, W)
    x = to_device(X, wl.cfg.dtype)
    out = layer.new_output(1, 64)
    with pytest.raises(binding.MsglaError) as e:
        binding.msgla_forward_noalloc(wl.cfg, layer.packed, x, wl.batch, wl.seq_len, out)
    assert e.value.status == 3
