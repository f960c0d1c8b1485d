"""GPU parity of the streaming decode step (msgla_decode_step) against the
oracle's forward at the same positions.  The cache semantics follow the MS-GLA
notes' paragraph on token-by-token inference: pending partial blocks, held
outputs, and one recurrence step per completed block."""
import dataclasses

import numpy as np
import pytest

from oracle import msgla_oracle as orc
from scale_gla_layer_amd.config import WORKLOADS
from scale_gla_layer_amd.runner import DeviceLayer, from_device, read_state, to_device
from scale_gla_layer_amd.synth import make_inputs
from tests.gpu_cases import TOL, say

pytestmark = pytest.mark.gpu


def _decode_case(cfg, B, L0, n_dec, seed, batches=None):
    import torch
    say(f"decode scales={cfg.scales} heads={cfg.heads} {cfg.dtype} B={B} L0={L0} steps={n_dec}")
    X, W = make_inputs(cfg, B, L0 + n_dec, seed=seed)
    layer = DeviceLayer(cfg, W)
    st = layer.new_state(B)
    if L0 == 0:
        layer.state_init(st, B)
    else:
        layer.forward(to_device(X[:, :L0], cfg.dtype), state_out=st)
    outs = []
    for t in range(L0, L0 + n_dec):
        outs.append(from_device(layer.decode_step(to_device(X[:, t], cfg.dtype), st)))
    torch.cuda.synchronize()
    O_dec = np.stack(outs, axis=1)  # [B, n_dec, d]
    idx = list(range(B)) if batches is None else list(batches)
    ref = orc.layer_forward(X[idx], W, cfg)[:, L0:]
    err, zeros = orc.row_relative_error(O_dec[idx], ref)
    say(f"decode row-relative error {err:.3e}")
    assert zeros
    assert err <= TOL[cfg.dtype], err
    assert read_state(cfg, st, B)["pos"] == L0 + n_dec
    return err


@pytest.mark.parametrize("L0", [0, 1, 13, 37, 64])
def test_decode_tiny_fp32(L0):
    _decode_case(WORKLOADS["tiny_f32"].cfg, 2, L0, 20, seed=3)


def test_decode_bf16_narrow_model():
    """d = 64: the step's projection splits K into fewer slabs than waves."""
    from scale_gla_layer_amd.config import BF16, MsglaConfig
    cfg = MsglaConfig((1, 2), (1, 1), 64, 32, 64, 4, 32, 16.0, 1.0, BF16)
    _decode_case(cfg, 3, 9, 12, seed=6)


@pytest.mark.parametrize("name", ["main", "sweep_1248", "sweep_24"])
def test_decode_bf16_small(name):
    _decode_case(WORKLOADS[name].cfg, 2, 45, 24, seed=4)


@pytest.mark.parametrize("name", ["sweep_1248", "sweep_24"])
def test_decode_after_full_prefill(name):
    """Config of the wide sweep: B=16, prefill 4096 tokens, then 256 decode
    steps, every sequence against the oracle."""
    wl = WORKLOADS[name]
    _decode_case(wl.cfg, wl.batch, wl.seq_len, 256, seed=0)


def test_decode_graph_replays_match_eager_steps():
    """The step captured once as a HIP graph and replayed for 24 steps, with
    eager work and synchronisation between replays, gives bit-identical
    outputs and state to eager steps from the same prefilled state."""
    import torch
    from scale_gla_layer_amd.runner import DecodeGraph
    cfg = WORKLOADS["sweep_1248"].cfg
    B, L0, n = 2, 45, 24
    say(f"decode graph sweep_1248 B={B} L0={L0} steps={n}")
    X, W = make_inputs(cfg, B, L0 + n, seed=11)
    layer = DeviceLayer(cfg, W)
    st_e = layer.new_state(B)
    layer.forward(to_device(X[:, :L0], cfg.dtype), state_out=st_e)
    st_g = st_e.clone()
    xs = [to_device(np.ascontiguousarray(X[:, t]), cfg.dtype) for t in range(L0, L0 + n)]
    eager = [layer.decode_step(x, st_e).clone() for x in xs]
    g = DecodeGraph(layer, st_g, B)
    scratch = torch.zeros(1 << 20, device="cuda")
    for t, x in enumerate(xs):
        out = g.step(x)
        scratch.add_(1.0)  # the program's own eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager[t]), t
    assert torch.equal(st_g, st_e)
