"""GPU parity with the optional per-head RMS normalisation of each branch's
output (configuration flag norm; the notes name a per-branch normalisation
without its form, see the header), against the fp64 oracle through the C ABI:
forward, streaming decode and continuation from a state.  Same bars as the
other parity tests (1e-4 fp32, 2e-2 bf16, exact zero rows)."""
import dataclasses

import numpy as np
import pytest

from oracle import msgla_oracle as orc
from scale_gla_layer_amd.config import WORKLOADS
from scale_gla_layer_amd.runner import DeviceLayer, from_device, to_device
from scale_gla_layer_amd.synth import make_inputs
from tests.gpu_cases import TOL, layer_case, say

pytestmark = pytest.mark.gpu


def _n(name, **kw):
    return dataclasses.replace(WORKLOADS[name].cfg, norm=True, **kw)


@pytest.mark.parametrize("L", [1, 17, 64, 257])
def test_tiny_fp32_normalised(L):
    layer_case(_n("tiny_f32"), 2, L, seed=L)


def test_fp32_normalised_wide_values():
    layer_case(_n("tiny_f32", d_v=512), 2, 70, seed=5)


def test_bf16_normalised_main_dims():
    layer_case(_n("main"), 2, 300, seed=6)


def test_bf16_normalised_full_size():
    wl = WORKLOADS["main"]
    layer_case(_n("main"), wl.batch, wl.seq_len, seed=7)


@pytest.mark.parametrize("name,L0", [("tiny_f32", 13), ("sweep_1248", 45)])
def test_normalised_decode(name, L0):
    import torch
    cfg = _n(name)
    B, n_dec = 2, 20
    say(f"normalised decode {name} L0={L0}")
    X, W = make_inputs(cfg, B, L0 + n_dec, seed=8)
    layer = DeviceLayer(cfg, W)
    st = layer.new_state(B)
    layer.forward(to_device(X[:, :L0], cfg.dtype), state_out=st)
    outs = [from_device(layer.decode_step(to_device(X[:, t], cfg.dtype), st))
            for t in range(L0, L0 + n_dec)]
    torch.cuda.synchronize()
    ref = orc.layer_forward(X, W, cfg)[:, L0:]
    err, zeros = orc.row_relative_error(np.stack(outs, axis=1), ref)
    say(f"row-relative error {err:.3e}")
    assert zeros and err <= TOL[cfg.dtype]


def test_normalised_continuation_from_a_state():
    import torch
    cfg = _n("tiny_f32")
    B, L1, L2 = 2, 32, 40
    X, W = make_inputs(cfg, B, L1 + L2, seed=9)
    layer = DeviceLayer(cfg, W)
    st = layer.new_state(B)
    layer.forward(to_device(X[:, :L1], cfg.dtype), state_out=st)
    out2 = layer.forward(to_device(X[:, L1:], cfg.dtype), state_in=st)
    torch.cuda.synchronize()
    ref = orc.layer_forward(X, W, cfg)[:, L1:]
    err, zeros = orc.row_relative_error(from_device(out2), ref)
    say(f"row-relative error {err:.3e}")
    assert zeros and err <= TOL[cfg.dtype]
