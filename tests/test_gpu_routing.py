"""GPU parity of msgla_fusion_weights (Eq. (10) alone) and of the routing-
stability procedure of Sec. 5.4 (mean fusion weights over the first, middle
and last tenth of the positions) applied to its output, against the fp64
oracle through the C ABI.

The weights come from bf16 (or fp32) inputs and weights with fp32 products
and sums and an fp32 softmax, and are returned in fp32, so both storage types
are held to 1e-4 row-relative (no bf16 rounding happens on this path)."""
import dataclasses

import numpy as np
import pytest

from oracle import msgla_oracle as orc
from scale_gla_layer_amd import binding
from scale_gla_layer_amd.config import WORKLOADS
from scale_gla_layer_amd.runner import DeviceLayer, from_device, to_device
from scale_gla_layer_amd.synth import make_inputs
from tests.gpu_cases import say

pytestmark = pytest.mark.gpu


def _weights(cfg, B, L, seed):
    import torch
    say(f"fusion weights scales={cfg.scales} d={cfg.d_model} {cfg.dtype} B={B} L={L} seed={seed}")
    X, W = make_inputs(cfg, B, L, seed=seed)
    layer = DeviceLayer(cfg, W)
    w = layer.fusion_weights(to_device(X, cfg.dtype))
    torch.cuda.synchronize()
    return X, W, from_device(w)


def _check(cfg, X, W, w_dev):
    m = len(cfg.scales)
    ref = orc.fusion_weights(X, W.W_f, W.b_f)
    err, _ = orc.row_relative_error(w_dev[..., :m], ref)
    say(f"row-relative error {err:.3e}")
    assert err <= 1e-4
    assert np.all(w_dev[..., m:] == 0.0)


@pytest.mark.parametrize("name,B,L", [("tiny_f32", 1, 64), ("tiny_f32", 3, 257), ("main", 2, 300),
                                      ("sweep_1248", 1, 1000)])
def test_fusion_weights_match_the_oracle(name, B, L):
    cfg = WORKLOADS[name].cfg
    X, W, w = _weights(cfg, B, L, seed=B + L)
    _check(cfg, X, W, w)


def test_routing_stability_of_a_32k_sequence():
    """The notes' setting: one 32,768-token sequence of the main configuration
    (synthetic weights, so the percentages are not the printed ones)."""
    cfg = WORKLOADS["main"].cfg
    X, W, w = _weights(cfg, 1, 32768, seed=3)
    _check(cfg, X, W, w)
    st_dev = orc.routing_stability(w[..., :3])
    st_ref = orc.routing_stability(orc.fusion_weights(X, W.W_f, W.b_f))
    say(f"regions (percent): {np.round(st_dev, 3).tolist()}")
    assert np.allclose(st_dev, st_ref, atol=1e-3)


def test_one_branch_has_no_fusion_weights():
    cfg = dataclasses.replace(WORKLOADS["tiny_f32"].cfg, scales=(1,), heads=(2,))
    X, W = make_inputs(cfg, 1, 16, seed=1)
    layer = DeviceLayer(cfg, W)
    with pytest.raises(binding.MsglaError):
        layer.fusion_weights(to_device(X, cfg.dtype))
