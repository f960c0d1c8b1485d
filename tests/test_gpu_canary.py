"""GPU: every buffer the library writes (workspace, output, state, decode
workspace and decode output) is passed with a guard band of a known byte
pattern on both sides; a masked forward with state export, a forward
continuing from that state and a few decode steps must leave every guard
byte untouched and give bit-identical results to the same calls on
unguarded buffers."""
import numpy as np
import pytest

from scale_gla_layer_amd import binding
from scale_gla_layer_amd.config import BF16, WORKLOADS
from scale_gla_layer_amd.runner import DeviceLayer, to_device
from scale_gla_layer_amd.synth import make_inputs, make_mask
from tests.gpu_cases import mask_to_device, say

pytestmark = pytest.mark.gpu

GUARD = 64 * 1024  # bytes on each side (keeps every view 256-byte aligned)


class Guarded:
    """A byte buffer of n bytes with a guard band of `fill` on both sides."""

    def __init__(self, n: int, fill: int):
        import torch
        self.n = n
        self.fill = fill
        self.raw = torch.full((n + 2 * GUARD,), fill, dtype=torch.uint8, device="cuda")
        self.body = self.raw[GUARD:GUARD + n]

    def intact(self) -> bool:
        import torch
        return bool(torch.all(self.raw[:GUARD] == self.fill)) and bool(
            torch.all(self.raw[GUARD + self.n:] == self.fill))


@pytest.mark.parametrize("name,B,L1,L2", [("tiny_f32", 3, 100, 36), ("main", 2, 300, 64)])
def test_calls_write_nothing_outside_their_buffers(name, B, L1, L2):
    import torch
    cfg = WORKLOADS[name].cfg
    dt = torch.bfloat16 if cfg.dtype == BF16 else torch.float32
    es = 2 if cfg.dtype == BF16 else 4
    d = cfg.d_model
    lcm = int(np.lcm.reduce(cfg.scales))
    L1 = L1 // lcm * lcm + 1  # the continuation starts one position into a block of every scale > 1
    X, W = make_inputs(cfg, B, L1 + L2 + 4, seed=41)
    M = make_mask(B, L1, seed=42, hole_prob=0.1)
    layer = DeviceLayer(cfg, W)
    say(f"canary {name} B={B} L={L1}+{L2} + 4 decode steps")

    def run(guarded: bool):
        bufs = []

        def buf(n, fill, dtype=torch.uint8, shape=(-1,)):
            if guarded:
                g = Guarded(n, fill)
                bufs.append(g)
                return g.body.view(dtype).view(shape)
            return torch.empty(n, dtype=torch.uint8, device="cuda").view(dtype).view(shape)

        st_bytes = binding.msgla_state_bytes(cfg, B)
        s1 = buf(st_bytes, 0x5A)
        s2 = buf(st_bytes, 0x3C)
        ws1 = buf(binding.msgla_workspace_bytes(cfg, B, L1), 0xA5)
        out1 = buf(B * L1 * d * es, 0x77, dt, (B, L1, d))
        x1 = to_device(X[:, :L1], cfg.dtype)
        binding.msgla_forward(cfg, layer.packed, x1, B, L1, out1, ws1, state_out=s1,
                              mask=mask_to_device(M))
        ws2 = buf(binding.msgla_workspace_bytes(cfg, B, L2), 0xA5)
        out2 = buf(B * L2 * d * es, 0x77, dt, (B, L2, d))
        x2 = to_device(X[:, L1:L1 + L2], cfg.dtype)
        binding.msgla_forward(cfg, layer.packed, x2, B, L2, out2, ws2, state_in=s1, state_out=s2)
        dws = buf(binding.msgla_decode_workspace_bytes(cfg, B), 0xC3)
        outs = []
        for t in range(4):
            o = buf(B * d * es, 0x77, dt, (B, d))
            xt = to_device(np.ascontiguousarray(X[:, L1 + L2 + t]), cfg.dtype)
            binding.msgla_decode_step(cfg, layer.packed, xt, B, s2, o, dws)
            outs.append(o)
        torch.cuda.synchronize()
        for i, g in enumerate(bufs):
            assert g.intact(), f"guard band of buffer {i} changed"
        return [out1.clone(), out2.clone()] + [o.clone() for o in outs]

    got = run(True)
    ref = run(False)
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
