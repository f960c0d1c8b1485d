"""Device-memory plumbing around the C ABI: uploads synthetic inputs and
weights with torch, packs the weights once, owns the workspace, and calls the
binding.  No arithmetic of the layer happens here."""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import binding
from .config import BF16, MsglaConfig
from .synth import LayerWeights, storage_array


def _torch():
    import torch
    return torch


def to_device(a: np.ndarray, dtype: str, device="cuda"):
    """Host float64 array (already rounded) -> device tensor in the storage type."""
    torch = _torch()
    host = storage_array(a, dtype)
    if dtype == BF16:
        t = torch.from_numpy(host.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(host.copy())
    return t.to(device)


def to_device_f32(a: np.ndarray, device="cuda"):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def from_device(t) -> np.ndarray:
    torch = _torch()
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def empty_bytes(n: int, device="cuda"):
    torch = _torch()
    return torch.empty(max(int(n), 16), dtype=torch.uint8, device=device)


class DeviceLayer:
    """Packed weights + workspace for one configuration on one device."""

    def __init__(self, cfg: MsglaConfig, W: LayerWeights, device="cuda", stream=None):
        torch = _torch()
        self.cfg, self.device, self.stream = cfg, device, stream
        dt = cfg.dtype
        self._src = []
        for bw in W.branches:
            self._src.append({
                "W_q": to_device(bw.W_q, dt, device), "W_k": to_device(bw.W_k, dt, device),
                "W_v": to_device(bw.W_v, dt, device), "W_g1": to_device(bw.W_g1, dt, device),
                "W_g2": to_device(bw.W_g2, dt, device), "b_g": to_device_f32(bw.b_g, device),
                "W_o": to_device(bw.W_o, dt, device),
                "norm_g": to_device_f32(bw.g_norm, device) if cfg.norm else None})
        m = len(cfg.scales)
        self._W_f = to_device(W.W_f, dt, device) if m > 1 else None
        self._b_f = to_device_f32(W.b_f, device) if m > 1 else None
        nbytes = binding.msgla_packed_weights_bytes(cfg)
        if nbytes == 0:
            raise ValueError("invalid configuration for the library")
        self.packed = empty_bytes(nbytes, device)
        binding.msgla_pack_weights(cfg, self._src, self._W_f, self._b_f, self.packed, stream)
        torch.cuda.synchronize()
        self._src = None  # the packed blob is all the kernels read
        self._W_f = self._b_f = None
        self.workspace = None
        self.dec_workspace = None
        self.bwd_workspace = None

    def ensure_workspace(self, B: int, L: int):
        n = binding.msgla_workspace_bytes(self.cfg, B, L)
        if n == 0:
            raise ValueError(f"invalid batch/length B={B} L={L}")
        if self.workspace is None or self.workspace.numel() < n:
            self.workspace = empty_bytes(n, self.device)
        return self.workspace

    def new_output(self, B: int, L: int):
        torch = _torch()
        dt = torch.bfloat16 if self.cfg.dtype == BF16 else torch.float32
        return torch.empty((B, L, self.cfg.d_model), dtype=dt, device=self.device)

    def new_state(self, B: int):
        return empty_bytes(binding.msgla_state_bytes(self.cfg, B), self.device)

    def forward(self, x, out=None, state_out=None, events=None, state_in=None, mask=None):
        B, L, _ = x.shape
        ws = self.ensure_workspace(B, L)
        if out is None:
            out = self.new_output(B, L)
        binding.msgla_forward(self.cfg, self.packed, x, B, L, out, ws, state_out=state_out,
                              state_in=state_in, mask=mask, stream=self.stream, events=events)
        return out

    def new_grads(self):
        """fp32 gradient tensors shaped as the weights ([in][out]); (branch dicts, W_f, b_f)."""
        torch = _torch()
        c = self.cfg
        d, dk, dv, r = c.d_model, c.d_k, c.d_v, c.gate_rank
        z = lambda *shape: torch.empty(shape, dtype=torch.float32, device=self.device)
        brs = [{"W_q": z(d, h * dk), "W_k": z(d, h * dk), "W_v": z(d, h * dv), "W_g1": z(d, r),
                "W_g2": z(r, h * dk), "b_g": z(h * dk), "W_o": z(h * dv, d)} for h in c.heads]
        if c.norm:
            for br, h in zip(brs, c.heads):
                br["norm_g"] = z(h * dv)
        m = len(c.scales)
        return brs, (z(d, m) if m > 1 else None), (z(m) if m > 1 else None)

    def ensure_bwd_workspace(self, B: int, L: int):
        n = binding.msgla_backward_workspace_bytes(self.cfg, B, L)
        if n == 0:
            raise ValueError(f"the backward does not support this configuration or size (B={B} L={L})")
        if self.bwd_workspace is None or self.bwd_workspace.numel() < n:
            self.bwd_workspace = empty_bytes(n, self.device)
        return self.bwd_workspace

    def forward_train(self, x, out=None, mask=None):
        """The training forward: the forward's output, with the backward's intermediates kept
        in the backward workspace for backward(..., saved=True)."""
        B, L, _ = x.shape
        ws = self.ensure_bwd_workspace(B, L)
        if out is None:
            out = self.new_output(B, L)
        binding.msgla_forward_train(self.cfg, self.packed, x, B, L, out, ws, mask=mask, stream=self.stream)
        return out

    def backward(self, x, dout, dx=None, grads=None, mask=None, saved=False):
        """Layer backward of a fresh-state forward of x (with the forward's token mask, if
        any): returns (dx, (branch grads, dW_f, db_f)).  saved: read the intermediates of
        the preceding forward_train of the same x (and mask) instead of recomputing them."""
        B, L, _ = x.shape
        ws = self.ensure_bwd_workspace(B, L)
        if dx is None:
            dx = self.new_output(B, L)
        if grads is None:
            grads = self.new_grads()
        binding.msgla_backward(self.cfg, self.packed, x, dout, B, L, dx, grads[0], grads[1], grads[2],
                               ws, mask=mask, stream=self.stream, saved=saved)
        return dx, grads

    def state_init(self, state, B: int):
        binding.msgla_state_init(self.cfg, B, state, self.stream)

    def fusion_weights(self, x, w_out=None):
        """Fusion weights [B, L, 8] fp32 (first n_branches entries) from the library."""
        torch = _torch()
        B, L, _ = x.shape
        if w_out is None:
            w_out = torch.empty((B, L, 8), dtype=torch.float32, device=self.device)
        binding.msgla_fusion_weights(self.cfg, self.packed, x, B, L, w_out, self.stream)
        return w_out

    def ensure_dec_workspace(self, B: int):
        n = binding.msgla_decode_workspace_bytes(self.cfg, B)
        if self.dec_workspace is None or self.dec_workspace.numel() < n:
            self.dec_workspace = empty_bytes(n, self.device)
        return self.dec_workspace

    def decode_step(self, x_t, state, out_t=None):
        torch = _torch()
        B = x_t.shape[0]
        self.ensure_dec_workspace(B)
        if out_t is None:
            dt = torch.bfloat16 if self.cfg.dtype == BF16 else torch.float32
            out_t = torch.empty((B, self.cfg.d_model), dtype=dt, device=self.device)
        binding.msgla_decode_step(self.cfg, self.packed, x_t, B, state, out_t, self.dec_workspace,
                                  self.stream)
        return out_t


class DecodeGraph:
    """One streaming step (msgla_decode_step) captured once as a HIP graph.

    The step takes its position from the state on the device and allocates
    nothing, so one graph serves every later step of the same state: step()
    copies the token into the captured input buffer and replays the graph.
    Capturing enqueues nothing; the state advances only on replay."""

    def __init__(self, layer: "DeviceLayer", state, B: int):
        torch = _torch()
        dt = torch.bfloat16 if layer.cfg.dtype == BF16 else torch.float32
        self.x = torch.zeros((B, layer.cfg.d_model), dtype=dt, device=layer.device)
        self.out = torch.empty_like(self.x)
        ws = layer.ensure_dec_workspace(B)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            binding.msgla_decode_step(layer.cfg, layer.packed, self.x, B, state, self.out, ws)

    def step(self, x_t):
        self.x.copy_(x_t)
        self.graph.replay()
        return self.out


def read_state(cfg: MsglaConfig, state, B: int) -> dict:
    """Decode a state blob (device tensor) into numpy arrays, mirroring the
    layout documented in include/msgla.h (header + per-branch S, psum, held,
    pending token count)."""
    raw = state.detach().cpu().numpy()
    hdr = raw[:24].view(np.int32)
    pos = int(raw[16:24].view(np.int64)[0])
    cur = 256
    align = lambda x: (x + 255) & ~255
    out = {"magic": int(hdr[0]) & 0xffffffff, "version": int(hdr[1]), "B": int(hdr[2]),
           "m": int(hdr[3]), "pos": pos, "branches": []}
    for h in cfg.heads:
        nS = B * h * cfg.d_k * cfg.d_v
        S = raw[cur: cur + 4 * nS].view(np.float32).reshape(B, h, cfg.d_k, cfg.d_v)
        cur += align(4 * nS)
        psum = raw[cur: cur + 4 * B * cfg.d_model].view(np.float32).reshape(B, cfg.d_model)
        cur += align(4 * B * cfg.d_model)
        held = raw[cur: cur + 4 * B * cfg.d_model].view(np.float32).reshape(B, cfg.d_model)
        cur += align(4 * B * cfg.d_model)
        tok = raw[cur: cur + 4 * B].view(np.float32)
        cur += align(4 * B)
        out["branches"].append({"S": S.astype(np.float64), "psum": psum.astype(np.float64),
                                "held": held.astype(np.float64), "tokens": tok.astype(np.float64)})
    return out
