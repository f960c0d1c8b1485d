"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded inputs, and compare."""
import sys

import numpy as np

from oracle import msgla_oracle as orc
from scale_gla_layer_amd.config import BF16, MsglaConfig
from scale_gla_layer_amd.runner import DeviceLayer, from_device, to_device
from scale_gla_layer_amd.synth import make_inputs

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(msg: str):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def mask_to_device(M: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(M, dtype=np.uint8)).to("cuda")


def run_device(cfg: MsglaConfig, X: np.ndarray, W, state_out=False, M=None):
    import torch
    layer = DeviceLayer(cfg, W)
    x = to_device(X, cfg.dtype)
    st = layer.new_state(X.shape[0]) if state_out else None
    out = layer.forward(x, state_out=st, mask=None if M is None else mask_to_device(M))
    torch.cuda.synchronize()
    return layer, x, out, st


def check_against_oracle(cfg, X, W, O_dev: np.ndarray, batches=None, tol=None, M=None):
    """Row-normalised max error vs the oracle on the sampled sequences."""
    tol = TOL[cfg.dtype] if tol is None else tol
    idx = list(range(X.shape[0])) if batches is None else list(batches)
    ref = orc.layer_forward(X[idx], W, cfg, M=None if M is None else M[idx])
    err, zeros_exact = orc.row_relative_error(O_dev[idx], ref)
    assert np.all(np.isfinite(O_dev[idx])), "non-finite output"
    assert zeros_exact, "rows the oracle gives as exactly zero are not zero on the device"
    say(f"row-relative error {err:.3e} (bar {tol:.0e}) on sequences {idx}")
    assert err <= tol, f"row-relative error {err:.3e} > {tol:.1e}"
    return err


def layer_case(cfg, B, L, seed=0, gate_bias=None, batches=None, tol=None):
    say(f"scales={cfg.scales} heads={cfg.heads} d={cfg.d_model} dk={cfg.d_k} dv={cfg.d_v} "
        f"C={cfg.chunk} {cfg.dtype} B={B} L={L} seed={seed} gate_bias={gate_bias}")
    X, W = make_inputs(cfg, B, L, seed=seed, gate_bias=gate_bias)
    _, _, out, _ = run_device(cfg, X, W)
    O = from_device(out)
    return check_against_oracle(cfg, X, W, O, batches=batches, tol=tol), X, W, O
