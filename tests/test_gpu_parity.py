"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar: row-normalised max relative error max_t ||O_t - O*_t||_inf / ||O*_t||_inf
<= 1e-4 for the fp32 path and <= 2e-2 for bf16 storage with fp32 accumulation;
rows the oracle gives as exactly zero must be exactly zero.  Every case,
the full-size workloads included, compares every sequence of the batch."""
import dataclasses

import numpy as np
import pytest

from oracle import msgla_oracle as orc
from scale_gla_layer_amd.config import BF16, F32, MsglaConfig, WORKLOADS
from scale_gla_layer_amd.runner import from_device, to_device
from scale_gla_layer_amd.synth import make_inputs
from tests.gpu_cases import TOL, check_against_oracle, layer_case, run_device, say

pytestmark = pytest.mark.gpu


def _with(cfg, **kw):
    return dataclasses.replace(cfg, **kw)


TINY = WORKLOADS["tiny_f32"].cfg
MAIN = WORKLOADS["main"].cfg


# ------------------------------------------------------------------ fp32 path


def test_tiny_fp32_workload():
    wl = WORKLOADS["tiny_f32"]
    layer_case(wl.cfg, wl.batch, wl.seq_len, seed=0)


@pytest.mark.parametrize("L", [1, 2, 3, 5, 17, 50, 64, 100, 257])
def test_tiny_fp32_lengths(L):
    layer_case(TINY, 2, L, seed=1)


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_fp32_chunk_invariance(chunk):
    cfg = _with(TINY, chunk=chunk)
    layer_case(cfg, 2, 200, seed=2)


def test_fp32_wider_heads_and_ranks():
    cfg = MsglaConfig((1, 3, 8), (1, 2, 1), 128, 32, 64, 20, 32, 16.0, 1.0, F32)
    layer_case(cfg, 3, 150, seed=3)


@pytest.mark.parametrize("dk,chunk", [(128, 32), (256, 16), (64, 64)])
def test_fp32_key_width_at_the_lds_limit(dk, chunk):
    """Widest key widths whose chunk-state stages still fit one CU's LDS
    (d_k 128 at chunk 32 needs 156 KB; d_k 256 at chunk 16 drops to two stages)."""
    cfg = MsglaConfig((1, 2), (1, 1), 128, dk, 64, 8, chunk, 16.0, 1.0, F32)
    layer_case(cfg, 2, 100, seed=9)


def test_fp32_strong_and_weak_gates():
    """Gate bias -8 (fast decay, 16-step sub-block growth exercised) and +8 (alpha ~ 1)."""
    for lo, hi in ((-8.0, -8.0), (8.0, 8.0), (-8.0, 8.0)):
        layer_case(TINY, 2, 130, seed=4, gate_bias=(lo, hi))


@pytest.mark.parametrize("gamma,bias", [
    (1.0, (-8.0, -8.0)),       # ~11.5 log2 units of decay per position
    (16.0, (-100.0, -100.0)),  # ~9 log2 units per position
    (16.0, (-100.0, 8.0)),     # channels from near-total decay to alpha ~ 1
    (1.0, (-30.0, -2.0)),
])
@pytest.mark.parametrize("chunk", [16, 64])
def test_fp32_decay_beyond_the_fast_diagonal(gamma, bias, chunk):
    """Gates whose 16-position tiles decay by far more than 2^-32 (the chunk
    kernel then forms each diagonal block pair by pair; a block factored
    through its first position would overflow fp32): finite, and within the
    bar.  Chunk 64 also covers the off-diagonal blocks between such tiles."""
    cfg = _with(TINY, gate_normalizer=gamma, chunk=chunk)
    layer_case(cfg, 2, 150, seed=21, gate_bias=bias)


# ------------------------------------------------------------------ bf16, small


def test_bf16_ragged_main_dims():
    """Main dimensions, a few chunks per branch with ragged tails and ragged GEMM tiles."""
    layer_case(MAIN, 2, 300, seed=1)


@pytest.mark.parametrize("L", [1, 3, 4, 7, 65, 129])
def test_bf16_short_sequences(L):
    layer_case(MAIN, 1, L, seed=5)


def test_bf16_chunk32():
    layer_case(_with(MAIN, chunk=32), 2, 200, seed=6)


@pytest.mark.parametrize("dk,chunk", [(256, 32), (64, 64), (32, 32)])
def test_bf16_key_widths(dk, chunk):
    """Other key widths, including d_k 256 (chunk 32: 144 KB of state-kernel stages)."""
    cfg = MsglaConfig((1, 2, 4), (1, 1, 1), 256, dk, 128, 16, chunk, 16.0, 1.0, BF16)
    layer_case(cfg, 2, 200, seed=10)


def test_bf16_no_fine_branch_first_row_zero():
    cfg = WORKLOADS["sweep_24"].cfg
    err, X, W, O = layer_case(cfg, 2, 130, seed=7)
    assert np.array_equal(O[:, 0], np.zeros_like(O[:, 0]))


def test_bf16_adversarial_gates():
    for gb in ((-8.0, -8.0), (8.0, 8.0), (-8.0, 8.0)):
        layer_case(MAIN, 1, 200, seed=8, gate_bias=gb)


@pytest.mark.parametrize("gamma,bias", [
    (1.0, (-8.0, -8.0)),
    (16.0, (-100.0, -100.0)),
    (16.0, (-100.0, 8.0)),
])
def test_bf16_decay_beyond_the_fast_diagonal(gamma, bias):
    """The strong-decay gates at the main dimensions (chunk 64, four tiles per
    chunk) on the bf16 path."""
    layer_case(_with(MAIN, gate_normalizer=gamma), 2, 200, seed=22, gate_bias=bias)


# ------------------------------------------------------------------ full-size workloads


@pytest.mark.parametrize("name", ["main", "gla_baseline", "long", "sweep_1248", "sweep_24"])
def test_full_size_workload(name):
    """Every sequence of the workload against the oracle (the device runs the
    whole batch in the benchmark's launch configuration)."""
    wl = WORKLOADS[name]
    layer_case(wl.cfg, wl.batch, wl.seq_len, seed=0, gate_bias=wl.gate_bias)


# ------------------------------------------------------------------ properties


def test_causality_on_device_is_bit_exact():
    cfg = MAIN
    X, W = make_inputs(cfg, 2, 260, seed=11)
    say("causality main dims B=2 L=260")
    _, _, out, _ = run_device(cfg, X, W)
    O = from_device(out)
    for t0 in (0, 63, 64, 130, 200):
        X2 = X.copy()
        X2[:, t0 + 1:] = make_inputs(cfg, 2, 260, seed=100 + t0)[0][:, t0 + 1:]
        _, _, out2, _ = run_device(cfg, X2, W)
        O2 = from_device(out2)
        assert np.array_equal(O[:, : t0 + 1], O2[:, : t0 + 1]), t0
        assert not np.array_equal(O[:, t0 + 1:], O2[:, t0 + 1:])


def test_repeat_runs_are_bitwise_identical():
    import torch
    wl = WORKLOADS["main"]
    X, W = make_inputs(wl.cfg, 2, 1024, seed=12)
    say("determinism main dims B=2 L=1024")
    layer, x, out, _ = run_device(wl.cfg, X, W)
    first = out.clone()
    for _ in range(3):
        layer.forward(x, out=out)
        torch.cuda.synchronize()
        assert torch.equal(first, out)


def test_exported_state_matches_oracle():
    cfg = _with(TINY)
    for L in (37, 64, 3, 600):  # 600: the chunk-state walk runs in segments
        X, W = make_inputs(cfg, 2, L, seed=13)
        say(f"state export tiny L={L}")
        layer, x, out, st = run_device(cfg, X, W, state_out=True)
        from scale_gla_layer_amd.runner import read_state
        dev = read_state(cfg, st, 2)
        _, ref = orc.layer_forward(X, W, cfg, return_state=True)
        assert dev["pos"] == L and dev["B"] == 2 and dev["m"] == 3
        for i, (bd, br) in enumerate(zip(dev["branches"], ref["branches"])):
            for key in ("S", "psum", "held"):
                a, b = bd[key], br[key]
                scale = max(1e-30, np.abs(b).max())
                assert np.abs(a - b).max() <= 1e-4 * scale + 1e-12, (L, i, key)
