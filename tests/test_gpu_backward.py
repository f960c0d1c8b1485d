"""GPU: the layer backward (msgla_backward through the C ABI) against the fp64
oracle's vector-Jacobian product (oracle.layer_backward, itself pinned by
finite differences of the pinned forward).

Every gradient is compared in full: dx per row (against the larger of the row's
norm and the magnitude of its fusion-logit term before cancellation, see
dx_error), each weight gradient as a whole (max |device - oracle| over
max |oracle|), at the forward's bars (1e-4 fp32, 2e-2 bf16).  The cases cover
several chunks with a ragged last chunk in every branch, tail positions past a
coarse branch's last complete block, chunks 16, 32 and 64 (bf16: 32 and 64, key widths
32 to 256), q_scale and gamma
off their defaults, strong gates, a scale set without a scale-1 branch, a
single branch (no fusion), a branch whose scale exceeds the sequence, sequences
shorter than a chunk (down to one position, where no coarse branch or, at scales
{2, 4}, no branch at all has a complete block), and the
main configuration's dimensions in bf16, and the full main workload (B = 8,
L = 2048)."""
import dataclasses

import numpy as np
import pytest

from oracle import msgla_oracle as orc
from scale_gla_layer_amd.config import BF16, F32, WORKLOADS, MsglaConfig
from scale_gla_layer_amd.runner import DeviceLayer, from_device, to_device
from scale_gla_layer_amd.synth import make_inputs, round_to
from scale_gla_layer_amd.synth import make_mask
from tests.gpu_cases import TOL, mask_to_device, say

pytestmark = pytest.mark.gpu

KEYS = ("W_q", "W_k", "W_v", "W_g1", "W_g2", "b_g", "W_o")


def dx_error(dX, dX_ref, X, W, cfg, dO, M=None):
    """Row error of dx: max_t ||dX_t - ref_t||_inf / max(||ref_t||_inf, ||dxbar_t||_inf).

    dxbar_t bounds the fusion logits' part of row t before cancellation:
    dxbar_t = (w_t * (dwbar_t + w_t . dwbar_t)) |W_f|^T with
    dwbar_{t,i} = sum_c |dO_tc Yhat^(i)_tc|.  The fusion logits' gradient dw is a
    d-term dot product of dO with the held outputs, which the bf16 layer stores
    in bf16 (a rounding of the layer itself), so its error scales with the sum
    of the terms' magnitudes, not with the possibly cancelling sum.  At a masked
    position x_t enters only through the fusion logits, and that row of dx is
    that term alone; everywhere else the pooled terms dominate both norms."""
    den = np.abs(dX_ref).max(axis=-1)
    m = len(cfg.scales)
    if m > 1:
        B, L, d = X.shape
        w = orc.fusion_weights(X, W.W_f, W.b_f)
        dwbar = np.zeros((B, L, m))
        for i, (s, bw) in enumerate(zip(cfg.scales, W.branches)):
            Y, _, _ = orc.branch_forward(X, bw, s, cfg, M)
            dwbar[:, :, i] = np.sum(np.abs(dO * orc.causal_hold(Y, s, L)), axis=-1)
        dzbar = w * (dwbar + np.sum(w * dwbar, axis=-1, keepdims=True))
        den = np.maximum(den, np.abs(dzbar @ np.abs(W.W_f).T).max(axis=-1))
    num = np.abs(dX - dX_ref).max(axis=-1)
    nz = den > 0
    assert np.all(num[~nz] == 0), "rows the oracle gives as exactly zero are not zero"
    return float((num[nz] / den[nz]).max()) if nz.any() else 0.0


def _tensor_err(got, ref):
    den = float(np.abs(ref).max())
    if den == 0.0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max()) / den


def backward_case(cfg, B, L, seed=0, gate_bias=None, tol=None, M=None):
    import torch
    tol = TOL[cfg.dtype] if tol is None else tol
    say(f"backward scales={cfg.scales} heads={cfg.heads} d={cfg.d_model} dk={cfg.d_k} dv={cfg.d_v} "
        f"r={cfg.gate_rank} C={cfg.chunk} gamma={cfg.gate_normalizer} q_scale={cfg.q_scale} "
        f"{cfg.dtype} B={B} L={L} seed={seed} gate_bias={gate_bias} masked={M is not None}")
    X, W = make_inputs(cfg, B, L, seed=seed, gate_bias=gate_bias)
    dO = round_to(np.random.default_rng(seed + 1000).normal(0.0, 1.0, X.shape), cfg.dtype)
    layer = DeviceLayer(cfg, W)
    x = to_device(X, cfg.dtype)
    dout = to_device(dO, cfg.dtype)
    dx, (gb, gWf, gbf) = layer.backward(x, dout, mask=None if M is None else mask_to_device(M))
    torch.cuda.synchronize()
    dX_ref, ref = orc.layer_backward(X, W, cfg, dO, M=M)
    errs = {}
    dX = from_device(dx)
    assert np.all(np.isfinite(dX)), "non-finite dx"
    errs["dx"] = dx_error(dX, dX_ref, X, W, cfg, dO, M)
    for i, g in enumerate(gb):
        for key in KEYS + (("norm_g",) if cfg.norm else ()):
            got = from_device(g[key])
            assert np.all(np.isfinite(got)), f"non-finite br{i}.{key}"
            errs[f"br{i}.{key}"] = _tensor_err(got, ref["branches"][i]["g_norm" if key == "norm_g" else key])
    if cfg.n_branches > 1:
        errs["W_f"] = _tensor_err(from_device(gWf), ref["W_f"])
        errs["b_f"] = _tensor_err(from_device(gbf), ref["b_f"])
    worst = max(errs, key=errs.get)
    say("errors " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert errs[worst] <= tol, f"{worst}: {errs[worst]:.3e} > {tol:.1e}"
    return errs


def _cfg(**kw):
    base = dict(scales=(1, 2, 4), heads=(2, 1, 1), d_model=64, d_k=32, d_v=64, gate_rank=8, chunk=16,
                gate_normalizer=16.0, q_scale=1.0, dtype=F32)
    base.update(kw)
    return MsglaConfig(**base)


def test_fp32_small():
    backward_case(_cfg(), B=2, L=100)


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_fp32_chunks(chunk):
    backward_case(_cfg(chunk=chunk, scales=(1, 3, 5), heads=(1, 2, 1)), B=2, L=150, seed=3)


def test_fp32_scaled_queries_and_strong_gates():
    backward_case(_cfg(q_scale=0.7, gate_normalizer=2.0, d_k=16), B=3, L=77, seed=5, gate_bias=(-4.0, 2.0))


def test_fp32_no_scale_one_branch():
    backward_case(_cfg(scales=(2, 4), heads=(1, 2)), B=2, L=90, seed=7)


def test_fp32_single_branch():
    backward_case(_cfg(scales=(1,), heads=(3,), d_k=64, gate_rank=20), B=2, L=70, seed=9)


def test_fp32_scale_longer_than_sequence():
    """The scale-8 branch has no complete block: zero gradients for its weights."""
    backward_case(_cfg(scales=(1, 8), heads=(1, 1)), B=2, L=7, seed=11)


@pytest.mark.parametrize("L", [1, 3, 5])
def test_bf16_main_dimensions_short_sequences(L):
    """Fewer positions than a chunk: at L = 1 the coarse branches have no complete
    block, at 3 the scale-2 branch has one, at 5 the scale-4 branch has one."""
    backward_case(WORKLOADS["main"].cfg, B=3, L=L, seed=61 + L)


def test_bf16_no_complete_block_in_any_branch():
    """Every branch's scale exceeds the sequence: the output is zero, so dx and every
    gradient are exactly zero (dx_error requires exact zeros where the oracle's are)."""
    cfg = _cfg(dtype=BF16, scales=(2, 4), heads=(1, 2), d_model=128, d_v=64, chunk=32)
    errs = backward_case(cfg, B=2, L=1, seed=67)
    assert all(v == 0.0 for v in errs.values()), errs


def test_fp32_single_position():
    backward_case(_cfg(), B=2, L=1, seed=71)


def test_fp32_key_width_128_rank_64():
    backward_case(_cfg(d_model=128, d_k=128, d_v=128, gate_rank=40, chunk=32), B=1, L=96, seed=13)


def test_bf16_main_dimensions():
    cfg = WORKLOADS["main"].cfg
    backward_case(cfg, B=2, L=320, seed=17)


@pytest.mark.parametrize("dk,dv,chunk,r,d", [(32, 64, 32, 8, 64), (64, 128, 64, 20, 128), (256, 64, 32, 8, 128)])
def test_bf16_other_key_widths_and_chunks(dk, dv, chunk, r, d):
    """bf16 storage at the other key widths, a chunk of 32 (tiles with rows past the
    chunk), a rank above 16 and a ragged last chunk in every branch."""
    cfg = _cfg(dtype=BF16, d_model=d, d_k=dk, d_v=dv, chunk=chunk, gate_rank=r, scales=(1, 2, 3), heads=(1, 2, 1))
    backward_case(cfg, B=2, L=150, seed=43 + dk)


def test_bf16_sweep_dimensions_with_gate_bias():
    cfg = dataclasses.replace(WORKLOADS["sweep_1248"].cfg)
    backward_case(cfg, B=1, L=264, seed=19, gate_bias=(1.0, 4.0))


@pytest.mark.parametrize("scales,heads", [((1, 3, 4), (2, 1, 1)), ((2, 4), (1, 2))])
def test_fp32_masked(scales, heads):
    """Holes anywhere (the first positions included), a fully padded sequence."""
    B, L = 3, 133
    M = make_mask(B, L, seed=29, hole_prob=0.15)
    M[2] = 0
    backward_case(_cfg(scales=scales, heads=heads), B=B, L=L, seed=29, M=M)


def test_bf16_main_dimensions_masked():
    B, L = 2, 320
    backward_case(WORKLOADS["main"].cfg, B=B, L=L, seed=31, M=make_mask(B, L, seed=31, hole_prob=0.1))


def test_fp32_normalised():
    """The per-head RMS normalisation before W_o, with its gains' gradient."""
    backward_case(_cfg(norm=True, scales=(1, 2, 3), heads=(1, 2, 1)), B=2, L=101, seed=37)


def test_fp32_normalised_and_masked():
    """The normalisation with the token mask: a masked scale-1 position has o = 0 and
    r = sqrt(eps), so its dLoss/do is large; every term it enters must carry q = 0."""
    B, L = 2, 133
    M = make_mask(B, L, seed=47, hole_prob=0.15)
    backward_case(_cfg(norm=True, scales=(1, 2, 3), heads=(1, 2, 1)), B=B, L=L, seed=47, M=M)


def test_bf16_main_dimensions_normalised_and_masked():
    B, L = 2, 200
    cfg = dataclasses.replace(WORKLOADS["main"].cfg, norm=True)
    backward_case(cfg, B=B, L=L, seed=41, M=make_mask(B, L, seed=41, hole_prob=0.1))


def test_bf16_weight_gradient_slices_with_a_ragged_step():
    """B = 3, L = 2731 at the main dimensions: the scale-1 branch's weight gradients
    reduce over 8193 positions, cut into two slices of which the second ends 1 position
    into a 32-position step (the step's other positions zeroed in the operands); the
    coarse branches reduce over 4095 and 2046 positions in one slice each."""
    backward_case(WORKLOADS["main"].cfg, B=3, L=2731, seed=47)


def test_bf16_full_size_main_workload():
    """The main workload at its full size (B = 8, L = 2048): every gradient against the
    oracle, which runs sequence by sequence (a weight gradient is the sum of the
    sequences' gradients; dx of a sequence depends on that sequence only)."""
    import torch
    wl = WORKLOADS["main"]
    cfg, B, L = wl.cfg, wl.batch, wl.seq_len
    say(f"backward full size main B={B} L={L}")
    X, W = make_inputs(cfg, B, L, seed=23)
    dO = round_to(np.random.default_rng(24).normal(0.0, 1.0, X.shape), cfg.dtype)
    layer = DeviceLayer(cfg, W)
    dx, (gb, gWf, gbf) = layer.backward(to_device(X, cfg.dtype), to_device(dO, cfg.dtype))
    torch.cuda.synchronize()
    dX = from_device(dx)
    got = {f"br{i}.{k}": from_device(g[k]) for i, g in enumerate(gb) for k in KEYS}
    got["W_f"], got["b_f"] = from_device(gWf), from_device(gbf)
    ref = {k: np.zeros_like(v, dtype=np.float64) for k, v in got.items()}
    dx_err = 0.0
    for b in range(B):
        dXb, rb = orc.layer_backward(X[b:b + 1], W, cfg, dO[b:b + 1])
        dx_err = max(dx_err, dx_error(dX[b:b + 1], dXb, X[b:b + 1], W, cfg, dO[b:b + 1]))
        for i, g in enumerate(rb["branches"]):
            for k in KEYS:
                ref[f"br{i}.{k}"] += g[k]
        ref["W_f"] += rb["W_f"]
        ref["b_f"] += rb["b_f"]
        say(f"sequence {b}: dx row-relative error so far {dx_err:.2e}")
    errs = {"dx": dx_err}
    for k in got:
        assert np.all(np.isfinite(got[k])), k
        errs[k] = _tensor_err(got[k], ref[k])
    say("errors " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    worst = max(errs, key=errs.get)
    assert errs[worst] <= TOL[cfg.dtype], f"{worst}: {errs[worst]:.3e}"


@pytest.mark.parametrize("case", ["bf16_masked", "bf16_normalised", "fp32"])
def test_saved_backward_matches_recompute(case):
    """msgla_forward_train writes msgla_forward's output bit for bit, and msgla_backward_saved
    after it returns msgla_backward's gradients bit for bit; a second saved backward with
    another dO (the saved intermediates unchanged by the first) matches that dO's
    recomputing backward."""
    import torch
    if case == "fp32":
        cfg, B, L, M = _cfg(), 2, 100, None
    else:
        cfg = dataclasses.replace(WORKLOADS["main"].cfg, norm=case == "bf16_normalised")
        B, L = 2, 200
        M = make_mask(B, L, seed=53, hole_prob=0.1) if case == "bf16_masked" else None
    say(f"saved backward {case} B={B} L={L}")
    X, W = make_inputs(cfg, B, L, seed=53)
    rng = np.random.default_rng(54)
    dO1, dO2 = (round_to(rng.normal(0.0, 1.0, X.shape), cfg.dtype) for _ in range(2))
    layer = DeviceLayer(cfg, W)
    x = to_device(X, cfg.dtype)
    m = None if M is None else mask_to_device(M)
    d1, d2 = to_device(dO1, cfg.dtype), to_device(dO2, cfg.dtype)

    def grads_of(res):
        dx, (gb, gWf, gbf) = res
        ts = [dx] + [g[k] for g in gb for k in sorted(g)] + [t for t in (gWf, gbf) if t is not None]
        return [t.clone() for t in ts]

    def same(a, b, what):
        for i, (u, v) in enumerate(zip(a, b)):
            assert torch.equal(u, v), f"{what}: tensor {i} differs"

    out_ref = layer.forward(x, mask=m).clone()
    ref1 = grads_of(layer.backward(x, d1, mask=m))
    ref2 = grads_of(layer.backward(x, d2, mask=m))
    out = layer.forward_train(x, mask=m)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref), "training forward output differs from the forward's"
    same(grads_of(layer.backward(x, d1, mask=m, saved=True)), ref1, "saved backward, first dO")
    same(grads_of(layer.backward(x, d2, mask=m, saved=True)), ref2, "saved backward, second dO")
    torch.cuda.synchronize()
