"""Pins of the oracle's layer backward (CPU only).

The backward is the vector-Jacobian product of the oracle's forward, which
the other oracle pins fix.  Here every gradient the backward returns (dX and
every weight of every branch, the fusion logits' W_f and b_f, the
normalisation gains) is compared element by element with central finite
differences of the forward's loss sum(dO * O) in fp64, on small
configurations that have a tail block in every coarse branch, several heads,
q_scale and gamma off their defaults and gates far from saturation.  A
dropped or doubled term, a wrong sign, index or transpose anywhere in the
chain rule moves some gradient by far more than the differences' error; the
planted-mistake tests show that for three such mistakes.
"""
import dataclasses

import numpy as np
import pytest

from oracle import msgla_oracle as orc
from scale_gla_layer_amd.config import F32, MsglaConfig
from scale_gla_layer_amd.synth import BranchWeights, LayerWeights

EPS = 1e-6


def _config(norm=False, scales=(1, 2, 3), heads=(1, 2, 1)):
    return MsglaConfig(tuple(scales), tuple(heads), d_model=5, d_k=3, d_v=2, gate_rank=2, chunk=16,
                       gate_normalizer=1.7, q_scale=0.8, dtype=F32, norm=norm)


def _weights(cfg, rng):
    d, dk, dv, r = cfg.d_model, cfg.d_k, cfg.d_v, cfg.gate_rank
    brs = []
    for h in cfg.heads:
        brs.append(BranchWeights(
            W_q=rng.normal(0, 0.5, (d, h * dk)), W_k=rng.normal(0, 0.5, (d, h * dk)),
            W_v=rng.normal(0, 0.5, (d, h * dv)), W_g1=rng.normal(0, 0.5, (d, r)),
            W_g2=rng.normal(0, 0.5, (r, h * dk)), b_g=rng.normal(1.0, 0.5, h * dk),
            W_o=rng.normal(0, 0.5, (h * dv, d)),
            g_norm=rng.normal(1.0, 0.2, h * dv) if cfg.norm else None))
    m = cfg.n_branches
    return LayerWeights(brs, rng.normal(0, 0.5, (d, m)), rng.normal(0, 0.5, m))


def _loss(X, W, cfg, dO):
    return float(np.sum(dO * orc.layer_forward(X, W, cfg)))


def _fd(f, arr):
    """Central differences of f() with respect to every element of arr (in place)."""
    g = np.zeros_like(arr)
    for idx in np.ndindex(arr.shape):
        old = arr[idx]
        arr[idx] = old + EPS
        fp = f()
        arr[idx] = old - EPS
        fm = f()
        arr[idx] = old
        g[idx] = (fp - fm) / (2 * EPS)
    return g


def _check(name, got, want):
    scale = max(1.0, float(np.abs(want).max()))
    err = float(np.abs(got - want).max()) / scale
    assert err < 2e-7, f"{name}: max error {err:.3e} (scale {scale:.3g})"


def _all_params(W, cfg):
    out = []
    for i, bw in enumerate(W.branches):
        for key in ("W_q", "W_k", "W_v", "W_g1", "W_g2", "b_g", "W_o"):
            out.append((f"br{i}.{key}", i, key, getattr(bw, key)))
        if cfg.norm:
            out.append((f"br{i}.g_norm", i, "g_norm", bw.g_norm))
    if cfg.n_branches > 1:
        out.append(("W_f", None, "W_f", W.W_f))
        out.append(("b_f", None, "b_f", W.b_f))
    return out


def _grad_of(grads, i, key):
    return grads[key] if i is None else grads["branches"][i][key]


@pytest.mark.parametrize("norm,scales,heads,L", [
    (False, (1, 2, 3), (1, 2, 1), 11),
    (True, (1, 2, 3), (1, 2, 1), 11),
    (False, (2, 4), (1, 1), 13),   # no scale-1 branch; t < 1 holds nothing
    (False, (1,), (2,), 7),        # one branch: no fusion weights
    (False, (1, 8), (1, 1), 7),    # the scale-8 branch has no complete block
])
def test_backward_matches_finite_differences(norm, scales, heads, L):
    cfg = _config(norm, scales, heads)
    rng = np.random.default_rng(7 + L)
    B = 2
    X = rng.normal(0, 1, (B, L, cfg.d_model))
    W = _weights(cfg, rng)
    dO = rng.normal(0, 1, (B, L, cfg.d_model))
    dX, grads = orc.layer_backward(X, W, cfg, dO)
    f = lambda: _loss(X, W, cfg, dO)
    _check("dX", dX, _fd(f, X))
    for name, i, key, arr in _all_params(W, cfg):
        _check(name, _grad_of(grads, i, key), _fd(f, arr))


@pytest.mark.parametrize("scales,heads,L", [((1, 2, 3), (1, 2, 1), 11), ((2, 4), (1, 1), 13)])
def test_masked_backward_matches_finite_differences(scales, heads, L):
    """Eq. (8) with a token mask: holes anywhere, a fully masked block, a block
    with one token; the mask enters the pooling only."""
    cfg = _config(False, scales, heads)
    rng = np.random.default_rng(31 + L)
    B = 2
    X = rng.normal(0, 1, (B, L, cfg.d_model))
    W = _weights(cfg, rng)
    dO = rng.normal(0, 1, (B, L, cfg.d_model))
    M = (rng.random((B, L)) > 0.3).astype(np.uint8)
    M[0, 4:8] = 0   # a whole padded block at s = 2 and s = 4
    M[1, 0:3] = 0   # one token left in the first block of s = 4
    dX, grads = orc.layer_backward(X, W, cfg, dO, M=M)
    f = lambda: float(np.sum(dO * orc.layer_forward(X, W, cfg, M=M)))
    _check("dX", dX, _fd(f, X))
    for name, i, key, arr in _all_params(W, cfg):
        _check(name, _grad_of(grads, i, key), _fd(f, arr))


def test_gla_backward_matches_finite_differences_with_strong_decay():
    """The recurrence alone, gates from alpha ~ 1 to alpha ~ 1e-3, 9 steps."""
    rng = np.random.default_rng(3)
    B, n, h, dk, dv = 2, 9, 2, 3, 4
    q, k = rng.normal(0, 1, (B, n, h, dk)), rng.normal(0, 1, (B, n, h, dk))
    v = rng.normal(0, 1, (B, n, h, dv))
    la = -rng.uniform(1e-3, 7.0, (B, n, h, dk))
    do = rng.normal(0, 1, (B, n, h, dv))
    dq, dk_, dv_, dla = orc.gla_recurrence_backward(q, k, v, la, do)
    f = lambda: float(np.sum(do * orc.gla_recurrence(q, k, v, la)[0]))
    _check("dq", dq, _fd(f, q))
    _check("dk", dk_, _fd(f, k))
    _check("dv", dv_, _fd(f, v))
    _check("dlog_alpha", dla, _fd(f, la))


def test_hold_backward_is_the_transpose_of_the_hold():
    """<causal_hold(Y), G> == <Y, causal_hold_backward(G)> for random Y, G."""
    rng = np.random.default_rng(5)
    for s, L in ((1, 6), (2, 9), (3, 11), (4, 4), (5, 3)):
        n = L // s
        Y = rng.normal(0, 1, (2, n, 3))
        G = rng.normal(0, 1, (2, L, 3))
        lhs = np.sum(orc.causal_hold(Y, s, L) * G)
        rhs = np.sum(Y * orc.causal_hold_backward(G, s, n))
        assert abs(lhs - rhs) < 1e-12


@pytest.mark.parametrize("mistake", ["no_decay_carry", "state_after_update", "no_sigmoid_factor"])
def test_planted_mistakes_fail_the_finite_difference_check(mistake, monkeypatch):
    """Each planted mistake in the backward moves a gradient far past the bar."""
    cfg = _config(False, (1, 2), (1, 1))
    rng = np.random.default_rng(11)
    B, L = 2, 8
    X = rng.normal(0, 1, (B, L, cfg.d_model))
    W = _weights(cfg, rng)
    dO = rng.normal(0, 1, (B, L, cfg.d_model))
    good = orc.gla_recurrence_backward

    def bad_gla(q, k, v, la, do):
        if mistake == "no_decay_carry":
            # forget Diag(alpha) when carrying G_t back to G_{t-1}
            return good(q, k, v, np.zeros_like(la), do)[:3] + (good(q, k, v, la, do)[3],)
        dq, dk, dv, dla = good(q, k, v, la, do)
        if mistake == "state_after_update":
            # dalpha_t from S_t instead of S_{t-1}: shift by one step
            dla = np.concatenate([dla[:, 1:], np.zeros_like(dla[:, :1])], axis=1)
        return dq, dk, dv, dla

    if mistake == "no_sigmoid_factor":
        monkeypatch.setattr(orc, "sigmoid", lambda z: np.ones_like(z))
    else:
        monkeypatch.setattr(orc, "gla_recurrence_backward", bad_gla)
    dX, grads = orc.layer_backward(X, W, cfg, dO)
    f = lambda: _loss(X, W, cfg, dO)
    errs = []
    for name, i, key, arr in _all_params(W, cfg):
        want = _fd(f, arr)
        errs.append(float(np.abs(_grad_of(grads, i, key) - want).max()) / max(1.0, float(np.abs(want).max())))
    errs.append(float(np.abs(dX - _fd(f, X)).max()))
    assert max(errs) > 1e-3, f"planted mistake {mistake} not detected: {max(errs):.2e}"


def test_normalised_query_and_key_gradients_are_sensitive_to_the_stored_output(monkeypatch):
    """The bar of the bf16 normalised backward: rounding only the GLA output o to
    bf16 (its storage type in the bf16 layer) inside the normalisation moves the
    exact gradients of the scale-1 branch's W_q and W_k by about 1e-2 of their
    largest entry, while W_v moves by far less.  The normalisation's backward
    removes the component of dLoss/do along o, and dq = do S^T nearly cancels
    when do is orthogonal to o = q S; so these two gradients carry o's storage
    rounding amplified, which bounds what a bf16 layer can reach against the
    fp64 function (main dimensions, B = 2, L = 200)."""
    from scale_gla_layer_amd.config import WORKLOADS
    from scale_gla_layer_amd.synth import make_inputs, round_to
    cfg = dataclasses.replace(WORKLOADS["main"].cfg, norm=True)
    X, W = make_inputs(cfg, 2, 200, seed=41)
    dO = round_to(np.random.default_rng(1041).normal(0.0, 1.0, X.shape), cfg.dtype)
    _, exact = orc.layer_backward(X, W, cfg, dO)
    fwd, bwd = orc.rms_norm_heads, orc.rms_norm_heads_backward
    monkeypatch.setattr(orc, "rms_norm_heads", lambda o, g: fwd(round_to(o, "bf16"), g))
    monkeypatch.setattr(orc, "rms_norm_heads_backward", lambda o, g, dy: bwd(round_to(o, "bf16"), g, dy))
    _, rounded = orc.layer_backward(X, W, cfg, dO)

    def moved(key):
        a, b = rounded["branches"][0][key], exact["branches"][0][key]
        return float(np.abs(a - b).max() / np.abs(b).max())

    assert 5e-3 < moved("W_q") < 2e-2 and 5e-3 < moved("W_k") < 2e-2
    assert moved("W_v") < 1e-3
