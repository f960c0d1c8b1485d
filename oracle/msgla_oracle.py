"""Plain fp64 CPU oracle of the MS-GLA token-mixing layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it and shares no code with it.

Source: the reading notes "MS-GLA：多时间尺度门控线性注意力研读笔记"
(cc.laoqi.cc, notes on arXiv:2609.35664 "MS-GLA: Multi-Scale Gated Linear
Attention ..."), Sec. 2.1 (GLA recurrence), Sec. 3.1-3.4 and Eqs. (8)-(11),
and its paragraph on streaming inference (the author's per-branch cache).

Everything is float64, one token at a time, in the order the notes describe:
pool (Eq. 8) -> per-branch projections and gate -> GLA recurrence
S_t = Diag(alpha_t) S_{t-1} + k_t^T v_t, o_t = q_t S_t -> per-branch output
projection -> causal hold (Sec. 3.3) -> softmax fusion over branches from the
unpooled x_t (Eqs. 10-11).  Row-vector convention throughout: x @ W with W
stored [in][out].

Readings where the notes leave a step open (all listed in the design doc):
  * the gate is log(alpha) = logsigmoid((xp @ W_g1) @ W_g2 + b_g) / gamma with
    gamma = 16 and no activation between the two factors; it is computed from
    the branch's pooled input;
  * each branch has an output projection W_o [h*d_v, d], no bias; the
    per-branch normalisation the notes name without a form is omitted
    (identity) unless the configuration asks for it (norm), where it is a
    per-head RMS normalisation over d_v with gains and eps = 1e-6 before W_o;
    there is no output gate; q is not scaled (q_scale = 1);
  * only complete pooling blocks enter the recurrence; a partial tail block is
    never read by the hold and is kept in the streaming cache instead;
  * positions before a branch's first complete block take zero from that
    branch, and the fusion weights are not renormalised there.

The layer backward (layer_backward and its parts, for training: the notes'
Sec. 3.4 training paragraph and Sec. 5.5, Table 4) is the vector-Jacobian
product of layer_forward written out by the chain rule, token by token, from
a fresh state, with or without a token mask.

Parity: every function here is pinned by tests under tests/ against values
the notes print (the s=4 hold table, the first pooled input), closed forms,
textbook identities and brute-force products; the backward against central
finite differences of the (pinned) forward; see the test module docstrings.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np

# --------------------------------------------------------------------------
# Elementary maps
# --------------------------------------------------------------------------


def logsigmoid(z: np.ndarray) -> np.ndarray:
    """log(1 / (1 + exp(-z))), evaluated without overflow in either tail.

    Gate form of the notes, Sec. 2.1 ("a sigmoid-type map of a low-rank
    projection", values of alpha in (0, 1)); the logsigmoid/16 form is the
    one the layer configuration fixes.
    """
    z = np.asarray(z, dtype=np.float64)
    return np.where(z >= 0, -np.log1p(np.exp(-np.abs(z))), z - np.log1p(np.exp(-np.abs(z))))


def softmax_lastdim(z: np.ndarray) -> np.ndarray:
    """Softmax over the last axis with max subtraction (Eq. (10))."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


# --------------------------------------------------------------------------
# Sec. 3.1, Eq. (8): non-overlapping (masked) mean pooling
# --------------------------------------------------------------------------


def pool_eq8(X: np.ndarray, s: int, M: Optional[np.ndarray] = None) -> np.ndarray:
    """Eq. (8) over all ceil(L/s) blocks, right-padding with zeros.

    X: [B, L, d]; M: [B, L] validity mask (1 = token, 0 = padding), default
    all ones on the real tokens.  Padded positions carry mask 0, so a partial
    tail block averages its real tokens, and an all-padding block gives 0
    (the max(1, .) floor of the denominator).
    """
    B, L, d = X.shape
    if M is None:
        M = np.ones((B, L))
    n = -(-L // s)
    out = np.zeros((B, n, d))
    for b in range(B):
        for i in range(n):
            num = np.zeros(d)
            den = 0.0
            for j in range(s):
                t = i * s + j
                if t < L:
                    num += X[b, t] * M[b, t]
                    den += M[b, t]
            out[b, i] = num / max(1.0, den)
    return out


def pool_complete_blocks(X: np.ndarray, s: int) -> np.ndarray:
    """Unmasked Eq. (8) restricted to the floor(L/s) complete blocks: [B, n_s, d]."""
    B, L, d = X.shape
    n = L // s
    out = np.zeros((B, n, d))
    for j in range(s):
        out += X[:, j: n * s: s, :] if n > 0 else 0.0
    return out / s


# --------------------------------------------------------------------------
# Sec. 3.2: independent per-branch projections and forget gate
# --------------------------------------------------------------------------


def branch_projections(xp: np.ndarray, bw, cfg):
    """q, k, v and log(alpha) of one branch from its pooled input.

    xp: [..., d].  Returns q, k [..., h, d_k], v [..., h, d_v], log_alpha
    [..., h, d_k].  Head j owns column slice j of every projection.
    """
    h = bw.W_q.shape[1] // cfg.d_k
    lead = xp.shape[:-1]
    q = cfg.q_scale * (xp @ bw.W_q)
    k = xp @ bw.W_k
    v = xp @ bw.W_v
    g = (xp @ bw.W_g1) @ bw.W_g2 + bw.b_g
    log_alpha = logsigmoid(g) / cfg.gate_normalizer
    return (q.reshape(*lead, h, cfg.d_k), k.reshape(*lead, h, cfg.d_k),
            v.reshape(*lead, h, cfg.d_v), log_alpha.reshape(*lead, h, cfg.d_k))


# --------------------------------------------------------------------------
# Sec. 2.1: the GLA recurrence, one token at a time
# --------------------------------------------------------------------------


def gla_recurrence(q, k, v, log_alpha, S0=None):
    """S_t = Diag(alpha_t) S_{t-1} + k_t^T v_t ;  o_t = q_t S_t.

    q, k, log_alpha: [B, n, h, d_k]; v: [B, n, h, d_v]; S0: [B, h, d_k, d_v]
    or None (zeros).  alpha_t scales row c of the state by alpha_{t,c}.
    Returns (o [B, n, h, d_v], S_n [B, h, d_k, d_v]).
    """
    B, n, h, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, h, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((B, n, h, dv))
    alpha = np.exp(log_alpha)
    for t in range(n):
        S = alpha[:, t, :, :, None] * S + k[:, t, :, :, None] * v[:, t, :, None, :]
        o[:, t] = np.einsum("bhc,bhcv->bhv", q[:, t], S)
    return o, S


# --------------------------------------------------------------------------
# Sec. 3.3: causal hold and fusion
# --------------------------------------------------------------------------


def hold_index(t: int, s: int) -> int:
    """Coarse output visible at original position t, or -1 for none.

    Block j covers positions js .. js+s-1, so it is complete (usable) from
    position (j+1)s-1 on, until block j+1 completes: t -> floor((t+1)/s) - 1.
    """
    return (t + 1) // s - 1


def causal_hold(Y: np.ndarray, s: int, L: int):
    """[B, n_s, d] coarse outputs -> [B, L, d] per original position; positions
    before the first complete block take zero."""
    B, n, d = Y.shape
    out = np.zeros((B, L, d))
    for t in range(L):
        j = hold_index(t, s)
        if j >= 0:
            out[:, t] = Y[:, j]
    return out


def fusion_weights(X: np.ndarray, W_f: np.ndarray, b_f: np.ndarray) -> np.ndarray:
    """Eq. (10): w_t = softmax(x_t W_f + b_f) from the unpooled x_t: [B, L, m]."""
    return softmax_lastdim(X @ W_f + b_f)


def routing_stability(w: np.ndarray, frac: float = 0.1) -> np.ndarray:
    """Sec. 5.4 / Table 3 procedure: mean fusion weight of each branch, in
    percent, over the first, the middle and the last `frac` of the positions.

    w: [B, L, m] fusion weights.  The first region is positions
    [0, ceil(frac L)), the last [L - ceil(frac L), L), and the middle the same
    count starting at floor((L - ceil(frac L)) / 2); each mean runs over the
    region's positions of every sequence.  Returns [3, m].
    """
    w = np.asarray(w, dtype=np.float64)
    B, L, m = w.shape
    n = max(1, math.ceil(frac * L))
    mid = (L - n) // 2
    out = np.zeros((3, m))
    for r, start in enumerate((0, mid, L - n)):
        acc = np.zeros(m)
        for b in range(B):
            for t in range(start, start + n):
                acc += w[b, t]
        out[r] = 100.0 * acc / (B * n)
    return out


# --------------------------------------------------------------------------
# The whole layer
# --------------------------------------------------------------------------


# --------------------------------------------------------------------------
# Sec. 3.2: the per-branch normalisation the notes name (form: a reading)
# --------------------------------------------------------------------------

NORM_EPS = 1e-6


def rms_norm_heads(o: np.ndarray, g: np.ndarray) -> np.ndarray:
    """Per-head RMS normalisation of a branch's GLA output before W_o.

    o: [..., h, d_v]; g: [h * d_v] gains.  Each head's row is divided by the
    root of its mean square plus NORM_EPS and multiplied by its gains:
    o_c / sqrt(mean_c' o_c'^2 + eps) * g_c.
    """
    o = np.asarray(o, dtype=np.float64)
    h, dv = o.shape[-2], o.shape[-1]
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return o / np.sqrt(ms + NORM_EPS) * np.asarray(g, dtype=np.float64).reshape(h, dv)


def branch_forward(X: np.ndarray, bw, s: int, cfg, M: Optional[np.ndarray] = None):
    """One branch: pool -> project -> recurrence -> output projection.

    M: optional [B, L] validity mask of Eq. (8); the branch then pools each
    complete block as the mask-weighted mean with the max(1, sum M) floor.
    Returns (Y [B, n_s, d], final state S [B, h, d_k, d_v], n_s).
    """
    B, L, d = X.shape
    xp = pool_complete_blocks(X, s) if M is None else pool_eq8(X, s, M)[:, : L // s]
    n = xp.shape[1]
    q, k, v, la = branch_projections(xp, bw, cfg)
    o, S = gla_recurrence(q, k, v, la)
    if getattr(cfg, "norm", False):
        o = rms_norm_heads(o, bw.g_norm)
    Y = o.reshape(B, n, o.shape[2] * o.shape[3]) @ bw.W_o
    return Y, S, n


def layer_forward(X: np.ndarray, W, cfg, return_state: bool = False, M: Optional[np.ndarray] = None):
    """MS-GLA layer forward from a fresh state (Sec. 3, Eqs. (8)-(11)).

    X: [B, L, d] float64 (the values the device sees, upcast).  Returns O
    [B, L, d]; with ``return_state`` also the streaming cache after the call
    (see ``decode_step``).
    M: optional [B, L] token mask of Eq. (8) (nonzero = token).  It enters the
    pooling only, as the equation is written: every branch pools its complete
    blocks as mask-weighted means (for s = 1 that is M_t x_t), while the
    fusion weights still come from the unpooled x_t.  The cache of a masked
    call keeps, for the incomplete block, the mask-weighted sum of its hidden
    states and its token count (the denominator of Eq. (8)) beside its count
    of positions.
    """
    X = np.asarray(X, dtype=np.float64)
    B, L, d = X.shape
    if M is not None:
        M = (np.asarray(M) != 0).astype(np.float64).reshape(B, L)
    m = len(cfg.scales)
    w = np.ones((B, L, 1)) if m == 1 else fusion_weights(X, W.W_f, W.b_f)
    O = np.zeros((B, L, d))
    state = {"pos": L, "branches": []}
    for i, (s, bw) in enumerate(zip(cfg.scales, W.branches)):
        Y, S, n = branch_forward(X, bw, s, cfg, M)
        O += w[:, :, i: i + 1] * causal_hold(Y, s, L)
        if return_state:
            tail = X[:, n * s: L, :]
            mt = np.ones((B, L - n * s)) if M is None else M[:, n * s: L]
            state["branches"].append({
                "S": S,
                "psum": (tail * mt[:, :, None]).sum(axis=1),
                "count": L - n * s,
                "tokens": mt.sum(axis=1),
                "held": Y[:, n - 1] if n > 0 else np.zeros((B, d)),
            })
    return (O, state) if return_state else O


def init_state(cfg, batch: int) -> Dict:
    """Empty streaming cache: zero state, empty pooling buffer, zero held output."""
    brs = []
    for h in cfg.heads:
        brs.append({"S": np.zeros((batch, h, cfg.d_k, cfg.d_v)),
                    "psum": np.zeros((batch, cfg.d_model)), "count": 0,
                    "tokens": np.zeros(batch),
                    "held": np.zeros((batch, cfg.d_model))})
    return {"pos": 0, "branches": brs}


def decode_step(state: Dict, x_t: np.ndarray, W, cfg):
    """One streaming step (the notes' paragraph on token-by-token inference).

    Each branch keeps its GLA state, the not-yet-complete block of hidden
    states (here its running sum, its count of positions and its count of
    tokens, which differ only after a masked forward) and its latest output.
    A new token is accumulated; when the block's s positions have arrived it
    is pooled as sum / max(1, tokens) (Eq. (8): the new tokens are real ones),
    the branch takes one recurrence step, and the held output is replaced;
    otherwise the held output is reused.  The branches are then fused with
    weights from the unpooled x_t (Eqs. (10)-(11)).
    x_t: [B, d].  Returns (o_t [B, d], new state); the input state is not
    modified.
    """
    x_t = np.asarray(x_t, dtype=np.float64)
    B, d = x_t.shape
    m = len(cfg.scales)
    new = {"pos": state["pos"] + 1, "branches": []}
    w = np.ones((B, 1)) if m == 1 else softmax_lastdim(x_t @ W.W_f + W.b_f)
    o = np.zeros((B, d))
    for i, (s, bw) in enumerate(zip(cfg.scales, W.branches)):
        st = state["branches"][i]
        psum = st["psum"] + x_t
        count = st["count"] + 1
        tokens = st["tokens"] + 1
        S, held = st["S"], st["held"]
        if count == s:
            xp = psum / np.maximum(1.0, tokens)[:, None]
            q, k, v, la = branch_projections(xp[:, None, :], bw, cfg)
            y, S = gla_recurrence(q, k, v, la, S0=S)
            if getattr(cfg, "norm", False):
                y = rms_norm_heads(y, bw.g_norm)
            held = y.reshape(B, -1) @ bw.W_o
            psum = np.zeros((B, d))
            count = 0
            tokens = np.zeros(B)
        new["branches"].append({"S": S, "psum": psum, "count": count, "tokens": tokens,
                                "held": held})
        o += w[:, i: i + 1] * held
    return o, new


def recurrence_updates(cfg, L: int) -> int:
    """Number of per-head state updates one forward of length L performs."""
    return sum(h * (L // s) for s, h in zip(cfg.scales, cfg.heads))


def row_relative_error(O_dev: np.ndarray, O_ref: np.ndarray):
    """max_t ||O_t - Ref_t||_inf / ||Ref_t||_inf over rows with Ref_t != 0,
    and whether every all-zero reference row is exactly zero on the device."""
    O_dev = np.asarray(O_dev, dtype=np.float64).reshape(-1, O_ref.shape[-1])
    O_ref = np.asarray(O_ref, dtype=np.float64).reshape(-1, O_ref.shape[-1])
    den = np.abs(O_ref).max(axis=1)
    num = np.abs(O_dev - O_ref).max(axis=1)
    nz = den > 0
    err = float((num[nz] / den[nz]).max()) if nz.any() else 0.0
    zero_rows_exact = bool(np.all(O_dev[~nz] == 0.0))
    return err, zero_rows_exact


# --------------------------------------------------------------------------
# Layer backward (training): the notes train each branch with GLA's chunkwise
# algorithm (Sec. 3.4, training paragraph) and compare training throughput in
# Sec. 5.5, Table 4.  What training needs from the layer is the vector-Jacobian
# product of layer_forward: given dO = dLoss/dO, the gradients of the loss
# with respect to X and every weight.  The functions below are that product
# written out by the chain rule, walking the forward's steps in reverse, one
# token at a time (no chunking), from a fresh state and without a mask.
# --------------------------------------------------------------------------


def sigmoid(z: np.ndarray) -> np.ndarray:
    """1 / (1 + exp(-z)) = exp(logsigmoid(z)), without overflow."""
    return np.exp(logsigmoid(z))


def gla_recurrence_backward(q, k, v, log_alpha, do):
    """VJP of gla_recurrence from a zero initial state.

    Forward: S_t = Diag(alpha_t) S_{t-1} + k_t^T v_t, o_t = q_t S_t (S_{-1} = 0).
    With G_t = dLoss/dS_t (everything the loss receives through S_t):
      G_t = q_t^T do_t + Diag(alpha_{t+1}) G_{t+1}          (G_n = 0 beyond the end)
      dq_t = do_t S_t^T,  dk_t = G_t v_t^T (per row c: sum_e G_t[c,e] v_t[e]),
      dv_t = k_t G_t (per column e: sum_c k_t[c] G_t[c,e]),
      dalpha_t[c] = sum_e G_t[c,e] S_{t-1}[c,e],  dlog_alpha_t = dalpha_t * alpha_t.
    Shapes as gla_recurrence; do [B, n, h, d_v].  Returns (dq, dk, dv, dlog_alpha).
    """
    B, n, h, dk = q.shape
    dv_ = v.shape[-1]
    alpha = np.exp(log_alpha)
    states = np.zeros((n + 1, B, h, dk, dv_))  # states[t + 1] = S_t, states[0] = S_{-1} = 0
    S = np.zeros((B, h, dk, dv_))
    for t in range(n):
        S = alpha[:, t, :, :, None] * S + k[:, t, :, :, None] * v[:, t, :, None, :]
        states[t + 1] = S
    dq = np.zeros_like(q)
    dk_ = np.zeros_like(k)
    dvv = np.zeros_like(v)
    dla = np.zeros_like(log_alpha)
    G = np.zeros((B, h, dk, dv_))
    for t in reversed(range(n)):
        G = G + q[:, t, :, :, None] * do[:, t, :, None, :]
        dq[:, t] = np.einsum("bhv,bhcv->bhc", do[:, t], states[t + 1])
        dk_[:, t] = np.einsum("bhcv,bhv->bhc", G, v[:, t])
        dvv[:, t] = np.einsum("bhcv,bhc->bhv", G, k[:, t])
        dla[:, t] = np.einsum("bhcv,bhcv->bhc", G, states[t]) * alpha[:, t]
        G = alpha[:, t, :, :, None] * G
    return dq, dk_, dvv, dla


def rms_norm_heads_backward(o: np.ndarray, g: np.ndarray, dy: np.ndarray):
    """VJP of rms_norm_heads: y_c = o_c g_c / r, r = sqrt(mean_c' o_c'^2 + eps).

    do_c = g_c dy_c / r - o_c (sum_c' g_c' dy_c' o_c') / (d_v r^3);
    dg_c = sum over positions of o_c dy_c / r.  o, dy: [..., h, d_v].
    Returns (do, dg [h d_v]).
    """
    o = np.asarray(o, dtype=np.float64)
    h, dv = o.shape[-2], o.shape[-1]
    gg = np.asarray(g, dtype=np.float64).reshape(h, dv)
    r = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + NORM_EPS)
    inner = np.sum(gg * dy * o, axis=-1, keepdims=True)
    do = gg * dy / r - o * inner / (dv * r ** 3)
    dg = (o * dy / r).reshape(-1, h, dv).sum(axis=0).reshape(h * dv)
    return do, dg


def causal_hold_backward(dH: np.ndarray, s: int, n: int) -> np.ndarray:
    """VJP of causal_hold: [B, L, d] -> [B, n, d]; coarse output j receives
    the gradients of the positions that show it (hold_index(t, s) == j)."""
    B, L, d = dH.shape
    dY = np.zeros((B, n, d))
    for t in range(L):
        j = hold_index(t, s)
        if j >= 0:
            dY[:, j] += dH[:, t]
    return dY


def branch_backward(X: np.ndarray, bw, s: int, cfg, dY: np.ndarray, M: Optional[np.ndarray] = None):
    """VJP of branch_forward (zero initial state).

    dY: [B, n_s, d], the gradient of the branch's coarse outputs; M: the
    optional [B, L] token mask of Eq. (8).  Returns (dX [B, L, d], grads) with
    grads holding W_q, W_k, W_v, W_g1, W_g2, b_g, W_o (and g_norm when the
    configuration normalises), shaped as the weights.
    """
    X = np.asarray(X, dtype=np.float64)
    B, L, d = X.shape
    xp = pool_complete_blocks(X, s) if M is None else pool_eq8(X, s, M)[:, : L // s]
    n = xp.shape[1]
    h = bw.W_q.shape[1] // cfg.d_k
    q, k, v, la = branch_projections(xp, bw, cfg)
    o, _ = gla_recurrence(q, k, v, la)
    norm = getattr(cfg, "norm", False)
    on = rms_norm_heads(o, bw.g_norm) if norm else o
    grads = {}
    # Y = on W_o
    grads["W_o"] = on.reshape(B * n, h * cfg.d_v).T @ dY.reshape(B * n, d)
    don = (dY @ bw.W_o.T).reshape(B, n, h, cfg.d_v)
    if norm:
        do, grads["g_norm"] = rms_norm_heads_backward(o, bw.g_norm, don)
    else:
        do = don
    dq, dk, dv, dla = gla_recurrence_backward(q, k, v, la, do)
    # log_alpha = logsigmoid(z) / gamma, z = (xp W_g1) W_g2 + b_g
    g1 = xp @ bw.W_g1
    z = g1 @ bw.W_g2 + bw.b_g
    dz = dla.reshape(B, n, h * cfg.d_k) / cfg.gate_normalizer * sigmoid(-z)
    r, hdk, hdv = bw.W_g1.shape[1], h * cfg.d_k, h * cfg.d_v
    grads["W_g2"] = g1.reshape(B * n, r).T @ dz.reshape(B * n, hdk)
    grads["b_g"] = dz.reshape(B * n, hdk).sum(axis=0)
    dg1 = dz @ bw.W_g2.T
    # q = q_scale xp W_q, k = xp W_k, v = xp W_v
    dq = cfg.q_scale * dq.reshape(B, n, hdk)
    dk = dk.reshape(B, n, hdk)
    dv = dv.reshape(B, n, hdv)
    xf = xp.reshape(B * n, d)
    grads["W_q"] = xf.T @ dq.reshape(B * n, hdk)
    grads["W_k"] = xf.T @ dk.reshape(B * n, hdk)
    grads["W_v"] = xf.T @ dv.reshape(B * n, hdv)
    grads["W_g1"] = xf.T @ dg1.reshape(B * n, r)
    dxp = dq @ bw.W_q.T + dk @ bw.W_k.T + dv @ bw.W_v.T + dg1 @ bw.W_g1.T
    dX = np.zeros((B, L, d))
    if M is None:
        # xp_j = mean of the s positions of complete block j
        for j in range(s):
            if n > 0:
                dX[:, j: n * s: s, :] += dxp / s
    else:
        # xp_j = sum_t M_t x_t / max(1, sum_t M_t) over the block's positions t
        Mf = (np.asarray(M) != 0).astype(np.float64).reshape(B, L)
        for b in range(B):
            for j in range(n):
                cnt = max(1.0, Mf[b, j * s: (j + 1) * s].sum())
                for t in range(j * s, (j + 1) * s):
                    dX[b, t] += Mf[b, t] * dxp[b, j] / cnt
    return dX, grads


def layer_backward(X: np.ndarray, W, cfg, dO: np.ndarray, M: Optional[np.ndarray] = None):
    """VJP of layer_forward (fresh state; M the optional token mask of Eq. (8),
    which enters the pooling only): dO [B, L, d] -> (dX [B, L, d], grads) with
    grads["branches"][i] as branch_backward's and grads["W_f"], grads["b_f"]
    for the fusion logits (zero when m == 1).

    O_t = sum_i w_{t,i} H^(i)_t with H^(i) the held coarse outputs and
    w_t = softmax(z_t), z_t = x_t W_f + b_f:
      dH^(i)_t = w_{t,i} dO_t,  dw_{t,i} = dO_t . H^(i)_t,
      dz_t = w_t * (dw_t - sum_i w_{t,i} dw_{t,i}).
    """
    X = np.asarray(X, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    B, L, d = X.shape
    m = len(cfg.scales)
    w = np.ones((B, L, 1)) if m == 1 else fusion_weights(X, W.W_f, W.b_f)
    dX = np.zeros((B, L, d))
    dw = np.zeros((B, L, m))
    grads = {"branches": []}
    for i, (s, bw) in enumerate(zip(cfg.scales, W.branches)):
        Y, _, n = branch_forward(X, bw, s, cfg, M)
        H = causal_hold(Y, s, L)
        dw[:, :, i] = np.sum(dO * H, axis=-1)
        dY = causal_hold_backward(w[:, :, i: i + 1] * dO, s, n)
        dXi, gi = branch_backward(X, bw, s, cfg, dY, M)
        dX += dXi
        grads["branches"].append(gi)
    if m > 1:
        dz = w * (dw - np.sum(w * dw, axis=-1, keepdims=True))
        grads["W_f"] = X.reshape(B * L, d).T @ dz.reshape(B * L, m)
        grads["b_f"] = dz.reshape(B * L, m).sum(axis=0)
        dX += dz @ W.W_f.T
    else:
        grads["W_f"] = np.zeros((d, 1))
        grads["b_f"] = np.zeros(1)
    return dX, grads
