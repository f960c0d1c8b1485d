"""CPU fp32 emulation of how the chunk kernel factors the intra-chunk matrix.

Within a chunk, A[t][i] = sum_c q_tc k_ic 2^(b_tc - b_ic) for i <= t, with
b the chunk-local cumulative log2 decay of the GLA recurrence (MS-GLA notes,
Sec. 2.1; chunkwise form, Sec. 3.4).  The kernel cannot exponentiate b_t - b_i
per pair cheaply, so it splits the factor into per-position pieces, one wave
per 16 positions.  This module replays those pieces in numpy float32, in the
kernel's order, and compares them with the fp64 pairwise definition:

* the factoring through each 16-position block's first position (query side
  2^(b_t - b_16T), key side 2^(b_16J - b_i)) grows the key side over up to 15
  positions and overflows fp32 for strongly decaying gates (gamma 16 with a
  gate pre-activation near -100, or gamma 1 with bias -8): the first tests
  reproduce those non-finite entries;
* the factoring the kernel uses references each stored key side at the END
  of its block (every stored factor 2^(<=0)); the diagonal block's one growing
  factor 2^(b_16T - b_end) is used only while it is at most 2^32 and finite,
  otherwise that block is formed pair by pair from products of per-step
  decays alpha_u <= 1: the last tests check it is finite and agrees with the
  definition to fp32 accuracy at benign, adversarial and mixed gates.

Test-only code: it shares nothing with the kernels or the oracle.
"""
import numpy as np
import pytest

F = np.float32
BLK = 16      # positions per wave
THRESH = 32.0  # log2 bound on the diagonal block's growing factor


def _gates(rng, C, dk, gamma, z_mean, z_std=1.0):
    """Per-step log2 decay la = log2(sigmoid(z)) / gamma for z ~ N(z_mean, z_std)."""
    z = rng.normal(z_mean, z_std, (C, dk))
    ls = np.where(z >= 0, -np.log1p(np.exp(-z)), z - np.log1p(np.exp(z)))  # ln sigmoid
    return (ls / np.log(2.0) / gamma).astype(F)


def _wave_scans(la):
    """Wave-local inclusive scans x (float32, in position order), and the
    chunk-level b = (sum of earlier waves' totals) + x."""
    C, dk = la.shape
    x = np.zeros_like(la)
    for w in range(C // BLK):
        acc = np.zeros(dk, F)
        for r in range(BLK):
            acc = F(acc + la[w * BLK + r])
            x[w * BLK + r] = acc
    carry = np.zeros((C // BLK, dk), F)
    for w in range(1, C // BLK):
        carry[w] = F(carry[w - 1] + x[w * BLK - 1])
    return x, carry


def reference(q, k, la):
    """fp64 definition: sum_c q_tc k_ic 2^(b_t - b_i), i <= t."""
    b = np.cumsum(la.astype(np.float64), axis=0)
    C = q.shape[0]
    A = np.zeros((C, C))
    scale = np.zeros((C, C))
    for t in range(C):
        for i in range(t + 1):
            f = np.exp2(b[t] - b[i])
            A[t, i] = np.sum(q[t].astype(np.float64) * k[i] * f)
            scale[t, i] = np.sum(np.abs(q[t].astype(np.float64) * k[i]) * f)
    return A, scale


def start_referenced(q, k, la):
    """Blocks referenced at their first position (the growing key side)."""
    x, carry = _wave_scans(la)
    C = q.shape[0]
    NW = C // BLK
    A = np.zeros((C, C), F)
    with np.errstate(over="ignore", invalid="ignore"):
        for T in range(NW):
            rows = slice(T * BLK, (T + 1) * BLK)
            first_T = x[T * BLK]
            Q = F(q[rows] * np.exp2(F(x[rows] - first_T)))
            for J in range(T + 1):
                cols = slice(J * BLK, (J + 1) * BLK)
                first_J = x[J * BLK]
                K = F(k[cols] * np.exp2(F(first_J - x[cols])))  # grows over < 16 positions
                if J < T:
                    D = np.exp2(F(F(carry[T] + first_T) - F(carry[J] + first_J)))
                    K = F(K * D)
                blk = F(Q @ K.T)
                if J == T:
                    blk = np.tril(blk)
                A[rows, cols] = blk
    return A


def end_referenced(q, k, la):
    """The kernel's factoring: stored key sides referenced at their block's
    last position; the diagonal block through one bounded growing factor, or
    pair by pair from per-step decay products.  Returns (A, exact_waves)."""
    x, carry = _wave_scans(la)
    C, dk = q.shape
    NW = C // BLK
    A = np.zeros((C, C), F)
    exact_waves = []
    with np.errstate(over="ignore", invalid="ignore"):
        kb = np.zeros_like(k)
        for J in range(NW):
            cols = slice(J * BLK, (J + 1) * BLK)
            kb[cols] = F(k[cols] * np.exp2(F(x[J * BLK + BLK - 1] - x[cols])))  # <= |k|
        for T in range(NW):
            rows = slice(T * BLK, (T + 1) * BLK)
            first_T, last_T = x[T * BLK], x[T * BLK + BLK - 1]
            b16T = F(carry[T] + first_T)
            Q = F(q[rows] * np.exp2(F(x[rows] - first_T)))  # <= |q|
            for J in range(T):
                cols = slice(J * BLK, (J + 1) * BLK)
                D = np.exp2(F(b16T - F(carry[J] + x[J * BLK + BLK - 1])))  # <= 1
                A[rows, cols] = F(Q @ F(kb[cols] * D).T)
            growth = F(first_T - last_T)  # log2 of the diagonal's growing factor
            Kd = F(kb[rows] * np.exp2(growth))
            if growth.max() <= THRESH and np.all(np.isfinite(Kd)):
                A[rows, rows] = np.tril(F(Q @ Kd.T))
                continue
            exact_waves.append(T)
            xs = x[rows]
            prev = np.vstack([np.zeros((1, dk), F), xs[:-1]])
            alpha = np.exp2(F(xs - prev))  # per-step decays, <= 1
            blk = np.zeros((BLK, BLK), F)
            for t in range(BLK):
                P = np.ones(dk, F)
                for d in range(t + 1):
                    if d > 0:
                        P = F(P * alpha[t - d + 1])
                    blk[t, t - d] = F(np.sum(F(F(q[T * BLK + t] * P) * k[T * BLK + t - d]), dtype=F))
            A[rows, rows] = blk
    return A, exact_waves


def _row_err(A, A_ref, scale):
    """Largest error of a row relative to the row's largest term magnitude
    (A enters the output as o_t = sum_i A[t][i] v_i, so that is the scale an
    error is seen at; entries far below it may underflow in fp32)."""
    row = scale.max(axis=1, keepdims=True)
    return float((np.abs(A - A_ref) / row).max())


def _case(seed, gamma, z_mean, C=64, dk=128, z_std=1.0):
    rng = np.random.default_rng(seed)
    q = rng.normal(0, 1, (C, dk)).astype(F)
    k = rng.normal(0, 1, (C, dk)).astype(F)
    la = _gates(rng, C, dk, gamma, z_mean, z_std)
    return q, k, la


@pytest.mark.parametrize("gamma,z_mean", [(16.0, -100.0), (1.0, -8.0)])
def test_start_referenced_blocks_overflow_at_strong_decay(gamma, z_mean):
    """Reproduces the fault: the fp64 definition is finite, the growing key
    side is not."""
    q, k, la = _case(1, gamma, z_mean)
    A_ref, _ = reference(q, k, la)
    assert np.all(np.isfinite(A_ref))
    A_old = start_referenced(q, k, la)
    assert not np.all(np.isfinite(A_old))


@pytest.mark.parametrize("gamma,z_mean,exact", [
    (16.0, 0.0, False),     # the benchmark gates: fast diagonal
    (16.0, -8.0, False),    # bias -8 at gamma 16: growth ~2^11, fast diagonal
    (16.0, -100.0, True),   # growth ~2^135: exact diagonal
    (1.0, -8.0, True),      # growth ~2^173: exact diagonal
    (1.0, 0.0, False),
])
def test_end_referenced_blocks_match_the_definition(gamma, z_mean, exact):
    q, k, la = _case(2, gamma, z_mean)
    A_ref, scale = reference(q, k, la)
    A_new, exact_waves = end_referenced(q, k, la)
    assert np.all(np.isfinite(A_new))
    assert (len(exact_waves) == 4) == exact and (len(exact_waves) == 0) == (not exact)
    assert _row_err(A_new, A_ref, scale) <= 2e-6


def test_mixed_waves_take_their_own_path():
    """A chunk whose first 32 positions decay strongly and the rest weakly:
    waves 0, 1 take the exact diagonal, waves 2, 3 the fast one, and the
    off-diagonal blocks bridging them stay finite and exact."""
    rng = np.random.default_rng(3)
    C, dk = 64, 128
    q = rng.normal(0, 1, (C, dk)).astype(F)
    k = rng.normal(0, 1, (C, dk)).astype(F)
    la = np.concatenate([_gates(rng, 32, dk, 1.0, -8.0), _gates(rng, 32, dk, 16.0, 0.0)])
    A_ref, scale = reference(q, k, la)
    A_new, exact_waves = end_referenced(q, k, la)
    assert exact_waves == [0, 1]
    assert np.all(np.isfinite(A_new))
    assert _row_err(A_new, A_ref, scale) <= 2e-6
