"""Pins of the oracle's gated recurrence (diagonal and input-dependent
decay) against values fixed by the pages and by maths.  CPU only.

The recurrence, per state row f: mu_j[f] = gamma_jf mu_{j-1}[f] +
(1 - gamma_jf) k'_jf v_j (and nu likewise), gamma = exp(lam): eqs 10-11 of
"2.2 Linear Attention" (efficient2 page) with the decay made diagonal as in
"2.3 State-Space Models" eqs 21-25, and input-dependent as in the Mamba
section of the "Linear attention research 2026" page.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import brute

MODES = (oracle.LD_CHANNEL, oracle.LD_POSITION, oracle.LD_BOTH)


def rel_err(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def rand_lam(rng, mode, B, H, n, df, lo=-2.5, hi=-0.01):
    shape = {oracle.LD_CHANNEL: (H, df), oracle.LD_POSITION: (B, H, n),
             oracle.LD_BOTH: (B, H, n, df)}[mode]
    return rng.uniform(lo, hi, size=shape)


def full_lam(lam, mode, B, H, n, df):
    """Broadcast any layout to [B, H, n, d_feat]."""
    if mode == oracle.LD_CHANNEL:
        return np.broadcast_to(lam[None, :, None, :], (B, H, n, df))
    if mode == oracle.LD_POSITION:
        return np.broadcast_to(lam[..., None], (B, H, n, df))
    return lam


def inputs(rng, B, H, n, d, m, mapk):
    dqk = m if mapk == oracle.MAP_IDENTITY else d
    q = rng.standard_normal((B, H, n, dqk)) * 0.7
    k = rng.standard_normal((B, H, n, dqk)) * 0.7
    if mapk == oracle.MAP_IDENTITY:
        q, k = np.abs(q) + 0.05, np.abs(k) + 0.05
    v = rng.standard_normal((B, H, n, d))
    om = rng.standard_normal((d, m)) / math.sqrt(d)
    return q, k, v, om


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("mapk", [oracle.MAP_ELU1, oracle.MAP_PERFORMER,
                                  oracle.MAP_IDENTITY])
@pytest.mark.parametrize("causal", [True, False])
def test_gated_recurrence_equals_dense_weights(mode, mapk, causal):
    """The recurrence against the dense form with weights built from
    explicit products of the decays (brute force, n <= 30)."""
    rng = np.random.default_rng(11 + mode)
    B, H, n, d, m = 2, 2, 23, 5, 6
    q, k, v, om = inputs(rng, B, H, n, d, m, mapk)
    df = m if mapk != oracle.MAP_ELU1 else d
    lam = rand_lam(rng, mode, B, H, n, df)
    got = oracle.forward_gated(q, k, v, mapk, om, lam, mode, causal)
    want = brute.gated_quadratic(brute.features(q, mapk, om),
                                 brute.features(k, mapk, om), v,
                                 full_lam(lam, mode, B, H, n, df), causal)
    assert rel_err(got, want) < 1e-12


def test_gated_hand_example_per_channel():
    """d' = 2 rows decaying by 0.5 and 0.25, identity features, d = 1:
    mu_1 = [1, 1.5], nu_1 = [0.5, 0.75]; mu_2 = [2.5, 6.375],
    nu_2 = [0.75, 1.6875]; out_2 = (2 * 2.5 + 6.375) / (2 * 0.75 + 1.6875)
    for q'_2 = [2, 1]."""
    q = np.array([[1.0, 1.0], [2.0, 1.0]]).reshape(1, 1, 2, 2)
    k = np.array([[1.0, 1.0], [1.0, 2.0]]).reshape(1, 1, 2, 2)
    v = np.array([2.0, 4.0]).reshape(1, 1, 2, 1)
    lam = np.log(np.array([[0.5, 0.25]]))
    got = oracle.forward_gated(q, k, v, oracle.MAP_IDENTITY, None, lam,
                               oracle.LD_CHANNEL).ravel()
    assert abs(got[0] - 2.0) < 1e-15
    assert abs(got[1] - 11.375 / 3.1875) < 1e-14


def test_gated_hand_example_per_position():
    """d' = 1, decays 0.5 then 0.2: mu_2 = 0.2 * 1 + 0.8 * 4 = 3.4,
    nu_2 = 0.2 * 0.5 + 0.8 = 0.9."""
    q = np.ones((1, 1, 2, 1))
    k = np.ones((1, 1, 2, 1))
    v = np.array([2.0, 4.0]).reshape(1, 1, 2, 1)
    lam = np.log(np.array([[[0.5, 0.2]]]))
    got = oracle.forward_gated(q, k, v, oracle.MAP_IDENTITY, None, lam,
                               oracle.LD_POSITION).ravel()
    assert abs(got[0] - 2.0) < 1e-15
    assert abs(got[1] - 3.4 / 0.9) < 1e-14


@pytest.mark.parametrize("causal", [True, False])
def test_gated_reduces_to_scalar_decay(causal):
    """Every row and position decaying by one a per head is eqs 10-11,
    which the (separately pinned) plain recurrence computes."""
    rng = np.random.default_rng(21)
    B, H, n, d = 2, 3, 40, 6
    q, k, v, _ = inputs(rng, B, H, n, d, d, oracle.MAP_ELU1)
    a = np.array([0.9, 0.5, 0.99])
    want = oracle.forward(q, k, v, oracle.MAP_ELU1, None, a, causal)
    la = np.log(a)
    for mode, lam in ((oracle.LD_CHANNEL, np.repeat(la[:, None], d, 1)),
                      (oracle.LD_POSITION,
                       np.broadcast_to(la[None, :, None], (B, H, n)).copy()),
                      (oracle.LD_BOTH,
                       np.broadcast_to(la[None, :, None, None],
                                       (B, H, n, d)).copy())):
        got = oracle.forward_gated(q, k, v, oracle.MAP_ELU1, None, lam, mode,
                                   causal)
        assert rel_err(got, want) < 1e-13, mode


@pytest.mark.parametrize("mode", MODES)
def test_gated_constant_v_and_full_reset(mode):
    """Constant v gives that constant (positive features, zero initial
    state); gamma = 0 everywhere (lam = -inf) keeps only the current token,
    so out_j = v_j."""
    rng = np.random.default_rng(31)
    B, H, n, d = 1, 2, 30, 4
    q, k, v, _ = inputs(rng, B, H, n, d, d, oracle.MAP_ELU1)
    lam = rand_lam(rng, mode, B, H, n, d)
    c = np.array([1.0, -2.0, 0.5, 3.0])
    vc = np.broadcast_to(c, v.shape).copy()
    got = oracle.forward_gated(q, k, vc, oracle.MAP_ELU1, None, lam, mode)
    assert rel_err(got, vc) < 1e-13
    got = oracle.forward_gated(q, k, v, oracle.MAP_ELU1, None,
                               np.full_like(lam, -np.inf), mode)
    assert rel_err(got, v) < 1e-15


@pytest.mark.parametrize("mode", MODES)
def test_gated_decode_chain_reproduces_forward(mode):
    """Decode steps from a zero state, position by position, equal the
    causal forward (the decode's per-position layouts take one position's
    slice)."""
    rng = np.random.default_rng(41)
    B, H, n, d = 2, 2, 12, 3
    q, k, v, _ = inputs(rng, B, H, n, d, d, oracle.MAP_ELU1)
    lam = rand_lam(rng, mode, B, H, n, d)
    fwd = oracle.forward_gated(q, k, v, oracle.MAP_ELU1, None, lam, mode)
    mu, nu = np.zeros((B, H, d, d)), np.zeros((B, H, d))
    for j in range(n):
        lj = lam if mode == oracle.LD_CHANNEL else lam[:, :, j]
        o, mu, nu = oracle.decode_gated(mu, nu, q[:, :, j], k[:, :, j],
                                        v[:, :, j], oracle.MAP_ELU1, None,
                                        lj, mode)
        assert rel_err(o, fwd[:, :, j]) < 1e-13, j
