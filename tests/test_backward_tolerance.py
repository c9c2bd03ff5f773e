"""Where the bf16 bar of the backward parity tests comes from (CPU only).

The gradients of the causal forward are sums that cancel: for each row t,
sum_s w_ts (q'_t . k'_s)(G_t . [v_s|1]) = 0, because out_t is the weighted
mean of the v_s.  A backward pass whose matrix-core operands are bf16 rounds
G = dout / den, K', Q' and the score tile to 8 significant bits, and it
reads the forward's bf16 output and a denominator accumulated from bf16
features.  Each of those roundings is about 2^-9 relative, and the
cancellation lets it show in the gradient at that order relative to the
gradient's largest element.

This test emulates exactly those roundings in fp64 NumPy (no GPU code) on
the shapes of the GPU parity grid, measures the resulting error of dq, dk,
dv against the oracle, and checks that it stays below half of BF16_BAR:
the bar of the GPU tests is twice the error any bf16-operand implementation
of these formulas shows, not a number fitted to the GPU's results.
"""
import numpy as np
import pytest
import torch

import oracle

BF16_BAR = 3e-2     # max |gpu - oracle| / max |oracle| per gradient, bf16
FP32_BAR = 1e-4     # fp32 storage: the forward's bar


def bf(x):
    return torch.tensor(x).to(torch.bfloat16).double().numpy()


def elu1(x):
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def emulated_bf16_grads(q, k, v, dout, a=None):
    """dq, dk, dv by the dense formulas with every matrix-core operand and
    the forward's out rounded to bf16, and den perturbed by its bf16
    accumulation (one rounding of each feature)."""
    n = q.shape[0]
    qf, kf = elu1(q), elu1(k)
    qb, kb = bf(qf), bf(kf)
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    W = (j <= i).astype(float)
    if a is not None:
        W = W * (1 - a) * a ** np.maximum(i - j, 0)
    P = (qb @ kb.T) * W                      # the forward's bf16 features
    den = P.sum(1)
    out = bf((P @ v) / den[:, None])         # the forward's bf16 output
    G = bf(dout / den[:, None])
    h = bf(-(dout * out).sum(1) / den)
    Vp = np.concatenate([v, np.ones((n, 1))], 1)
    Gp = np.concatenate([G, h[:, None]], 1)
    A = bf((Gp @ Vp.T) * W)                  # score tile, rounded
    dq = (A @ kb) * np.where(q > 0, 1.0, np.exp(np.minimum(q, 0.0)))
    dk = (A.T @ qb) * np.where(k > 0, 1.0, np.exp(np.minimum(k, 0.0)))
    dv = bf(P).T @ G
    return dq, dk, dv


@pytest.mark.parametrize("n,d,decayed", [(1000, 64, False), (700, 128, True),
                                         (17, 32, True), (333, 16, False),
                                         (500, 64, True)])
def test_bf16_roundings_stay_below_half_the_bar(n, d, decayed):
    rng = np.random.default_rng(n + d)
    to_bf = lambda x: bf(x)
    q = to_bf(rng.standard_normal((n, d)))
    k = to_bf(rng.standard_normal((n, d)))
    v = to_bf(rng.standard_normal((n, d)))
    g = to_bf(rng.standard_normal((n, d)))
    a = 0.9 if decayed else None
    ref = oracle.backward(q[None, None], k[None, None], v[None, None],
                          g[None, None], oracle.MAP_ELU1, None,
                          None if a is None else np.array([a]))
    emu = emulated_bf16_grads(q, k, v, g, a)
    for name, e, r in zip(("dq", "dk", "dv"), emu, ref):
        err = np.max(np.abs(e - r[0, 0])) / np.max(np.abs(r[0, 0]))
        assert err <= BF16_BAR / 2, (name, err)
