"""Pins of the oracle's backward pass (gradients of the causal forward),
CPU only.

The backward is the adjoint of the literal recurrence ("2.2 Linear
Attention" eqs 7-11; feature maps of the "Linear attention research 2026"
page).  It is pinned against things other than itself:
  * central finite differences of the (separately pinned) forward oracle,
    every input element, fp64;
  * torch autograd through the dense masked quadratic form (the
    D^-1 (Mask(Q'K'^T) V) of "3.2 Reducing d" eqs 19-27), a different
    formulation differentiated by a library routine;
  * closed forms: constant V gives a constant output, so dq = dk = 0; one
    position gives out = v, so dq = dk = 0 and dv = dout.
"""
import math

import numpy as np
import pytest
import torch

import oracle

MAPS = [oracle.MAP_ELU1, oracle.MAP_PERFORMER, oracle.MAP_IDENTITY]


def rel_err(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def inputs(rng, B, H, n, d, m, mapk, away_from_zero=True):
    dqk = m if mapk == oracle.MAP_IDENTITY else d
    q = rng.standard_normal((B, H, n, dqk)) * 0.7
    k = rng.standard_normal((B, H, n, dqk)) * 0.7
    if mapk == oracle.MAP_IDENTITY:
        q, k = np.abs(q) + 0.05, np.abs(k) + 0.05
    elif away_from_zero:   # keep elu's kink at 0 out of the differences
        q = np.where(np.abs(q) < 0.05, 0.05 * np.sign(q) + 0.05, q)
        k = np.where(np.abs(k) < 0.05, 0.05 * np.sign(k) + 0.05, k)
    v = rng.standard_normal((B, H, n, d))
    om = rng.standard_normal((d, m)) / math.sqrt(d)
    return q, k, v, om


@pytest.mark.parametrize("mapk", MAPS)
@pytest.mark.parametrize("decayed", [False, True])
def test_backward_matches_finite_differences(mapk, decayed):
    rng = np.random.default_rng(3 + mapk + 10 * decayed)
    B, H, n, d, m = 1, 2, 6, 3, 4
    q, k, v, om = inputs(rng, B, H, n, d, m, mapk)
    dec = np.array([0.8, 0.6]) if decayed else None
    g = rng.standard_normal((B, H, n, d))

    def f(q_, k_, v_):
        return float(np.sum(oracle.forward(q_, k_, v_, mapk, om, dec) * g))

    dq, dk, dv = oracle.backward(q, k, v, g, mapk, om, dec)
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num[idx] = (f(*args_p) - f(*args_m)) / (2 * eps)
        assert rel_err(grad, num) < 1e-6, name


def _torch_phi(x, mapk, om):
    if mapk == oracle.MAP_IDENTITY:
        return x
    if mapk == oracle.MAP_ELU1:
        return torch.nn.functional.elu(x) + 1.0
    sq = 0.5 * (x * x).sum(-1, keepdim=True)
    return torch.exp(x @ om - sq) / math.sqrt(om.shape[1])


@pytest.mark.parametrize("mapk", MAPS)
@pytest.mark.parametrize("decayed", [False, True])
def test_backward_matches_autograd_of_dense_form(mapk, decayed):
    rng = np.random.default_rng(7 + mapk + 10 * decayed)
    B, H, n, d, m = 2, 2, 33, 5, 6
    q, k, v, om = inputs(rng, B, H, n, d, m, mapk)
    dec = np.array([0.9, 0.5]) if decayed else None
    g = rng.standard_normal((B, H, n, d))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    tom = torch.tensor(om)
    qf, kf = _torch_phi(tq, mapk, tom), _torch_phi(tk, mapk, tom)
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    mask = (j <= i).double()
    if dec is None:
        W = mask.expand(H, n, n)
    else:
        a = torch.tensor(dec)[:, None, None]
        W = mask * (1 - a) * a ** (i - j).clamp(min=0).double()
    A = (qf @ kf.transpose(-1, -2)) * W             # [B, H, n, n]
    out = (A @ tv) / A.sum(-1, keepdim=True)
    (out * torch.tensor(g)).sum().backward()
    dq, dk, dv = oracle.backward(q, k, v, g, mapk, om, dec)
    assert rel_err(dq, tq.grad.numpy()) < 1e-11
    assert rel_err(dk, tk.grad.numpy()) < 1e-11
    assert rel_err(dv, tv.grad.numpy()) < 1e-11


@pytest.mark.parametrize("decayed", [False, True])
def test_backward_constant_v_and_single_position(decayed):
    rng = np.random.default_rng(11)
    B, H, n, d = 1, 2, 20, 4
    q, k, v, _ = inputs(rng, B, H, n, d, d, oracle.MAP_ELU1)
    dec = np.array([0.7, 0.95]) if decayed else None
    g = rng.standard_normal((B, H, n, d))
    c = np.array([1.0, -2.0, 0.5, 3.0])
    vc = np.broadcast_to(c, v.shape).copy()
    dq, dk, dv = oracle.backward(q, k, vc, g, oracle.MAP_ELU1, None, dec)
    scale = np.max(np.abs(dv))
    assert np.max(np.abs(dq)) < 1e-12 * scale
    assert np.max(np.abs(dk)) < 1e-12 * scale
    # one position: out = v
    dq, dk, dv = oracle.backward(q[:, :, :1], k[:, :, :1], v[:, :, :1],
                                 g[:, :, :1], oracle.MAP_ELU1, None, dec)
    assert np.max(np.abs(dq)) < 1e-14 and np.max(np.abs(dk)) < 1e-14
    assert rel_err(dv, g[:, :, :1]) < 1e-14


# ---- the gated recurrence (a decay per position, per state row, or both) --

LD_MODES = [oracle.LD_POSITION, oracle.LD_CHANNEL, oracle.LD_BOTH]


def _log_decay(rng, mode, B, H, n, df):
    """log gamma in (log 0.3, log 0.99) for the given layout."""
    shape = {oracle.LD_POSITION: (B, H, n), oracle.LD_CHANNEL: (H, df),
             oracle.LD_BOTH: (B, H, n, df)}[mode]
    return np.log(rng.uniform(0.3, 0.99, size=shape))


@pytest.mark.parametrize("mode", LD_MODES)
@pytest.mark.parametrize("mapk", [oracle.MAP_ELU1, oracle.MAP_PERFORMER])
def test_gated_backward_matches_finite_differences(mode, mapk):
    rng = np.random.default_rng(19 + mode + 5 * mapk)
    B, H, n, d, m = 1, 2, 6, 3, 4
    q, k, v, om = inputs(rng, B, H, n, d, m, mapk)
    df = m if mapk == oracle.MAP_PERFORMER else d
    lam = _log_decay(rng, mode, B, H, n, df)
    g = rng.standard_normal((B, H, n, d))

    def f(q_, k_, v_):
        return float(np.sum(oracle.forward_gated(q_, k_, v_, mapk, om, lam,
                                                 mode) * g))

    dq, dk, dv = oracle.backward_gated(q, k, v, g, mapk, om, lam, mode)
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num[idx] = (f(*args_p) - f(*args_m)) / (2 * eps)
        assert rel_err(grad, num) < 1e-6, name


def test_gated_backward_matches_autograd_of_dense_form():
    """A decay per position: weights w_ij = (1 - g_j) prod_{j<u<=i} g_u in
    the dense masked form, differentiated by torch."""
    rng = np.random.default_rng(23)
    B, H, n, d = 2, 2, 29, 5
    mapk = oracle.MAP_ELU1
    q, k, v, om = inputs(rng, B, H, n, d, d, mapk)
    lam = _log_decay(rng, oracle.LD_POSITION, B, H, n, d)
    g = rng.standard_normal((B, H, n, d))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    qf, kf = _torch_phi(tq, mapk, None), _torch_phi(tk, mapk, None)
    tl = torch.tensor(lam)
    cs = torch.cumsum(tl, -1)                        # sum_{u<=i} log g_u
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    diff = (cs[..., :, None] - cs[..., None, :]).masked_fill(j > i, -1e300)
    W = torch.exp(diff) * (1 - torch.exp(tl))[..., None, :]
    A = (qf @ kf.transpose(-1, -2)) * W
    out = (A @ tv) / A.sum(-1, keepdim=True)
    (out * torch.tensor(g)).sum().backward()
    dq, dk, dv = oracle.backward_gated(q, k, v, g, mapk, None, lam,
                                       oracle.LD_POSITION)
    assert rel_err(dq, tq.grad.numpy()) < 1e-11
    assert rel_err(dk, tk.grad.numpy()) < 1e-11
    assert rel_err(dv, tv.grad.numpy()) < 1e-11


def test_gated_backward_with_one_decay_per_head_is_the_plain_one():
    """Every position of head h at log a_h: the gated adjoint must give the
    per-head adjoint exactly (up to rounding)."""
    rng = np.random.default_rng(29)
    B, H, n, d = 2, 2, 40, 4
    q, k, v, _ = inputs(rng, B, H, n, d, d, oracle.MAP_ELU1)
    a = np.array([0.9, 0.65])
    lam = np.broadcast_to(np.log(a)[None, :, None], (B, H, n)).copy()
    g = rng.standard_normal((B, H, n, d))
    got = oracle.backward_gated(q, k, v, g, oracle.MAP_ELU1, None, lam,
                                oracle.LD_POSITION)
    ref = oracle.backward(q, k, v, g, oracle.MAP_ELU1, None, a)
    for x, y in zip(got, ref):
        assert rel_err(x, y) < 1e-12
