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
