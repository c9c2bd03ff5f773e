"""fp64 CPU oracle for causal kernelized linear attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library under ``kernelized_attention_scan_amd/``; neither imports
the other.

Two independent formulations live here:

* ``forward`` / ``decode`` / ``featmap`` -- the literal per-position
  recurrence of "2.2 Linear Attention" eqs 7-11 (efficient2 page), written in
  plain C (``linattn_oracle.c``), fp64, OpenMP over the independent
  (batch, head) units.
* ``brute.masked_quadratic`` -- the quadratic form D^-1 (Mask(Q'K'^T) V) of
  "3.2 Reducing d" eqs 19-27 (efficient1 page) with the causal mask of eq 2,
  evaluated densely with NumPy in fp64.  It is the brute-force pin of the
  recurrence at small n.

Inputs are NumPy arrays (any float dtype; widened to fp64 here).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import brute  # noqa: F401  (re-exported)

MAP_IDENTITY, MAP_ELU1, MAP_PERFORMER = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "linattn_oracle.c")
_LIB = os.path.join(_HERE, "liblinattn_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, IEEE: no fast-math) and OpenMP."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-std=c99", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.POINTER(ctypes.c_double)
        i64, i32 = ctypes.c_int64, ctypes.c_int
        lib.oracle_featmap.argtypes = [P, P, P, i64, i32, i32, i32]
        lib.oracle_forward.argtypes = [P, P, P, P, i32, i32, i64, i32, i32,
                                       i32, i32, P, P, i32]
        lib.oracle_decode.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32,
                                      i32, i32, P, P]
        lib.oracle_forward_gated.argtypes = [P, P, P, P, i32, i32, i64, i32,
                                             i32, i32, i32, P, P, i32, i32]
        lib.oracle_decode_gated.argtypes = [P, P, P, P, P, P, i32, i32, i32,
                                            i32, i32, i32, P, P, i32]
        lib.oracle_backward.argtypes = [P, P, P, P, P, P, P, i32, i32, i64,
                                        i32, i32, i32, i32, P, P]
        lib.oracle_backward_gated.argtypes = [P, P, P, P, P, P, P, i32, i32,
                                              i64, i32, i32, i32, i32, P, P,
                                              i32]
        lib.oracle_num_threads.restype = i32
        _lib = lib
    return _lib


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def feat_dim(d: int, mapk: int, omega) -> int:
    return int(np.asarray(omega).shape[1]) if mapk == MAP_PERFORMER else d


def featmap(x, mapk: int, omega=None) -> np.ndarray:
    """Row-wise phi over the last axis: [..., d] -> [..., d_feat]."""
    x = _f64(x)
    d = x.shape[-1]
    om = _f64(omega) if mapk == MAP_PERFORMER else None
    df = feat_dim(d, mapk, om)
    rows = x.size // d
    y = np.empty(x.shape[:-1] + (df,), dtype=np.float64)
    _load().oracle_featmap(_ptr(x), _ptr(y), _ptr(om), rows, d, df, mapk)
    return y


def forward(q, k, v, mapk: int = MAP_ELU1, omega=None, decay=None,
            causal: bool = True) -> np.ndarray:
    """Literal recurrence over q, k [B, H, n, d_qk] and v [B, H, n, d].

    d_qk = d for ELU1 and PERFORMER; for IDENTITY, q and k are already
    features and d_qk = d_feat.  decay is [H] (one a per head) or None."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, n, d = v.shape
    dqk = q.shape[-1]
    assert q.shape == k.shape == (B, H, n, dqk)
    om = _f64(omega) if mapk == MAP_PERFORMER else None
    df = feat_dim(dqk, mapk, om)
    if mapk == MAP_ELU1:
        assert dqk == d
    dec = None if decay is None else _f64(decay).reshape(H)
    out = np.empty((B, H, n, d), dtype=np.float64)
    _load().oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, n, d,
                           dqk, df, mapk, _ptr(om), _ptr(dec),
                           int(bool(causal)))
    return out


def backward(q, k, v, dout, mapk: int = MAP_ELU1, omega=None, decay=None):
    """Gradients (dq, dk, dv) of sum(out * dout) for the causal forward:
    the adjoint of the literal recurrence, position by position (see
    linattn_oracle.c)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, n, d = v.shape
    dqk = q.shape[-1]
    assert q.shape == k.shape == (B, H, n, dqk) and dout.shape == v.shape
    om = _f64(omega) if mapk == MAP_PERFORMER else None
    df = feat_dim(dqk, mapk, om)
    if mapk == MAP_ELU1:
        assert dqk == d
    dec = None if decay is None else _f64(decay).reshape(H)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    _load().oracle_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq),
                            _ptr(dk), _ptr(dv), B, H, n, d, dqk, df, mapk,
                            _ptr(om), _ptr(dec))
    return dq, dk, dv


# Layouts of the log decay of the gated recurrence (see linattn_oracle.c).
LD_CHANNEL, LD_POSITION, LD_BOTH = 0, 1, 2


def forward_gated(q, k, v, mapk: int, omega, log_decay, mode: int,
                  causal: bool = True) -> np.ndarray:
    """The recurrence with decay gamma = exp(log_decay) per state row
    (LD_CHANNEL: [H, d_feat]), per position (LD_POSITION: [B, H, n]) or per
    both (LD_BOTH: [B, H, n, d_feat]); input weight 1 - gamma (eqs 10-11
    per row, "2.3 State-Space Models" eqs 14 and 21-25; Mamba's selective
    decay)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, n, d = v.shape
    dqk = q.shape[-1]
    assert q.shape == k.shape == (B, H, n, dqk)
    om = _f64(omega) if mapk == MAP_PERFORMER else None
    df = feat_dim(dqk, mapk, om)
    lam = _f64(log_decay)
    want = {LD_CHANNEL: (H, df), LD_POSITION: (B, H, n),
            LD_BOTH: (B, H, n, df)}[mode]
    assert lam.shape == want, (lam.shape, want)
    out = np.empty((B, H, n, d), dtype=np.float64)
    _load().oracle_forward_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H,
                                 n, d, dqk, df, mapk, _ptr(om), _ptr(lam),
                                 mode, int(bool(causal)))
    return out


def backward_gated(q, k, v, dout, mapk: int, omega, log_decay, mode: int):
    """Gradients (dq, dk, dv) of sum(out * dout) for the causal gated
    forward (forward_gated's log_decay and mode): the adjoint with each
    position's and row's decay in place of one per head (see
    linattn_oracle.c).  The decay is not differentiated."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, n, d = v.shape
    dqk = q.shape[-1]
    assert q.shape == k.shape == (B, H, n, dqk) and dout.shape == v.shape
    om = _f64(omega) if mapk == MAP_PERFORMER else None
    df = feat_dim(dqk, mapk, om)
    lam = _f64(log_decay)
    want = {LD_CHANNEL: (H, df), LD_POSITION: (B, H, n),
            LD_BOTH: (B, H, n, df)}[mode]
    assert lam.shape == want, (lam.shape, want)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    _load().oracle_backward_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                  _ptr(dq), _ptr(dk), _ptr(dv), B, H, n, d,
                                  dqk, df, mapk, _ptr(om), _ptr(lam), mode)
    return dq, dk, dv


def decode_gated(mu, nu, q, k, v, mapk: int, omega, log_decay, mode: int):
    """One decode step of the gated recurrence; log_decay is [H, d_feat]
    (LD_CHANNEL), [S, H] (LD_POSITION) or [S, H, d_feat] (LD_BOTH).
    Returns (out, mu_new, nu_new); the inputs are not modified."""
    mu, nu = _f64(mu).copy(), _f64(nu).copy()
    q, k, v = _f64(q), _f64(k), _f64(v)
    S, H, d = v.shape
    dqk = q.shape[-1]
    om = _f64(omega) if mapk == MAP_PERFORMER else None
    df = mu.shape[2]
    assert df == feat_dim(dqk, mapk, om)
    lam = _f64(log_decay)
    want = {LD_CHANNEL: (H, df), LD_POSITION: (S, H), LD_BOTH: (S, H, df)}[mode]
    assert lam.shape == want, (lam.shape, want)
    out = np.empty((S, H, d), dtype=np.float64)
    _load().oracle_decode_gated(_ptr(mu), _ptr(nu), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(out), S, H, d, dqk, df, mapk, _ptr(om),
                                _ptr(lam), mode)
    return out, mu, nu


def decode(mu, nu, q, k, v, mapk: int = MAP_ELU1, omega=None, decay=None):
    """One decode step.  mu [S,H,d_feat,d], nu [S,H,d_feat], q,k [S,H,d_qk],
    v [S,H,d].  Returns (out, mu_new, nu_new); the inputs are not modified."""
    mu, nu = _f64(mu).copy(), _f64(nu).copy()
    q, k, v = _f64(q), _f64(k), _f64(v)
    S, H, d = v.shape
    dqk = q.shape[-1]
    om = _f64(omega) if mapk == MAP_PERFORMER else None
    df = mu.shape[2]
    assert df == feat_dim(dqk, mapk, om)
    assert mu.shape == (S, H, df, d) and nu.shape == (S, H, df)
    assert q.shape == k.shape == (S, H, dqk)
    dec = None if decay is None else _f64(decay).reshape(H)
    out = np.empty((S, H, d), dtype=np.float64)
    _load().oracle_decode(_ptr(mu), _ptr(nu), _ptr(q), _ptr(k), _ptr(v),
                          _ptr(out), S, H, d, dqk, df, mapk, _ptr(om),
                          _ptr(dec))
    return out, mu, nu
