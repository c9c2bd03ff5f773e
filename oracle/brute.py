"""Dense quadratic-form evaluation of kernelized attention (fp64 NumPy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

This is the brute-force pin of the recurrence oracle.  It never forms a
running state: it builds the full n x n similarity matrix and normalises it
row by row, which is the definition the recurrence regroups:

* "3.2 Reducing d" (efficient1 page), eqs 19-21: Att = D^-1 Mask(A~) V with
  D_ii the row sums of the masked similarity matrix; eq 22: A~(i, j) =
  <phi(q_i), phi(k_j)>; eqs 25-26: c_i = sum_j alpha_ij v_j.
* Causal mask of eq 2 on the same page: M(i, j) = 0 for j <= i, else -inf,
  i.e. position i sees positions 1..i including itself.
* With a decay a ("2.2 Linear Attention", eqs 10-11 on the efficient2 page)
  and a zero initial state, unrolling the recurrence gives the weight
  (1 - a) a^(i - j) on the pair (i, j); the non-causal readout (eq 9 with the
  final state) puts weight (1 - a) a^(n - j) on key j for every query.

Cost O(n^2 d) time and O(n^2) memory per unit: for n up to a few hundred.
"""
from __future__ import annotations

import numpy as np

MAP_IDENTITY, MAP_ELU1, MAP_PERFORMER = 0, 1, 2


def features(x, mapk: int, omega=None) -> np.ndarray:
    """phi over the last axis, vectorised NumPy fp64.

    ELU1 is elu(x) + 1 with alpha = 1; PERFORMER is
    exp(x omega - |x|^2 / 2) / sqrt(m) with omega [d, m]; IDENTITY passes x
    through ("Linear attention research 2026" page, Performer and Linear
    Transformer sections)."""
    x = np.asarray(x, dtype=np.float64)
    if mapk == MAP_IDENTITY:
        return x.copy()
    if mapk == MAP_ELU1:
        return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))
    om = np.asarray(omega, dtype=np.float64)
    m = om.shape[1]
    sq = 0.5 * np.sum(x * x, axis=-1, keepdims=True)
    return np.exp(x @ om - sq) / np.sqrt(m)


def pair_weights(n: int, a=None, causal: bool = True) -> np.ndarray:
    """[n, n] weight matrix W with out_i = sum_j W_ij s_ij v_j / sum_j W_ij s_ij.

    0-based positions.  No decay: W_ij = 1 on the mask.  Decay a:
    W_ij = (1 - a) a^(i - j) for j <= i (causal) or (1 - a) a^(n - 1 - j)
    (non-causal, every row reads the final state)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    if causal:
        mask = (j <= i).astype(np.float64)
        lag = np.where(j <= i, i - j, 0)
    else:
        mask = np.ones((n, n))
        lag = np.broadcast_to((n - 1) - j, (n, n))
    if a is None:
        return mask
    a = float(a)
    return mask * (1.0 - a) * np.power(a, lag.astype(np.float64))


def masked_quadratic(qf, kf, v, decay=None, causal: bool = True) -> np.ndarray:
    """Att = D^-1 ((W o Q'K'^T) V) per (batch, head).

    qf, kf: [B, H, n, d_feat] features; v: [B, H, n, d]; decay: [H] or None."""
    qf = np.asarray(qf, dtype=np.float64)
    kf = np.asarray(kf, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, n, d = v.shape
    out = np.empty((B, H, n, d))
    for h in range(H):
        W = pair_weights(n, None if decay is None else np.asarray(decay)[h],
                         causal)
        for b in range(B):
            A = (qf[b, h] @ kf[b, h].T) * W          # masked similarity
            D = A.sum(axis=1, keepdims=True)           # row normaliser
            out[b, h] = (A @ v[b, h]) / D
    return out


def attention(q, k, v, mapk: int = MAP_ELU1, omega=None, decay=None,
              causal: bool = True) -> np.ndarray:
    """Brute-force kernelized attention straight from the raw q, k, v."""
    return masked_quadratic(features(q, mapk, omega), features(k, mapk, omega),
                            v, decay, causal)


def gated_weights(lam_full, causal: bool = True) -> np.ndarray:
    """[n, n, d_feat] weights of the gated recurrence, by explicit products.

    lam_full: [n, d_feat] log decay of every state row at every position.
    Entry (i, j, f) is the weight of key j in row i on feature f: the input
    weight 1 - gamma_{j,f} times the product of gamma_{l,f} over the
    positions l after j up to i (causal), or up to the last position
    (non-causal: every row reads the final state).  "2.2 Linear Attention"
    eqs 10-11 per state row, "2.3 State-Space Models" eqs 16-17 (powers of
    the diagonal A) with the selective, per-position decay."""
    g = np.exp(np.asarray(lam_full, dtype=np.float64))
    n, df = g.shape
    W = np.zeros((n, n, df))
    for i in range(n):
        for j in range(n):
            if causal and j > i:
                continue
            last = i if causal else n - 1
            W[i, j] = (1.0 - g[j]) * np.prod(g[j + 1:last + 1], axis=0)
    return W


def gated_quadratic(qf, kf, v, lam_full, causal: bool = True) -> np.ndarray:
    """Att_i = sum_j sum_f q'_if k'_jf W_ijf v_j / sum_j sum_f q'_if k'_jf W_ijf
    per (batch, head); lam_full is [B, H, n, d_feat] (broadcast the per-
    channel or per-position layouts to it first)."""
    qf = np.asarray(qf, dtype=np.float64)
    kf = np.asarray(kf, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, n, d = v.shape
    out = np.empty((B, H, n, d))
    for b in range(B):
        for h in range(H):
            W = gated_weights(lam_full[b, h], causal)
            A = np.einsum("if,jf,ijf->ij", qf[b, h], kf[b, h], W)
            out[b, h] = (A @ v[b, h]) / A.sum(axis=1, keepdims=True)
    return out
