"""Pins of the fp64 oracle against values fixed by the pages and by maths.

Nothing here runs on a GPU or touches the HIP library.  Each test states what
it pins and where the fact comes from:

* "2.2 Linear Attention" (efficient2 page) eqs 7-11: the running sums and the
  decayed sums, the readout q'mu / q'nu and its causal form;
* "3.2 Reducing d" (efficient1 page) eqs 19-27: the dense form
  D^-1 (Mask(Q'K'^T) V), with the causal mask of eq 2 (diagonal included);
* "Linear attention research 2026" page: elu(x) + 1 and the Performer
  features exp(x omega - |x|^2/2)/sqrt(m).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute

MAPS = [oracle.MAP_ELU1, oracle.MAP_PERFORMER, oracle.MAP_IDENTITY]


def rel_err(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def rand_inputs(B, H, n, d, m, mapk, seed, qk_std=0.7):
    rng = np.random.default_rng(seed)
    dqk = m if mapk == oracle.MAP_IDENTITY else d
    q = rng.standard_normal((B, H, n, dqk)) * qk_std
    k = rng.standard_normal((B, H, n, dqk)) * qk_std
    if mapk == oracle.MAP_IDENTITY:      # identity features must be positive
        q, k = np.abs(q) + 0.05, np.abs(k) + 0.05
    v = rng.standard_normal((B, H, n, d))
    omega = rng.standard_normal((d, m)) / math.sqrt(d)
    decay = 1.0 - 10.0 ** rng.uniform(-3, -0.3, size=H)
    return q, k, v, omega, decay


# --------------------------------------------------------------------------
# Feature maps
# --------------------------------------------------------------------------

def test_elu1_matches_library_elu():
    """phi = elu(x) + 1 with alpha = 1: compare with torch's elu (fp64)."""
    x = np.concatenate([np.linspace(-30, 30, 4001), [0.0, -0.0, 1e-300,
                                                     -1e-300, -700.0]])
    ref = (torch.nn.functional.elu(torch.tensor(x, dtype=torch.float64),
                                   alpha=1.0) + 1.0).numpy()
    got = oracle.featmap(x.reshape(-1, 1), oracle.MAP_ELU1).ravel()
    assert np.array_equal(got, ref) or rel_err(got, ref) < 1e-15


def test_elu1_hand_values():
    x = np.array([[0.0, 1.0, -1.0, 2.5]])
    got = oracle.featmap(x, oracle.MAP_ELU1)[0]
    assert got[0] == 1.0 and got[1] == 2.0 and got[3] == 3.5
    assert abs(got[2] - math.exp(-1.0)) < 1e-16


def test_feature_maps_positive():
    """Both maps are positive everywhere (exp > 0; elu + 1 > 0), so every
    denominator q' . nu is positive."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((500, 16)) * 6
    om = rng.standard_normal((16, 32)) / 4
    assert np.all(oracle.featmap(x, oracle.MAP_ELU1) > 0)
    assert np.all(oracle.featmap(x * 0.2, oracle.MAP_PERFORMER, om) > 0)


def test_performer_hand_values():
    """omega with one non-zero entry, omega[0][1] = 1: for x = t e_0 the
    projection is u_1 = t, u_r = 0 otherwise, so phi_1 = exp(t - t^2/2)/sqrt(m)
    and phi_r = exp(-t^2/2)/sqrt(m).  A transposed omega would put u at r = 0.
    """
    d, m, t = 4, 6, 0.8
    om = np.zeros((d, m))
    om[0, 1] = 1.0
    x = np.zeros((1, d))
    x[0, 0] = t
    got = oracle.featmap(x, oracle.MAP_PERFORMER, om)[0]
    base = math.exp(-t * t / 2) / math.sqrt(m)
    want = np.full(m, base)
    want[1] = math.exp(t - t * t / 2) / math.sqrt(m)
    assert rel_err(got, want) < 1e-15
    # x = 0 gives 1/sqrt(m) everywhere; omega = 0 gives exp(-|x|^2/2)/sqrt(m)
    z = oracle.featmap(np.zeros((1, d)), oracle.MAP_PERFORMER, om)[0]
    assert np.allclose(z, 1 / math.sqrt(m), rtol=1e-15, atol=0)
    y = np.array([[0.3, -0.4, 1.2, 0.0]])
    w = oracle.featmap(y, oracle.MAP_PERFORMER, np.zeros((d, m)))[0]
    assert np.allclose(w, math.exp(-0.5 * 1.69) / math.sqrt(m), rtol=1e-14)


def _mean_kernel_z(q, k, sigma, m, seed):
    """z-score of phi(q).phi(k) against E_omega[.] for omega ~ N(0, sigma^2).

    phi(q).phi(k) = (1/m) sum_r X_r with X_r = exp(omega_r.(q+k) -
    (|q|^2+|k|^2)/2); E[X] = exp(sigma^2 |q+k|^2/2 - (|q|^2+|k|^2)/2)."""
    d = q.size
    rng = np.random.default_rng(seed)
    om = rng.standard_normal((d, m)) * sigma
    fq = oracle.featmap(q[None], oracle.MAP_PERFORMER, om)[0]
    fk = oracle.featmap(k[None], oracle.MAP_PERFORMER, om)[0]
    est = float(fq @ fk)
    X = fq * fk * m                   # the m per-feature samples
    se = X.std(ddof=1) / math.sqrt(m)
    s = q + k
    exact = math.exp(sigma ** 2 * (s @ s) / 2 - (q @ q + k @ k) / 2)
    return (est - exact) / se, est, exact


def test_performer_mean_kernel_is_softmax_kernel():
    """With omega ~ N(0, I) the features are unbiased for exp(q . k) (the
    page's "unbiased, exact as the feature count grows")."""
    rng = np.random.default_rng(11)
    d = 8
    for trial in range(4):
        q = rng.standard_normal(d) * 0.15
        k = rng.standard_normal(d) * 0.15
        z, est, exact = _mean_kernel_z(q, k, 1.0, 40000, 100 + trial)
        assert abs(z) < 5, (z, est, exact)
        assert abs(exact - math.exp(q @ k)) < 1e-12 * exact
        # the estimate must approach exp(q.k): far tighter than a scale error
        assert abs(est / math.exp(q @ k) - 1) < 0.02


def test_performer_mean_kernel_sigma_one_over_d():
    """The draw used by the page's code (omega = randn / sqrt(d)) and the
    workload's input scale: the mean kernel is the closed form with
    sigma^2 = 1/d, not exp(q . k)."""
    rng = np.random.default_rng(12)
    d = 64
    q = rng.standard_normal(d) * 0.5
    k = rng.standard_normal(d) * 0.5
    z, est, exact = _mean_kernel_z(q, k, 1 / math.sqrt(d), 65536, 7)
    assert abs(z) < 5, (z, est, exact)


# --------------------------------------------------------------------------
# Hand-derived tiny examples (inline derivations)
# --------------------------------------------------------------------------

def test_hand_example_scalar_no_decay():
    """d = d' = 1, identity map, q' = 1, k' = (1, 2, 3), v = (2, 4, 6).
    mu_j = sum k'v = 2, 10, 28;  nu_j = 1, 3, 6.
    causal out = 2, 10/3, 28/6; non-causal out = 28/6 everywhere (eq 9)."""
    q = np.ones((1, 1, 3, 1))
    k = np.array([1.0, 2.0, 3.0]).reshape(1, 1, 3, 1)
    v = np.array([2.0, 4.0, 6.0]).reshape(1, 1, 3, 1)
    for fn in (oracle.forward, brute.attention):
        c = fn(q, k, v, oracle.MAP_IDENTITY, causal=True).ravel()
        assert np.allclose(c, [2.0, 10 / 3, 28 / 6], rtol=1e-15, atol=0)
        nc = fn(q, k, v, oracle.MAP_IDENTITY, causal=False).ravel()
        assert np.allclose(nc, [28 / 6] * 3, rtol=1e-15, atol=0)


def test_hand_example_scalar_decay():
    """Same inputs, a = 0.5 (eqs 10-11): mu = 0.5 mu + 0.5 k'v,
    nu = 0.5 nu + 0.5 k'.  mu_j = 1, 4.5, 11.25; nu_j = 0.5, 1.25, 2.125.
    causal out = 2, 3.6, 11.25/2.125; non-causal = 11.25/2.125 everywhere."""
    q = np.ones((1, 1, 3, 1))
    k = np.array([1.0, 2.0, 3.0]).reshape(1, 1, 3, 1)
    v = np.array([2.0, 4.0, 6.0]).reshape(1, 1, 3, 1)
    a = np.array([0.5])
    for fn in (oracle.forward, brute.attention):
        c = fn(q, k, v, oracle.MAP_IDENTITY, decay=a, causal=True).ravel()
        assert np.allclose(c, [2.0, 3.6, 11.25 / 2.125], rtol=1e-15, atol=0)
        nc = fn(q, k, v, oracle.MAP_IDENTITY, decay=a, causal=False).ravel()
        assert np.allclose(nc, [11.25 / 2.125] * 3, rtol=1e-15, atol=0)


def test_hand_example_two_features():
    """d' = 2 so the query matters: q' = k' = (1,0), (0,1), (1,1); v = 1, 2, 3.
    Row 0 sees key 0 (score 1): out 1.  Row 1 sees scores 0, 1: out 2.
    Row 2 sees scores 1, 1, 2: out (1 + 2 + 6) / 4 = 9/4."""
    f = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]]).reshape(1, 1, 3, 2)
    v = np.array([1.0, 2.0, 3.0]).reshape(1, 1, 3, 1)
    for fn in (oracle.forward, brute.attention):
        c = fn(f, f, v, oracle.MAP_IDENTITY, causal=True).ravel()
        assert np.allclose(c, [1.0, 2.0, 2.25], rtol=1e-15, atol=0)
    # value dimension 2 with v = (v, -2v): each column is read out separately
    v2 = np.concatenate([v, -2 * v], axis=-1)
    c2 = oracle.forward(f, f, v2, oracle.MAP_IDENTITY).reshape(3, 2)
    assert np.allclose(c2[:, 0], [1.0, 2.0, 2.25], rtol=1e-15)
    assert np.allclose(c2[:, 1], [-2.0, -4.0, -4.5], rtol=1e-15)


def test_hand_example_decode():
    """d = d' = 1: mu = 2, nu = 1, q' = k' = 1, v = 4, a = 0.5:
    mu' = 0.5*2 + 0.5*4 = 3, nu' = 0.5 + 0.5 = 1, out = 3 (after update)."""
    out, mu, nu = oracle.decode(np.full((1, 1, 1, 1), 2.0), np.ones((1, 1, 1)),
                                np.ones((1, 1, 1)), np.ones((1, 1, 1)),
                                np.full((1, 1, 1), 4.0), oracle.MAP_IDENTITY,
                                decay=np.array([0.5]))
    assert out.item() == 3.0 and mu.item() == 3.0 and nu.item() == 1.0
    out, mu, nu = oracle.decode(np.full((1, 1, 1, 1), 2.0), np.ones((1, 1, 1)),
                                np.ones((1, 1, 1)), np.ones((1, 1, 1)),
                                np.full((1, 1, 1), 4.0), oracle.MAP_IDENTITY)
    assert out.item() == 3.0 and mu.item() == 6.0 and nu.item() == 2.0


# --------------------------------------------------------------------------
# Recurrence vs dense quadratic form
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mapk", MAPS)
@pytest.mark.parametrize("decay", [False, True])
@pytest.mark.parametrize("causal", [True, False])
def test_recurrence_matches_bruteforce(mapk, decay, causal):
    """Eqs 7-11 regroup D^-1 (W o Q'K'^T) V exactly: agree to ~1e-12."""
    for seed, (B, H, n, d, m) in enumerate([(1, 2, 37, 8, 12), (2, 1, 64, 16, 16),
                                            (1, 1, 1, 4, 8)]):
        q, k, v, om, dec = rand_inputs(B, H, n, d, m, mapk, seed)
        dec = dec if decay else None
        got = oracle.forward(q, k, v, mapk, om, dec, causal)
        want = brute.attention(q, k, v, mapk, om, dec, causal)
        assert rel_err(got, want) < 1e-12


def test_bruteforce_tril_matmul():
    """No decay, identity map: the dense form is tril(Q'K'^T) V divided by
    tril(Q'K'^T) 1 -- torch's tril and matmul as an independent route."""
    q, k, v, _, _ = rand_inputs(1, 1, 50, 6, 5, oracle.MAP_IDENTITY, 9)
    Q, K, V = (torch.tensor(t[0, 0]) for t in (q, k, v))
    A = torch.tril(Q @ K.T)
    want = (A @ V) / A.sum(dim=1, keepdim=True)
    assert rel_err(brute.attention(q, k, v, oracle.MAP_IDENTITY)[0, 0],
                   want.numpy()) < 1e-13
    assert rel_err(oracle.forward(q, k, v, oracle.MAP_IDENTITY)[0, 0],
                   want.numpy()) < 1e-12


# --------------------------------------------------------------------------
# Closed forms and invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mapk", [oracle.MAP_ELU1, oracle.MAP_PERFORMER])
@pytest.mark.parametrize("decay", [False, True])
@pytest.mark.parametrize("causal", [True, False])
def test_constant_v_gives_constant_output(mapk, decay, causal):
    """v_j = c for every j: numerator = c * denominator, out_j = c."""
    q, k, v, om, dec = rand_inputs(2, 2, 200, 8, 16, mapk, 21)
    c = np.array([1.5, -0.25, 3.0, 0.0, 7.0, -2.0, 0.5, 1e-3])
    v = np.broadcast_to(c, v.shape).copy()
    got = oracle.forward(q, k, v, mapk, om, dec if decay else None, causal)
    assert np.max(np.abs(got - c)) < 1e-13 * np.max(np.abs(c))


@pytest.mark.parametrize("mapk", [oracle.MAP_ELU1, oracle.MAP_PERFORMER])
@pytest.mark.parametrize("decay", [False, True])
def test_first_position_is_v1(mapk, decay):
    """Causal, zero initial state: position 1 sees only itself, out_1 = v_1."""
    q, k, v, om, dec = rand_inputs(1, 3, 20, 8, 16, mapk, 22)
    got = oracle.forward(q, k, v, mapk, om, dec if decay else None, True)
    assert rel_err(got[:, :, 0], v[:, :, 0]) < 1e-15


def test_decay_zero_gives_v():
    """a = 0: mu_j = k'_j^T v_j, nu_j = k'_j, so out_j = v_j exactly."""
    q, k, v, om, _ = rand_inputs(1, 2, 40, 8, 16, oracle.MAP_ELU1, 23)
    got = oracle.forward(q, k, v, oracle.MAP_ELU1, decay=np.zeros(2))
    assert rel_err(got, v) < 1e-15


def test_decay_near_one_tends_to_plain_sums():
    """Zero initial state: the (1 - a) factor cancels in the ratio, and as
    a -> 1 the weights a^(i-j) -> 1, giving the eq-7 output."""
    q, k, v, _, _ = rand_inputs(1, 2, 60, 8, 16, oracle.MAP_ELU1, 24)
    plain = oracle.forward(q, k, v, oracle.MAP_ELU1)
    near = oracle.forward(q, k, v, oracle.MAP_ELU1,
                          decay=np.full(2, 1.0 - 1e-9))
    assert rel_err(near, plain) < 1e-6


@pytest.mark.parametrize("decay", [False, True])
def test_causal_last_row_equals_noncausal(decay):
    """Both read mu_n, nu_n at the last position (eq 9 vs its causal form)."""
    q, k, v, om, dec = rand_inputs(2, 2, 77, 8, 16, oracle.MAP_PERFORMER, 25)
    dec = dec if decay else None
    c = oracle.forward(q, k, v, oracle.MAP_PERFORMER, om, dec, True)
    nc = oracle.forward(q, k, v, oracle.MAP_PERFORMER, om, dec, False)
    assert rel_err(c[:, :, -1], nc[:, :, -1]) < 1e-13
    assert rel_err(c[:, :, 5], nc[:, :, 5]) > 1e-6  # earlier rows differ


def test_scale_invariances():
    """k' -> c k' for every key, or q'_i -> c_i q'_i per row: unchanged."""
    q, k, v, _, dec = rand_inputs(1, 2, 50, 6, 10, oracle.MAP_IDENTITY, 26)
    base = oracle.forward(q, k, v, oracle.MAP_IDENTITY, decay=dec)
    k2 = oracle.forward(q, k * 37.0, v, oracle.MAP_IDENTITY, decay=dec)
    rs = np.random.default_rng(1).uniform(0.1, 10, size=(1, 2, 50, 1))
    q2 = oracle.forward(q * rs, k, v, oracle.MAP_IDENTITY, decay=dec)
    assert rel_err(k2, base) < 1e-13 and rel_err(q2, base) < 1e-13
    # a per-key scale is NOT an invariance: it re-weights the keys
    kk = k * np.random.default_rng(2).uniform(0.1, 10, size=(1, 2, 50, 1))
    assert rel_err(oracle.forward(q, kk, v, oracle.MAP_IDENTITY, decay=dec),
                   base) > 1e-3


# --------------------------------------------------------------------------
# Decode
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mapk", [oracle.MAP_ELU1, oracle.MAP_PERFORMER])
@pytest.mark.parametrize("decay", [False, True])
def test_decode_chain_reproduces_forward(mapk, decay):
    """Token-by-token decode from a zero state is the causal forward pass
    (the sums maintained and updated as keys and values arrive)."""
    B, H, n, d, m = 2, 3, 30, 8, 16
    q, k, v, om, dec = rand_inputs(B, H, n, d, m, mapk, 31)
    dec = dec if decay else None
    df = m if mapk == oracle.MAP_PERFORMER else d
    mu, nu = np.zeros((B, H, df, d)), np.zeros((B, H, df))
    outs = []
    for j in range(n):
        o, mu, nu = oracle.decode(mu, nu, q[:, :, j], k[:, :, j], v[:, :, j],
                                  mapk, om, dec)
        outs.append(o)
    chain = np.stack(outs, axis=2)
    fwd = oracle.forward(q, k, v, mapk, om, dec, True)
    assert rel_err(chain, fwd) < 1e-13


def test_decode_constant_v_state():
    """mu = nu c^T and v = c: out = c, mu' = nu' c^T, for any a."""
    rng = np.random.default_rng(41)
    S, H, d = 3, 2, 8
    c = rng.standard_normal(d)
    nu = np.abs(rng.standard_normal((S, H, d))) * 100
    mu = nu[..., None] * c
    q, k = rng.standard_normal((S, H, d)), rng.standard_normal((S, H, d))
    v = np.broadcast_to(c, (S, H, d)).copy()
    out, mu2, nu2 = oracle.decode(mu, nu, q, k, v, oracle.MAP_ELU1,
                                  decay=np.array([0.9, 0.99]))
    assert rel_err(out, np.broadcast_to(c, out.shape)) < 1e-13
    assert rel_err(mu2, nu2[..., None] * c) < 1e-13


def test_decode_one_minus_a_matters():
    """In decode the state is not zero, so (1 - a) on the new term does not
    cancel: a = 0.5 and a literal 'a mu + k'v' update differ."""
    rng = np.random.default_rng(42)
    mu = np.abs(rng.standard_normal((1, 1, 4, 4)))
    nu = np.abs(rng.standard_normal((1, 1, 4)))
    q, k, v = (rng.standard_normal((1, 1, 4)) for _ in range(3))
    out, mu2, nu2 = oracle.decode(mu, nu, q, k, v, oracle.MAP_ELU1,
                                  decay=np.array([0.5]))
    kf = np.where(k > 0, k + 1, np.exp(k))[0, 0]
    assert np.allclose(mu2[0, 0], 0.5 * mu[0, 0] + 0.5 * np.outer(kf, v[0, 0]),
                       rtol=1e-15)
    assert not np.allclose(mu2[0, 0], 0.5 * mu[0, 0] + np.outer(kf, v[0, 0]))
