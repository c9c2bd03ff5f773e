"""Planted mistakes in the oracle must be caught by its pins.

Each case copies the oracle's C source, plants one plausible mistake by a
textual edit (a dropped term, a wrong sign, a swapped factor, a transposed
operand, an off-by-one in the mask), compiles the copy into a temporary
library, and runs the pin checks of ``test_oracle_pins`` against it.  The
unmodified source must pass every check; every mutant must fail at least one.
Everything runs on the CPU.
"""
import ctypes
import math
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import brute

SRC = os.path.join(os.path.dirname(oracle.__file__), "linattn_oracle.c")

MUTANTS = {
    "exclusive_mask": (
        "      state_update(mu, nu, kf, vu + j * d, d, dfeat, has_decay, a);\n"
        "      if (causal) {\n"
        "        feature_row(qu + j * dqk, qf, dqk, dfeat, map, omega);\n"
        "        readout(mu, nu, qf, ou + j * d, d, dfeat);\n"
        "      }\n",
        "      if (causal) {\n"
        "        feature_row(qu + j * dqk, qf, dqk, dfeat, map, omega);\n"
        "        readout(mu, nu, qf, ou + j * d, d, dfeat);\n"
        "      }\n"
        "      state_update(mu, nu, kf, vu + j * d, d, dfeat, has_decay, a);\n"),
    "nu_missing_one_minus_a": ("nu[f] = a * nu[f] + b * kf[f];",
                               "nu[f] = a * nu[f] + kf[f];"),
    "decay_factors_swapped": ("a * mu[f * d + e] + b * kf[f] * v[e]",
                              "b * mu[f * d + e] + a * kf[f] * v[e]"),
    "state_transposed_in_readout": ("num += qf[f] * mu[f * d + e];",
                                    "num += qf[f] * mu[e * dfeat + f];"),
    "denominator_dropped": ("out[e] = num / den;", "out[e] = num;"),
    "elu_wrong_sign": ("x > 0.0 ? x + 1.0 : exp(x)",
                       "x > 0.0 ? x + 1.0 : exp(-x)"),
    "elu_no_plus_one": ("x > 0.0 ? x + 1.0 : exp(x)",
                        "x > 0.0 ? x : exp(x) - 1.0"),
    "performer_norm_sign": ("exp(u - 0.5 * sq)", "exp(u + 0.5 * sq)"),
    "performer_no_half": ("exp(u - 0.5 * sq)", "exp(u - sq)"),
    "performer_no_sqrt_m": ("y[r] = exp(u - 0.5 * sq) * inv_sqrt_m;",
                            "y[r] = exp(u - 0.5 * sq);"),
    "performer_omega_transposed": ("omega[(int64_t)c * dfeat + r]",
                                   "omega[(int64_t)r * d + c]"),
    "decode_readout_before_update": (
        "    state_update(muu, nuu, kf, v + u * d, d, dfeat, has_decay, a);\n"
        "    feature_row(q + u * dqk, qf, dqk, dfeat, map, omega);\n"
        "    readout(muu, nuu, qf, out + u * d, d, dfeat);\n",
        "    feature_row(q + u * dqk, qf, dqk, dfeat, map, omega);\n"
        "    readout(muu, nuu, qf, out + u * d, d, dfeat);\n"
        "    state_update(muu, nuu, kf, v + u * d, d, dfeat, has_decay, a);\n"),
    "noncausal_reads_first_state": (
        "    if (!causal) {\n      for (int64_t j = 0; j < n; ++j) {",
        "    if (!causal) {\n      memset(mu, 0, sizeof(double) * dfeat * d);\n"
        "      for (int64_t j = 0; j < n; ++j) {"),
    # planted mistakes in the gated (diagonal / input-dependent) recurrence
    "gated_factors_swapped": ("g * mu[f * d + e] + b * kf[f] * v[e]",
                              "b * mu[f * d + e] + g * kf[f] * v[e]"),
    "gated_nu_no_input_weight": ("nu[f] = g * nu[f] + b * kf[f];",
                                 "nu[f] = g * nu[f] + kf[f];"),
    "gated_channel_ignored": (
        "if (mode == ORC_LD_CHANNEL) return lam[(int64_t)h * dfeat + f];",
        "if (mode == ORC_LD_CHANNEL) return lam[(int64_t)h * dfeat];"),
    "gated_previous_position": (
        "if (mode == ORC_LD_POSITION) return lam[u * n + j];",
        "if (mode == ORC_LD_POSITION) return lam[u * n + (j > 0 ? j - 1 : 0)];"),
    "gated_both_transposed": ("return lam[(u * n + j) * dfeat + f];",
                              "return lam[(u * dfeat + f) * n + j];"),
    "gated_decode_readout_before_update": (
        "    gated_update(muu, nuu, kf, v + u * d, d, dfeat, lam, mode, u, h, 0, 1);\n"
        "    feature_row(q + u * dqk, qf, dqk, dfeat, map, omega);\n"
        "    readout(muu, nuu, qf, out + u * d, d, dfeat);\n",
        "    feature_row(q + u * dqk, qf, dqk, dfeat, map, omega);\n"
        "    readout(muu, nuu, qf, out + u * d, d, dfeat);\n"
        "    gated_update(muu, nuu, kf, v + u * d, d, dfeat, lam, mode, u, h, 0, 1);\n"),
    # planted mistakes in the backward pass
    "bwd_dden_sign": ("dden[j] = -dn / (den * den);",
                      "dden[j] = dn / (den * den);"),
    "bwd_dk_missing_input_weight": ("gf[f] = b * acc;", "gf[f] = acc;"),
    "bwd_elu_chain_rule_dropped": (
        "gx[c] = x[c] > 0.0 ? gf[c] : gf[c] * exp(x[c]);", "gx[c] = gf[c];"),
    "bwd_adjoint_not_decayed": ("for (int e = 0; e < d; ++e) mu[f * d + e] *= gw[f];",
                                ";"),
    "bwd_dv_state_transposed": (
        "for (int f = 0; f < dfeat; ++f) acc += mu[f * d + e] * kf[f] * bw[f];",
        "for (int f = 0; f < dfeat; ++f) acc += mu[e * dfeat + f] * kf[f] * bw[f];"),
    "bwd_performer_norm_term_dropped": ("gx[c] = acc - x[c] * s;",
                                        "gx[c] = acc;"),
}


def _compile(src_text, tmp_path, tag):
    c = tmp_path / f"{tag}.c"
    so = tmp_path / f"lib{tag}.so"
    c.write_text(src_text)
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared",
                           "-std=c99", "-o", str(so), str(c), "-lm"])
    lib = ctypes.CDLL(str(so))
    P = ctypes.POINTER(ctypes.c_double)
    i64, i32 = ctypes.c_int64, ctypes.c_int
    lib.oracle_featmap.argtypes = [P, P, P, i64, i32, i32, i32]
    lib.oracle_forward.argtypes = [P, P, P, P, i32, i32, i64, i32, i32, i32,
                                   i32, P, P, i32]
    lib.oracle_decode.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                  i32, P, P]
    lib.oracle_forward_gated.argtypes = [P, P, P, P, i32, i32, i64, i32, i32,
                                         i32, i32, P, P, i32, i32]
    lib.oracle_decode_gated.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32,
                                        i32, i32, P, P, i32]
    lib.oracle_backward.argtypes = [P, P, P, P, P, P, P, i32, i32, i64, i32,
                                    i32, i32, i32, P, P]
    lib.oracle_num_threads.restype = i32
    return lib


def _close(a, b, tol):
    a, b = np.asarray(a), np.asarray(b)
    if not np.all(np.isfinite(a)):
        return False
    return np.max(np.abs(a - b)) <= tol * max(np.max(np.abs(b)), 1e-300)


# ---- pin checks (each returns True when the pin holds) ---------------------

def chk_bruteforce():
    rng = np.random.default_rng(5)
    for mapk in (oracle.MAP_ELU1, oracle.MAP_PERFORMER, oracle.MAP_IDENTITY):
        for dec in (None, np.array([0.9, 0.7])):
            for causal in (True, False):
                d, m, n = 6, 8, 25
                dqk = m if mapk == oracle.MAP_IDENTITY else d
                q = rng.standard_normal((1, 2, n, dqk)) * 0.7
                k = rng.standard_normal((1, 2, n, dqk)) * 0.7
                if mapk == oracle.MAP_IDENTITY:
                    q, k = np.abs(q) + 0.05, np.abs(k) + 0.05
                v = rng.standard_normal((1, 2, n, d))
                om = rng.standard_normal((d, m)) / math.sqrt(d)
                got = oracle.forward(q, k, v, mapk, om, dec, causal)
                want = brute.attention(q, k, v, mapk, om, dec, causal)
                if not _close(got, want, 1e-12):
                    return False
    return True


def chk_hand_examples():
    q = np.ones((1, 1, 3, 1))
    k = np.array([1.0, 2.0, 3.0]).reshape(1, 1, 3, 1)
    v = np.array([2.0, 4.0, 6.0]).reshape(1, 1, 3, 1)
    ok = _close(oracle.forward(q, k, v, oracle.MAP_IDENTITY).ravel(),
                [2.0, 10 / 3, 28 / 6], 1e-15)
    ok &= _close(oracle.forward(q, k, v, oracle.MAP_IDENTITY,
                                decay=np.array([0.5])).ravel(),
                 [2.0, 3.6, 11.25 / 2.125], 1e-15)
    ok &= _close(oracle.forward(q, k, v, oracle.MAP_IDENTITY,
                                causal=False).ravel(), [28 / 6] * 3, 1e-15)
    return bool(ok)


def chk_featmaps():
    x = np.array([[0.0, 1.0, -1.0, 2.5]])
    e = oracle.featmap(x, oracle.MAP_ELU1)[0]
    if not _close(e, [1.0, 2.0, math.exp(-1.0), 3.5], 1e-15):
        return False
    d, m, t = 4, 6, 0.8
    om = np.zeros((d, m))
    om[0, 1] = 1.0
    xx = np.zeros((1, d))
    xx[0, 0] = t
    want = np.full(m, math.exp(-t * t / 2) / math.sqrt(m))
    want[1] = math.exp(t - t * t / 2) / math.sqrt(m)
    return _close(oracle.featmap(xx, oracle.MAP_PERFORMER, om)[0], want, 1e-15)


def chk_decode():
    out, mu, nu = oracle.decode(np.full((1, 1, 1, 1), 2.0), np.ones((1, 1, 1)),
                                np.ones((1, 1, 1)), np.ones((1, 1, 1)),
                                np.full((1, 1, 1), 4.0), oracle.MAP_IDENTITY,
                                decay=np.array([0.5]))
    return out.item() == 3.0 and mu.item() == 3.0 and nu.item() == 1.0


def chk_constant_v():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 1, 40, 4))
    k = rng.standard_normal((1, 1, 40, 4))
    c = np.array([1.0, -2.0, 0.5, 3.0])
    v = np.broadcast_to(c, (1, 1, 40, 4)).copy()
    for dec in (None, np.array([0.8])):
        if not _close(oracle.forward(q, k, v, oracle.MAP_ELU1, decay=dec),
                      np.broadcast_to(c, v.shape), 1e-13):
            return False
    return True


def chk_gated_bruteforce():
    rng = np.random.default_rng(7)
    B, H, n, d = 1, 2, 17, 4
    for mode in (oracle.LD_CHANNEL, oracle.LD_POSITION, oracle.LD_BOTH):
        for causal in (True, False):
            q = rng.standard_normal((B, H, n, d))
            k = rng.standard_normal((B, H, n, d))
            v = rng.standard_normal((B, H, n, d))
            shape = {oracle.LD_CHANNEL: (H, d), oracle.LD_POSITION: (B, H, n),
                     oracle.LD_BOTH: (B, H, n, d)}[mode]
            lam = rng.uniform(-2.0, -0.05, size=shape)
            full = {oracle.LD_CHANNEL: lambda l: np.broadcast_to(
                        l[None, :, None, :], (B, H, n, d)),
                    oracle.LD_POSITION: lambda l: np.broadcast_to(
                        l[..., None], (B, H, n, d)),
                    oracle.LD_BOTH: lambda l: l}[mode](lam)
            got = oracle.forward_gated(q, k, v, oracle.MAP_ELU1, None, lam,
                                       mode, causal)
            want = brute.gated_quadratic(brute.features(q, oracle.MAP_ELU1),
                                         brute.features(k, oracle.MAP_ELU1),
                                         v, full, causal)
            if not _close(got, want, 1e-12):
                return False
    return True


def chk_gated_decode():
    # one step from mu = [2], nu = [1] with gamma = 0.5: mu' = 0.5 * 2 +
    # 0.5 * 1 * 4 = 3, nu' = 1, out = 3 (every layout)
    for mode, lam in ((oracle.LD_CHANNEL, np.log([[0.5]])),
                      (oracle.LD_POSITION, np.log([[0.5]])),
                      (oracle.LD_BOTH, np.log([[[0.5]]]))):
        out, mu, nu = oracle.decode_gated(
            np.full((1, 1, 1, 1), 2.0), np.ones((1, 1, 1)), np.ones((1, 1, 1)),
            np.ones((1, 1, 1)), np.full((1, 1, 1), 4.0), oracle.MAP_IDENTITY,
            None, lam, mode)
        if not (out.item() == 3.0 and mu.item() == 3.0 and nu.item() == 1.0):
            return False
    # out is read after the update: a new token with a different value
    # moves the output (readout-before-update would return mu / nu = 2)
    out, _, _ = oracle.decode_gated(
        np.full((1, 1, 1, 1), 2.0), np.ones((1, 1, 1)), np.ones((1, 1, 1)),
        np.ones((1, 1, 1)), np.full((1, 1, 1), 10.0), oracle.MAP_IDENTITY,
        None, np.log([[0.5]]), oracle.LD_CHANNEL)
    return out.item() == 6.0


def chk_backward():
    import torch
    rng = np.random.default_rng(9)
    B, H, n, d, m = 1, 2, 21, 4, 5   # d != m: a transposed state is caught
    for mapk in (oracle.MAP_ELU1, oracle.MAP_PERFORMER):
        for dec in (None, np.array([0.8, 0.6])):
            q = rng.standard_normal((B, H, n, d)) * 0.7
            k = rng.standard_normal((B, H, n, d)) * 0.7
            v = rng.standard_normal((B, H, n, d))
            g = rng.standard_normal((B, H, n, d))
            om = rng.standard_normal((d, m)) / math.sqrt(d)
            tq, tk, tv = (torch.tensor(x, requires_grad=True)
                          for x in (q, k, v))
            if mapk == oracle.MAP_ELU1:
                qf = torch.nn.functional.elu(tq) + 1.0
                kf = torch.nn.functional.elu(tk) + 1.0
            else:
                tom = torch.tensor(om)
                qf = torch.exp(tq @ tom - 0.5 * (tq * tq).sum(-1, keepdim=True))
                kf = torch.exp(tk @ tom - 0.5 * (tk * tk).sum(-1, keepdim=True))
                qf, kf = qf / math.sqrt(m), kf / math.sqrt(m)
            i = torch.arange(n)[:, None]
            j = torch.arange(n)[None, :]
            W = (j <= i).double()
            if dec is not None:
                a = torch.tensor(dec)[:, None, None]
                W = W * (1 - a) * a ** (i - j).clamp(min=0).double()
            A = (qf @ kf.transpose(-1, -2)) * W
            out = (A @ tv) / A.sum(-1, keepdim=True)
            (out * torch.tensor(g)).sum().backward()
            got = oracle.backward(q, k, v, g, mapk, om, dec)
            for x, t in zip(got, (tq, tk, tv)):
                if not _close(x, t.grad.numpy(), 1e-10):
                    return False
    return True


CHECKS = [chk_bruteforce, chk_hand_examples, chk_featmaps, chk_decode,
          chk_constant_v, chk_gated_bruteforce, chk_gated_decode,
          chk_backward]


def _run_checks(lib, monkeypatch):
    monkeypatch.setattr(oracle, "_lib", lib)
    return {c.__name__: bool(c()) for c in CHECKS}


def test_unmodified_oracle_passes_all_checks(tmp_path, monkeypatch):
    lib = _compile(open(SRC).read(), tmp_path, "clean")
    res = _run_checks(lib, monkeypatch)
    assert all(res.values()), res


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    lib = _compile(src.replace(old, new), tmp_path, name)
    res = _run_checks(lib, monkeypatch)
    assert not all(res.values()), f"mutant {name} passed every pin: {res}"
