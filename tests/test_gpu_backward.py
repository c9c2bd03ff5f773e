"""GPU parity of the training forward (denominators) and the backward pass
(dq, dk, dv of sum(out * dout), causal) against the fp64 oracle's adjoint
recurrence, through the C ABI.

Tolerance (max |gpu - oracle| / max |oracle| per gradient tensor): 1e-4 for
fp32 storage; for bf16 storage 3e-2, twice the error that the bf16 operand
roundings alone give these cancelling sums (derived on the CPU in
test_backward_tolerance.py).  The forward outputs keep the 1e-2 bar.  The
GPU's backward reads the out and den its own training forward wrote; the
oracle recomputes everything in fp64 from the same storage-rounded inputs.
"""
import numpy as np
import pytest
import torch

import kernelized_attention_scan_amd as K
from kernelized_attention_scan_amd import inputs as I
import oracle

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2}     # forward outputs
GTOL = {torch.float32: 1e-4, torch.bfloat16: 3e-2}    # gradients


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    K.load_library()
    torch.cuda.set_device(0)
    yield


def f64(t):
    return None if t is None else t.detach().cpu().double().numpy()


def dev(t):
    return None if t is None else t.cuda()


def rel(gpu_out, ref):
    g = gpu_out.detach().float().cpu().double().numpy()
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    return float(np.max(np.abs(g - r)) / max(np.max(np.abs(r)), 1e-300))


def make(cfg, seed):
    """Inputs of cfg plus a gradient dout ~ N(0, 1) in the storage type
    (drawn after the prefill inputs, from the next seed)."""
    x = I.make_prefill(cfg, seed)
    if cfg.mapk == I.MAP_IDENTITY:       # positive features of width d
        g = torch.Generator().manual_seed(seed + 1000)
        sh = (cfg.B, cfg.H, cfg.n, cfg.d)
        x["q"] = (torch.rand(sh, generator=g) + 0.05).to(cfg.dtype)
        x["k"] = (torch.rand(sh, generator=g) + 0.05).to(cfg.dtype)
    g = torch.Generator().manual_seed(seed + 7)
    x["dout"] = torch.randn(cfg.B, cfg.H, cfg.n, cfg.d,
                            generator=g).to(cfg.dtype)
    return x


def run(cfg, seed=0):
    x = make(cfg, seed)
    name = I.MAP_NAMES[cfg.mapk]
    q, k, v, dec = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["decay"])
    out, den = K.forward_train(q, k, v, name, decay=dec)
    dq, dk, dv = K.backward(q, k, v, out, den, dev(x["dout"]), name,
                            decay=dec)
    torch.cuda.synchronize()
    return x, out, den, (dq, dk, dv)


GRID = [
    # (name, B, H, n, d, map, decayed)
    ("elu1_ragged", 2, 3, 1000, 64, "elu1", False),
    ("elu1_decay_d128", 1, 2, 700, 128, "elu1", True),
    ("elu1_d32_n17", 1, 2, 17, 32, "elu1", True),
    ("elu1_d16", 2, 2, 333, 16, "elu1", False),
    ("identity_d64", 1, 2, 500, 64, "identity", True),
    ("identity_d128_long", 1, 1, 3000, 128, "identity", False),
    # d = 128 bf16 runs as segmented roles: a ragged tail, one chunk (one
    # segment), and units enough for few segments each
    ("elu1_d128_ragged", 2, 2, 1001, 128, "elu1", False),
    ("elu1_d128_one_chunk", 1, 3, 40, 128, "elu1", True),
    ("elu1_d128_many_units", 8, 8, 300, 128, "elu1", True),
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("case", GRID, ids=[c[0] for c in GRID])
def test_backward_grid(case, dtype):
    name, B, H, n, d, mp, decayed = case
    mapk = I.MAP_ELU1 if mp == "elu1" else I.MAP_IDENTITY
    cfg = I.PrefillConfig(f"bwd_{name}", B=B, H=H, n=n, d=d, dtype=dtype,
                          mapk=mapk, decay=(-2.0, -0.5) if decayed else None)
    x, out, den, grads = run(cfg, seed=5)
    ref = oracle.backward(f64(x["q"]), f64(x["k"]), f64(x["v"]),
                          f64(x["dout"]), mapk, None, f64(x["decay"]))
    errs = [rel(gq, r) for gq, r in zip(grads, ref)]
    print(f"{name} {dtype}: dq {errs[0]:.2e} dk {errs[1]:.2e} "
          f"dv {errs[2]:.2e}", flush=True)
    assert max(errs) <= GTOL[dtype], errs
    # the training forward: out as la_forward, den against the oracle's
    # q'_j . nu_j (nu from its decode chain would be slow: use out * den =
    # num instead, i.e. check den through the forward identity)
    ref_out = oracle.forward(f64(x["q"]), f64(x["k"]), f64(x["v"]), mapk,
                             None, f64(x["decay"]), True)
    assert rel(out, ref_out) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_backward_one_position(dtype):
    """n = 1: out = v whatever q and k are, so dq = dk = 0 and dv = dout
    (the oracle's values are exactly that; relative errors against a zero
    tensor are undefined, so this case is checked against the scale of
    dout / den |v| |k'|)."""
    cfg = I.ELU1_CAUSAL.replace(B=1, H=2, n=1, dtype=dtype,
                                decay=(-2.0, -0.5))
    x, out, den, (dq, dk, dv) = run(cfg, seed=6)
    scale = (x["dout"].abs().max() * x["v"].abs().max()).item()
    assert dq.abs().max().item() <= 1e-5 * scale * 10
    assert dk.abs().max().item() <= 1e-5 * scale * 10
    assert rel(dv, f64(x["dout"])) <= TOL[dtype]


def test_forward_train_denominators_match_oracle():
    """den_j = q'_j . nu_j, nu_j from the oracle's decode chain (eq 8 /
    eq 11 applied position by position)."""
    cfg = I.ELU1_CAUSAL.replace(B=1, H=2, n=300, d=32, dtype=torch.float32,
                                decay=(-2.0, -1.0))
    x = I.make_prefill(cfg, 3)
    out, den = K.forward_train(dev(x["q"]), dev(x["k"]), dev(x["v"]),
                               decay=dev(x["decay"]))
    torch.cuda.synchronize()
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    mu, nu = np.zeros((1, 2, 32, 32)), np.zeros((1, 2, 32))
    ref = np.zeros((1, 2, 300))
    for j in range(300):
        _, mu, nu = oracle.decode(mu, nu, q[:, :, j], k[:, :, j], v[:, :, j],
                                  oracle.MAP_ELU1, None, f64(x["decay"]))
        qf = oracle.featmap(q[:, :, j], oracle.MAP_ELU1)
        ref[:, :, j] = np.sum(qf * nu, axis=-1)
    assert rel(den, ref) <= 1e-4


def test_backward_full_size_every_unit():
    """B=2 H=16 n=65536 d=128 with per-head decay (the decayed workload's
    sizes), every unit and every gradient against the oracle."""
    cfg = I.DECAYED
    x, out, den, grads = run(cfg, seed=0)
    grads = [t.cpu() for t in grads]
    worst = [0.0, 0.0, 0.0]
    for b in range(cfg.B):
        sl = slice(b, b + 1)
        ref = oracle.backward(f64(x["q"][sl]), f64(x["k"][sl]),
                              f64(x["v"][sl]), f64(x["dout"][sl]), cfg.mapk,
                              None, f64(x["decay"]))
        for i in range(3):
            got = grads[i][sl].double().numpy()
            assert np.all(np.isfinite(got))
            for h in range(cfg.H):
                r = ref[i][0, h]
                worst[i] = max(worst[i], np.max(np.abs(got[0, h] - r)) /
                               np.max(np.abs(r)))
        del ref
    print(f"backward full size: max per-unit rel err dq {worst[0]:.2e} "
          f"dk {worst[1]:.2e} dv {worst[2]:.2e}", flush=True)
    assert max(worst) <= GTOL[torch.bfloat16]


PF_GRID = [
    # (name, B, H, n, d, m, dtype, decayed): the Performer map's backward
    # (features, column-block roles over d' = m, then the map's chain rule)
    ("pf_d64_m256_bf16", 1, 2, 300, 64, 256, torch.bfloat16, False),
    ("pf_d64_m256_bf16_decay", 1, 2, 333, 64, 256, torch.bfloat16, True),
    ("pf_d32_m64_fp32", 2, 1, 200, 32, 64, torch.float32, False),
    ("pf_d32_m64_fp32_decay", 1, 2, 129, 32, 64, torch.float32, True),
    ("pf_d128_m128_bf16", 1, 1, 150, 128, 128, torch.bfloat16, True),
    ("pf_d64_m32_fp32_one_chunk", 1, 3, 40, 64, 32, torch.float32, False),
]


@pytest.mark.parametrize("case", PF_GRID, ids=[c[0] for c in PF_GRID])
def test_backward_performer_matches_oracle(case):
    name, B, H, n, d, m, dtype, decayed = case
    cfg = I.PERFORMER.replace(B=B, H=H, n=n, d=d, m=m, dtype=dtype,
                              decay=I.DECAYED.decay if decayed else None)
    x = make(cfg, 31)
    q, k, v, om = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["omega"])
    dec = dev(x["decay"])
    out, den = K.forward_train(q, k, v, "performer", decay=dec, omega=om)
    dq, dk, dv = K.backward(q, k, v, out, den, dev(x["dout"]), "performer",
                            decay=dec, omega=om)
    torch.cuda.synchronize()
    ref_out = oracle.forward(f64(x["q"]), f64(x["k"]), f64(x["v"]),
                             oracle.MAP_PERFORMER, f64(x["omega"]),
                             f64(x["decay"]))
    assert rel(out, ref_out) <= TOL[dtype]
    refs = oracle.backward(f64(x["q"]), f64(x["k"]), f64(x["v"]),
                           f64(x["dout"]), oracle.MAP_PERFORMER,
                           f64(x["omega"]), f64(x["decay"]))
    errs = [rel(t, r) for t, r in zip((dq, dk, dv), refs)]
    print(f"{name}: rel err dq {errs[0]:.2e} dk {errs[1]:.2e} "
          f"dv {errs[2]:.2e}", flush=True)
    assert max(errs) <= GTOL[dtype]


def test_autograd_op_performer_matches_oracle():
    """linear_attention() with the performer map: forward_train through the
    fused map, la_backward's gradients through the map's chain rule."""
    cfg = I.PERFORMER.replace(B=1, H=2, n=257, d=64, m=128,
                              dtype=torch.float32)
    x = make(cfg, 41)
    q, k, v = (dev(x[n]).requires_grad_(True) for n in ("q", "k", "v"))
    om = dev(x["omega"])
    out = K.linear_attention(q, k, v, "performer", omega=om)
    out.backward(dev(x["dout"]))
    torch.cuda.synchronize()
    refs = oracle.backward(f64(x["q"]), f64(x["k"]), f64(x["v"]),
                           f64(x["dout"]), oracle.MAP_PERFORMER,
                           f64(x["omega"]), None)
    for t, r in zip((q, k, v), refs):
        assert rel(t.grad, r) <= GTOL[torch.float32]


def test_backward_performer_rejects_unbuilt_sizes():
    x = torch.zeros(1, 2, 64, 16, dtype=torch.bfloat16, device="cuda")
    den = torch.ones(1, 2, 64, device="cuda")
    om = torch.zeros(16, 64, device="cuda")
    with pytest.raises(K.LinAttnError) as e:
        K.backward(x, x, x, x, den, x, "performer", omega=om)
    assert e.value.status == K._binding.LA_ERR_UNSUPPORTED


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_autograd_op_matches_oracle(dtype):
    """linear_attention() as a torch op: its autograd gradients are those of
    la_backward, checked against the oracle's adjoint."""
    cfg = I.DECAYED.replace(B=1, H=2, n=333, d=64, dtype=dtype)
    x = I.make_prefill(cfg, 21)
    g = torch.Generator("cpu").manual_seed(22)
    dout = torch.randn(cfg.B, cfg.H, cfg.n, cfg.d, generator=g).to(dtype)
    q, k, v = (dev(x[n]).requires_grad_(True) for n in ("q", "k", "v"))
    out = K.linear_attention(q, k, v, "elu1", decay=dev(x["decay"]))
    out.backward(dev(dout))
    torch.cuda.synchronize()
    refs = oracle.backward(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(dout),
                           oracle.MAP_ELU1, None, f64(x["decay"]))
    for t, r in zip((q, k, v), refs):
        assert rel(t.grad, r) <= GTOL[dtype]
    ref_out = oracle.forward(f64(x["q"]), f64(x["k"]), f64(x["v"]),
                             oracle.MAP_ELU1, None, f64(x["decay"]))
    assert rel(out.detach(), ref_out) <= (1e-4 if dtype == torch.float32
                                          else 1e-2)


# A decay per position (la_forward_gated_train, la_backward_gated): the
# oracle's adjoint of the gated recurrence (oracle.backward_gated).  Gate
# ranges are log10 of the per-head rate that scales softplus(z) (the input
# recipe of the gated forward), from slow decay to about 3e-7 per step.
GATED_GRID = [
    # (name, B, H, n, d, map, gate)
    ("ragged_d64", 2, 2, 1000, 64, "elu1", (-3.0, -1.0)),
    ("d128", 1, 2, 700, 128, "elu1", (-2.0, -0.5)),
    ("identity_d32_n17", 1, 2, 17, 32, "identity", (-2.0, -0.5)),
    ("d16_fast", 2, 1, 333, 16, "elu1", (-1.0, 0.5)),
    ("identity_d128_long", 1, 1, 3000, 128, "identity", (-3.0, -1.0)),
    ("one_chunk", 1, 3, 40, 128, "elu1", (-2.0, -0.5)),
]


def run_gated(cfg, seed, lam=None):
    x = make(cfg, seed)
    if lam is not None:
        x["log_decay"] = lam
    name = I.MAP_NAMES[cfg.mapk]
    q, k, v, ld = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["log_decay"])
    out, den = K.forward_train(q, k, v, name, log_decay=ld)
    grads = K.backward(q, k, v, out, den, dev(x["dout"]), name, log_decay=ld)
    torch.cuda.synchronize()
    ref = oracle.backward_gated(f64(x["q"]), f64(x["k"]), f64(x["v"]),
                                f64(x["dout"]), cfg.mapk, None,
                                f64(x["log_decay"]), oracle.LD_POSITION)
    ref_out = oracle.forward_gated(f64(x["q"]), f64(x["k"]), f64(x["v"]),
                                   cfg.mapk, None, f64(x["log_decay"]),
                                   oracle.LD_POSITION, True)
    return out, grads, ref_out, ref


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("case", GATED_GRID, ids=[c[0] for c in GATED_GRID])
def test_backward_gated_grid(case, dtype):
    name, B, H, n, d, mp, gate = case
    mapk = I.MAP_ELU1 if mp == "elu1" else I.MAP_IDENTITY
    cfg = I.PrefillConfig(f"bwd_gated_{name}", B=B, H=H, n=n, d=d,
                          dtype=dtype, mapk=mapk, gate=gate)
    print(f"gated backward {name} {dtype}", flush=True)
    out, grads, ref_out, ref = run_gated(cfg, seed=9)
    errs = [rel(gq, r) for gq, r in zip(grads, ref)]
    print(f"  dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}", flush=True)
    assert max(errs) <= GTOL[dtype], errs
    assert rel(out, ref_out) <= TOL[dtype]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_backward_gated_resets(dtype, d):
    """lam = -inf (gamma = 0: the state restarts) at scattered positions,
    one of them a chunk's first row and one its last, and very negative
    values elsewhere among ordinary ones: the kernel floors lam at -104,
    where exp(lam) is 0 in fp32 as it is for -inf.  (bf16 at d = 128 runs
    the segmented roles, here one chunk per segment, so the resets also
    sit on segment edges.)"""
    cfg = I.PrefillConfig("bwd_gated_resets", B=1, H=2, n=300, d=d,
                          dtype=dtype, mapk=I.MAP_ELU1, gate=(-2.0, -0.5))
    lam = I.make_prefill(cfg, 11)["log_decay"].clone()
    lam[0, 0, [0, 64, 127, 200]] = -float("inf")
    lam[0, 1, [5, 130, 131]] = -500.0
    out, grads, ref_out, ref = run_gated(cfg, seed=11, lam=lam)
    errs = [rel(gq, r) for gq, r in zip(grads, ref)]
    print(f"resets {dtype}: dq {errs[0]:.2e} dk {errs[1]:.2e} "
          f"dv {errs[2]:.2e}", flush=True)
    assert max(errs) <= GTOL[dtype], errs
    assert rel(out, ref_out) <= TOL[dtype]


def test_backward_gated_full_size_every_unit():
    """The gated workload's sizes (B2 H16 n65536 d128, bf16, elu + 1, a
    decay per position), every unit and every gradient against the
    oracle's adjoint (one oracle call per batch row, its heads in
    parallel)."""
    cfg = I.PrefillConfig("bwd_gated_full", B=2, H=16, n=65536, d=128,
                          dtype=torch.bfloat16, mapk=I.MAP_ELU1,
                          gate=(-3.0, -1.0))
    x = make(cfg, 0)
    q, k, v, ld = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["log_decay"])
    out, den = K.forward_train(q, k, v, "elu1", log_decay=ld)
    grads = K.backward(q, k, v, out, den, dev(x["dout"]), "elu1",
                       log_decay=ld)
    torch.cuda.synchronize()
    grads = [t.cpu() for t in grads]
    worst = [0.0, 0.0, 0.0]
    for b in range(cfg.B):
        sl = slice(b, b + 1)
        ref = oracle.backward_gated(f64(x["q"][sl]), f64(x["k"][sl]),
                                    f64(x["v"][sl]), f64(x["dout"][sl]),
                                    cfg.mapk, None, f64(x["log_decay"][sl]),
                                    oracle.LD_POSITION)
        for i in range(3):
            got = grads[i][sl].double().numpy()
            assert np.all(np.isfinite(got))
            for h in range(cfg.H):
                r = ref[i][0, h]
                worst[i] = max(worst[i], np.max(np.abs(got[0, h] - r)) /
                               np.max(np.abs(r)))
        del ref
    print(f"gated backward full size: max per-unit rel err dq {worst[0]:.2e} "
          f"dk {worst[1]:.2e} dv {worst[2]:.2e}", flush=True)
    assert max(worst) <= GTOL[torch.bfloat16]


GATED_PF = [
    # (name, B, H, n, d, m, dtype): the Performer map with a decay per
    # position (features, column-block roles with the decay tables, the
    # map's chain rule)
    ("d64_m256_bf16", 1, 2, 300, 64, 256, torch.bfloat16),
    ("d32_m64_fp32", 2, 1, 200, 32, 64, torch.float32),
    ("d128_m128_bf16_one_chunk", 1, 2, 50, 128, 128, torch.bfloat16),
]


@pytest.mark.parametrize("case", GATED_PF, ids=[c[0] for c in GATED_PF])
def test_backward_gated_performer(case):
    name, B, H, n, d, m, dtype = case
    cfg = I.PERFORMER.replace(B=B, H=H, n=n, d=d, m=m, dtype=dtype,
                              gate=(-2.0, -0.5))
    x = make(cfg, 31)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    om, ld = dev(x["omega"]), dev(x["log_decay"])
    out, den = K.forward_train(q, k, v, "performer", omega=om, log_decay=ld)
    grads = K.backward(q, k, v, out, den, dev(x["dout"]), "performer",
                       omega=om, log_decay=ld)
    torch.cuda.synchronize()
    ref = oracle.backward_gated(f64(x["q"]), f64(x["k"]), f64(x["v"]),
                                f64(x["dout"]), I.MAP_PERFORMER,
                                f64(x["omega"]), f64(x["log_decay"]),
                                oracle.LD_POSITION)
    errs = [rel(gq, r) for gq, r in zip(grads, ref)]
    print(f"gated performer {name}: dq {errs[0]:.2e} dk {errs[1]:.2e} "
          f"dv {errs[2]:.2e}", flush=True)
    assert max(errs) <= GTOL[dtype], errs


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_autograd_op_gated_matches_oracle(dtype):
    """linear_attention(..., log_decay=...) as a torch op: autograd
    gradients through la_forward_gated_train and la_backward_gated."""
    cfg = I.PrefillConfig("bwd_gated_op", B=1, H=2, n=333, d=64, dtype=dtype,
                          mapk=I.MAP_ELU1, gate=(-2.0, -0.5))
    x = make(cfg, 23)
    q, k, v = (dev(x[n]).requires_grad_(True) for n in ("q", "k", "v"))
    out = K.linear_attention(q, k, v, "elu1", log_decay=dev(x["log_decay"]))
    out.backward(dev(x["dout"]))
    torch.cuda.synchronize()
    refs = oracle.backward_gated(f64(x["q"]), f64(x["k"]), f64(x["v"]),
                                 f64(x["dout"]), oracle.MAP_ELU1, None,
                                 f64(x["log_decay"]), oracle.LD_POSITION)
    for t, r in zip((q, k, v), refs):
        assert rel(t.grad, r) <= GTOL[dtype]


def test_backward_random_shapes():
    """Seeded random configurations of the whole backward, run in one
    sequence on the binding's shared workspace: map (elu + 1, identity,
    Performer), d and d' within the built sizes, ragged n, B and H, no
    decay, a decay per head or a decay per position, and the storage type;
    every unit's gradients against the oracle's adjoint."""
    rng = np.random.default_rng(20261203)
    worst = {torch.bfloat16: 0.0, torch.float32: 0.0}
    for i in range(24):
        dtype = [torch.bfloat16, torch.float32][int(rng.integers(2))]
        mp = ["elu1", "identity", "performer"][int(rng.integers(3))]
        if mp == "performer":
            d = int(rng.choice([32, 64, 128]))
            m = int(rng.choice([m for m in (32, 64, 128, 256)
                                if d * m <= 16384]))
        else:
            d = int(rng.choice([16, 32, 64, 128]))
            m = d
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        n = int(rng.integers(1, 700))
        kind = ["none", "head", "position"][int(rng.integers(3))]
        mapk = {"elu1": I.MAP_ELU1, "identity": I.MAP_IDENTITY,
                "performer": I.MAP_PERFORMER}[mp]
        base = I.PERFORMER if mp == "performer" else I.ELU1_CAUSAL
        cfg = base.replace(B=B, H=H, n=n, d=d, m=m, dtype=dtype, mapk=mapk,
                           decay=(-2.0, -0.5) if kind == "head" else None,
                           gate=(-2.0, -0.5) if kind == "position" else None)
        print(f"case {i}: {mp} d={d} m={m} B={B} H={H} n={n} {kind} "
              f"{dtype}", flush=True)
        x = make(cfg, 100 + i)
        q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
        om, dec, ld = dev(x["omega"]), dev(x["decay"]), dev(x["log_decay"])
        out, den = K.forward_train(q, k, v, mp, decay=dec, omega=om,
                                   log_decay=ld)
        grads = K.backward(q, k, v, out, den, dev(x["dout"]), mp, decay=dec,
                           omega=om, log_decay=ld)
        torch.cuda.synchronize()
        if kind == "position":
            ref = oracle.backward_gated(f64(x["q"]), f64(x["k"]), f64(x["v"]),
                                        f64(x["dout"]), mapk, f64(x["omega"]),
                                        f64(x["log_decay"]),
                                        oracle.LD_POSITION)
        else:
            ref = oracle.backward(f64(x["q"]), f64(x["k"]), f64(x["v"]),
                                  f64(x["dout"]), mapk, f64(x["omega"]),
                                  f64(x["decay"]))
        if n == 1:   # dq = dk = 0 exactly: compare dv only (see above)
            errs = [rel(grads[2], ref[2])]
        else:
            errs = [rel(gq, r) for gq, r in zip(grads, ref)]
        worst[dtype] = max(worst[dtype], max(errs))
        assert max(errs) <= GTOL[dtype], (i, errs)
    print(f"random shapes: worst bf16 {worst[torch.bfloat16]:.2e}, "
          f"fp32 {worst[torch.float32]:.2e}", flush=True)
