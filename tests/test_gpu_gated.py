"""GPU parity of the gated recurrence (input-dependent, per-position decay
in the chunked forward; per-row, per-unit and per-both decay in the decode
step) against the fp64 oracle's gated recurrence, through the C ABI.

Tolerance (max |gpu - oracle| / max |oracle|): 1e-4 for fp32 storage, 1e-2
for bf16 storage, as for every parity test.
"""
import numpy as np
import pytest
import torch

import kernelized_attention_scan_amd as K
from kernelized_attention_scan_amd import inputs as I
import oracle

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2}
SYNC_BYTES = 4 * (64 + 512 * 32)


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


def gated_inputs(cfg, seed):
    x = I.make_prefill(cfg, seed)
    if cfg.mapk == I.MAP_IDENTITY:           # positive features of width m
        g = torch.Generator().manual_seed(seed + 1000)
        sh = (cfg.B, cfg.H, cfg.n, cfg.m)
        x["q"] = (torch.rand(sh, generator=g) + 0.05).to(cfg.dtype)
        x["k"] = (torch.rand(sh, generator=g) + 0.05).to(cfg.dtype)
    return x


def run_gated(cfg, seed=0, causal=None):
    causal = cfg.causal if causal is None else causal
    x = gated_inputs(cfg, seed)
    name = I.MAP_NAMES[cfg.mapk]
    out = K.forward_gated(dev(x["q"]), dev(x["k"]), dev(x["v"]),
                          dev(x["log_decay"]), "position", name,
                          omega=dev(x["omega"]), causal=causal)
    torch.cuda.synchronize()
    ref = oracle.forward_gated(f64(x["q"]), f64(x["k"]), f64(x["v"]),
                               cfg.mapk, f64(x["omega"]), f64(x["log_decay"]),
                               oracle.LD_POSITION, causal)
    return rel(out, ref)


GATE = (-3.0, -1.0)
GRID = [
    # (name, B, H, n, d, map, m, causal, gate)
    ("elu1_ragged_segmented", 2, 3, 1000, 64, "elu1", 0, True, GATE),
    ("elu1_d128", 1, 2, 1500, 128, "elu1", 0, True, GATE),
    ("elu1_d32_one_partial_chunk", 1, 2, 17, 32, "elu1", 0, True, GATE),
    ("elu1_d16", 2, 2, 333, 16, "elu1", 0, True, GATE),
    ("elu1_one_unit_many_segments", 1, 1, 4099, 64, "elu1", 0, True, GATE),
    ("elu1_strong_decay", 1, 3, 900, 64, "elu1", 0, True, (-1.0, 0.7)),
    ("noncausal_elu1", 2, 2, 700, 64, "elu1", 0, False, GATE),
    ("noncausal_one_segment", 8, 64, 40, 32, "elu1", 0, False, GATE),
    ("identity_df128_d64", 1, 2, 600, 64, "identity", 128, True, GATE),
    ("performer_m256", 1, 2, 900, 64, "performer", 256, True, GATE),
    ("performer_d32_m64", 1, 2, 400, 32, "performer", 64, True, GATE),
    ("identity_df256_d128", 1, 2, 500, 128, "identity", 256, True, GATE),
    ("identity_df256_d128_noncausal", 1, 1, 300, 128, "identity", 256, False,
     GATE),
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("case", GRID, ids=[c[0] for c in GRID])
def test_forward_gated_grid(case, dtype):
    name, B, H, n, d, mp, m, causal, gate = case
    mapk = {"identity": I.MAP_IDENTITY, "elu1": I.MAP_ELU1,
            "performer": I.MAP_PERFORMER}[mp]
    cfg = I.PrefillConfig(f"gated_{name}", B=B, H=H, n=n, d=d, dtype=dtype,
                          mapk=mapk, m=m, causal=causal, gate=gate,
                          qk_std=0.5 if mp == "performer" else 1.0)
    try:
        err = run_gated(cfg, seed=3)
    except K.LinAttnError as e:
        if e.status == K._binding.LA_ERR_UNSUPPORTED:
            pytest.skip(f"not built: {e}")
        raise
    assert err <= TOL[dtype]


def test_forward_gated_full_size_every_unit():
    """B=2 H=16 n=65536 d=128, per-position decay, every unit."""
    cfg = I.GATED
    x = I.make_prefill(cfg, 0)
    out = K.forward_gated(dev(x["q"]), dev(x["k"]), dev(x["v"]),
                          dev(x["log_decay"]))
    torch.cuda.synchronize()
    out = out.cpu()
    worst = 0.0
    for b in range(cfg.B):
        sl = slice(b, b + 1)
        ref = oracle.forward_gated(f64(x["q"][sl]), f64(x["k"][sl]),
                                   f64(x["v"][sl]), cfg.mapk, None,
                                   f64(x["log_decay"][sl]),
                                   oracle.LD_POSITION, True)
        got = out[sl].double().numpy()
        assert np.all(np.isfinite(got))
        for h in range(cfg.H):
            r = ref[0, h]
            worst = max(worst, np.max(np.abs(got[0, h] - r)) / np.max(np.abs(r)))
    print(f"gated full size: max per-unit rel err {worst:.3e}", flush=True)
    assert worst <= 1e-2


@pytest.mark.parametrize("causal", [True, False])
def test_gated_constant_decay_matches_decayed_forward(causal):
    """A per-position log decay equal to log(a) at every position is the
    per-head decayed forward (eqs 10-11)."""
    cfg = I.ELU1_CAUSAL.replace(B=2, H=4, n=2500, decay=(-3.0, -1.0))
    x = I.make_prefill(cfg, 5)
    dec = x["decay"]
    lam = torch.log(dec)[None, :, None].expand(2, 4, 2500).contiguous()
    a = K.forward(dev(x["q"]), dev(x["k"]), dev(x["v"]), decay=dev(dec),
                  causal=causal)
    b = K.forward_gated(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(lam),
                        causal=causal)
    torch.cuda.synchronize()
    assert rel(b, f64(a)) <= 1e-2


def test_gated_full_reset_returns_v():
    """log decay -inf everywhere: gamma = 0, each position sees only
    itself, out = v (bf16 storage: to rounding of the final division)."""
    cfg = I.ELU1_CAUSAL.replace(B=1, H=2, n=700)
    x = I.make_prefill(cfg, 8)
    lam = torch.full((1, 2, 700), -float("inf"))
    out = K.forward_gated(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(lam))
    torch.cuda.synchronize()
    assert rel(out, f64(x["v"])) <= 1e-2


def test_gated_exchange_deterministic_and_area_zero():
    cfg = I.ELU1_CAUSAL.replace(B=1, H=2, n=4096, gate=GATE)
    x = I.make_prefill(cfg, 31)
    need = K.forward_workspace_bytes(cfg.B, cfg.H, cfg.n, cfg.d, cfg.d_feat)
    assert need > SYNC_BYTES
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    args = [dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["log_decay"])]
    first = K.forward_gated(*args, workspace=ws)
    for _ in range(20):
        assert torch.equal(first, K.forward_gated(*args, workspace=ws))
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws[:SYNC_BYTES]).item() == 0
    K.workspace_check(ws)


def test_gated_state_handoff_then_gated_decode():
    """Prefill the first n0 positions with the state handed out, then decode
    the rest token by token with this position's decay: the outputs equal
    one gated forward over all n; the handed-out state matches the oracle's
    decode chain."""
    n, n0, B, H, d = 600, 536, 2, 2, 32
    cfg = I.ELU1_CAUSAL.replace(B=B, H=H, n=n, d=d, dtype=torch.float32,
                                gate=GATE)
    x = I.make_prefill(cfg, 41)
    q, k, v, lam = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["log_decay"])
    full = K.forward_gated(q, k, v, lam)
    mu = torch.empty(B, H, d, d, device="cuda")
    nu = torch.empty(B, H, d, device="cuda")
    K.forward_gated(q[:, :, :n0].contiguous(), k[:, :, :n0].contiguous(),
                    v[:, :, :n0].contiguous(), lam[:, :, :n0].contiguous(),
                    mu_out=mu, nu_out=nu)
    torch.cuda.synchronize()
    # the handed-out state against the oracle's gated decode chain
    rmu, rnu = np.zeros((B, H, d, d)), np.zeros((B, H, d))
    qn, kn, vn, ln = f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["log_decay"])
    for j in range(n0):
        _, rmu, rnu = oracle.decode_gated(rmu, rnu, qn[:, :, j], kn[:, :, j],
                                          vn[:, :, j], oracle.MAP_ELU1, None,
                                          ln[:, :, j], oracle.LD_POSITION)
    assert rel(mu, rmu) <= 1e-4 and rel(nu, rnu) <= 1e-4
    outs = [K.decode_step_gated(mu, nu, q[:, :, j].contiguous(),
                                k[:, :, j].contiguous(),
                                v[:, :, j].contiguous(),
                                lam[:, :, j].contiguous(), "position")
            for j in range(n0, n)]
    torch.cuda.synchronize()
    chain = torch.stack(outs, dim=2)
    assert rel(chain, f64(full[:, :, n0:])) <= 1e-4


@pytest.mark.parametrize("layout", ["channel", "position", "both"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("mapk", [I.MAP_ELU1, I.MAP_PERFORMER])
def test_decode_gated(layout, dtype, mapk):
    cfg = I.DECODE.replace(S=6, H=4, d=64, dtype=dtype, mapk=mapk,
                           m=128 if mapk == I.MAP_PERFORMER else 0)
    x = I.make_decode(cfg, 9)
    df = cfg.d_feat
    g = torch.Generator().manual_seed(19)
    shape = {"channel": (cfg.H, df), "position": (cfg.S, cfg.H),
             "both": (cfg.S, cfg.H, df)}[layout]
    lam = -torch.pow(10.0, torch.empty(shape).uniform_(-3, 0, generator=g))
    mu, nu = dev(x["mu"]), dev(x["nu"])
    out = K.decode_step_gated(mu, nu, dev(x["q"]), dev(x["k"]), dev(x["v"]),
                              dev(lam), layout, I.MAP_NAMES[mapk],
                              omega=dev(x["omega"]))
    torch.cuda.synchronize()
    mode = {"channel": oracle.LD_CHANNEL, "position": oracle.LD_POSITION,
            "both": oracle.LD_BOTH}[layout]
    ro, rmu, rnu = oracle.decode_gated(f64(x["mu"]), f64(x["nu"]),
                                       f64(x["q"]), f64(x["k"]), f64(x["v"]),
                                       mapk, f64(x["omega"]), f64(lam), mode)
    assert rel(out, ro) <= TOL[dtype]
    assert rel(mu, rmu) <= 1e-4 and rel(nu, rnu) <= 1e-4
