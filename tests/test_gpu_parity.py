"""GPU parity: the HIP library (called through its C ABI) against the fp64
oracle on the very same seeded, storage-rounded inputs.

Tolerance (max |gpu - oracle| / max |oracle|): 1e-4 where the compared tensor
is stored in fp32, 1e-2 where it is stored in bf16.
"""
import math

import numpy as np
import pytest
import torch

import kernelized_attention_scan_amd as K
from kernelized_attention_scan_amd import inputs as I
import oracle

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2}
MAPK = {"identity": I.MAP_IDENTITY, "elu1": I.MAP_ELU1,
        "performer": I.MAP_PERFORMER}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    K.load_library()
    torch.cuda.set_device(0)
    yield


def rel(gpu_out, ref):
    g = gpu_out.detach().float().cpu().double().numpy()
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    return float(np.max(np.abs(g - r)) / max(np.max(np.abs(r)), 1e-300))


def f64(t):
    return None if t is None else t.detach().cpu().double().numpy()


def dev(t):
    return None if t is None else t.cuda()


def run_forward(cfg: I.PrefillConfig, seed=0, units=None):
    """GPU forward on the whole config; oracle on `units` (list of (b, h))
    or on everything.  Returns the relative error."""
    x = I.make_prefill(cfg, seed)
    name = I.MAP_NAMES[cfg.mapk]
    out = K.forward(dev(x["q"]), dev(x["k"]), dev(x["v"]), feature_map=name,
                    omega=dev(x["omega"]), decay=dev(x["decay"]),
                    causal=cfg.causal)
    torch.cuda.synchronize()
    q, k, v = x["q"], x["k"], x["v"]
    if units is None:
        ref = oracle.forward(f64(q), f64(k), f64(v), cfg.mapk, f64(x["omega"]),
                             f64(x["decay"]), cfg.causal)
        return rel(out, ref)
    errs = []
    for b, h in units:
        dec = None if x["decay"] is None else f64(x["decay"][h:h + 1])
        ref = oracle.forward(f64(q[b:b + 1, h:h + 1]), f64(k[b:b + 1, h:h + 1]),
                             f64(v[b:b + 1, h:h + 1]), cfg.mapk,
                             f64(x["omega"]), dec, cfg.causal)
        errs.append(rel(out[b:b + 1, h:h + 1], ref))
    return max(errs)


# --------------------------------------------------------------------------
# Feature maps
# --------------------------------------------------------------------------

@pytest.mark.parametrize("in_dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("out_dt", [torch.float32, torch.bfloat16])
def test_featmap_elu1(in_dt, out_dt):
    g = torch.Generator().manual_seed(1)
    x = (torch.randn(777, 64, generator=g) * 3).to(in_dt)
    y = K.featmap(x.cuda(), "elu1", out_dtype=out_dt)
    ref = oracle.featmap(f64(x), oracle.MAP_ELU1)
    assert rel(y, ref) <= TOL[out_dt]


@pytest.mark.parametrize("d,m", [(16, 16), (64, 256), (128, 64), (32, 48)])
@pytest.mark.parametrize("in_dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("out_dt", [torch.float32, torch.bfloat16])
def test_featmap_performer(d, m, in_dt, out_dt):
    g = torch.Generator().manual_seed(2)
    x = (torch.randn(333, d, generator=g) * 0.5).to(in_dt)
    om = torch.randn(d, m, generator=g) / math.sqrt(d)
    y = K.featmap(x.cuda(), "performer", omega=om.cuda(), out_dtype=out_dt)
    ref = oracle.featmap(f64(x), oracle.MAP_PERFORMER, f64(om))
    assert rel(y, ref) <= TOL[out_dt]


# --------------------------------------------------------------------------
# Forward: the tiny workload exactly, then a grid of reduced shapes
# --------------------------------------------------------------------------

def test_forward_tiny_fp32_workload():
    """B=1, H=1, n=256, d=d'=16, fp32, elu+1, causal, no decay, seed 0."""
    assert run_forward(I.TINY_FP32) <= 1e-4


GRID = [
    # (name, B, H, n, d, map, m, decay, causal)
    ("elu1_ragged", 2, 3, 1000, 64, "elu1", 0, False, True),
    ("elu1_n1", 1, 2, 1, 64, "elu1", 0, False, True),
    ("elu1_n17", 1, 1, 17, 32, "elu1", 0, True, True),
    ("elu1_one_unit_many_segments", 1, 1, 4099, 64, "elu1", 0, False, True),
    ("elu1_d128_decay", 1, 2, 1500, 128, "elu1", 0, True, True),
    ("elu1_d16", 2, 2, 333, 16, "elu1", 0, True, True),
    ("noncausal_elu1", 2, 2, 700, 64, "elu1", 0, False, False),
    ("noncausal_decay", 1, 3, 300, 32, "elu1", 0, True, False),
    ("identity_df128_d64", 1, 2, 600, 64, "identity", 128, False, True),
    ("identity_df16_d128", 1, 1, 300, 128, "identity", 16, True, True),
    # layouts chosen by LDS: two tile sets with one S^T copy (d = 128,
    # d' = 128 bf16; d = 64, d' = 128 fp32) and register-weighted keys
    ("elu1_d128_nodecay", 1, 2, 1500, 128, "elu1", 0, False, True),
    ("elu1_d128_noncausal_decay", 1, 2, 700, 128, "elu1", 0, True, False),
    ("identity_df128_d64_decay", 1, 2, 600, 64, "identity", 128, True, True),
    ("identity_df64_d128_decay", 1, 2, 500, 128, "identity", 64, True, True),
    ("identity_df256_d128", 1, 1, 200, 128, "identity", 256, False, True),
    # fp32 storage: value columns split in halves (d = 128, d' = 256), and
    # the decay weights of the state update taken in registers (d' = 256)
    ("identity_df256_d128_decay_segmented", 1, 2, 700, 128, "identity", 256,
     True, True),
    ("identity_df256_d128_noncausal", 1, 2, 300, 128, "identity", 256, True,
     False),
    ("identity_df256_d64_decay", 2, 2, 650, 64, "identity", 256, True, True),
    ("performer_d128_m256_decay", 1, 1, 400, 128, "performer", 256, True,
     True),
    ("performer_m256", 1, 2, 900, 64, "performer", 256, False, True),
    ("performer_m64_decay", 1, 2, 400, 32, "performer", 64, True, True),
    ("performer_noncausal", 1, 1, 300, 64, "performer", 128, False, False),
    ("performer_d128_m128", 1, 2, 500, 128, "performer", 128, False, True),
    ("performer_d32_m256_decay", 1, 1, 333, 32, "performer", 256, True, True),
]


def grid_cfg(case, dtype):
    name, B, H, n, d, mp, m, decay, causal = case
    mapk = MAPK[mp]
    cfg = I.PrefillConfig(f"{name}_{dtype}", B=B, H=H, n=n, d=d, dtype=dtype,
                          mapk=mapk, m=m, decay=(-2.0, -0.5) if decay else None,
                          causal=causal, qk_std=0.5 if mp == "performer" else 1.0)
    return cfg


def _identity_inputs(cfg, seed):
    """Identity map: positive pre-featured q, k of width m."""
    g = torch.Generator().manual_seed(seed)
    sh = (cfg.B, cfg.H, cfg.n, cfg.m)
    q = (torch.rand(sh, generator=g) + 0.05).to(cfg.dtype)
    k = (torch.rand(sh, generator=g) + 0.05).to(cfg.dtype)
    v = torch.randn((cfg.B, cfg.H, cfg.n, cfg.d), generator=g).to(cfg.dtype)
    dec = None
    if cfg.decay is not None:
        dec = (1 - 10 ** torch.empty(cfg.H).uniform_(-2, -0.5, generator=g)
               ).float()
    return q, k, v, dec


def _supported_or_skip(fn):
    """Run fn(); a combination the library reports as not built (LDS limit)
    is skipped with the library's reason, any other error fails."""
    try:
        return fn()
    except K.LinAttnError as e:
        if e.status == K._binding.LA_ERR_UNSUPPORTED:
            pytest.skip(f"not built: {e}")
        raise


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("case", GRID, ids=[c[0] for c in GRID])
def test_forward_grid(case, dtype):
    cfg = grid_cfg(case, dtype)
    if cfg.mapk == I.MAP_IDENTITY:
        q, k, v, dec = _identity_inputs(cfg, 5)
        out = _supported_or_skip(lambda: K.forward(
            q.cuda(), k.cuda(), v.cuda(), "identity", decay=dev(dec),
            causal=cfg.causal))
        torch.cuda.synchronize()
        ref = oracle.forward(f64(q), f64(k), f64(v), oracle.MAP_IDENTITY,
                             None, f64(dec), cfg.causal)
        assert rel(out, ref) <= TOL[dtype]
        return
    assert _supported_or_skip(lambda: run_forward(cfg, seed=3)) <= TOL[dtype]


def test_forward_empty_inputs_are_noops():
    z = torch.empty(0, 2, 16, 64, dtype=torch.bfloat16, device="cuda")
    assert K.forward(z, z, z).shape == z.shape
    z = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    assert K.forward(z, z, z).shape == z.shape


# --------------------------------------------------------------------------
# Forward at the full workload sizes, in the benchmark's launch configuration,
# against the oracle on every (batch, head) unit.
# --------------------------------------------------------------------------

def full_size_errors(cfg, seed=0):
    """GPU forward on the whole config; the oracle on every unit, one batch
    index at a time (its OpenMP loop runs over that batch's heads).  Returns
    the per-unit relative errors, [B][H]."""
    x = I.make_prefill(cfg, seed)
    name = I.MAP_NAMES[cfg.mapk]
    out = K.forward(dev(x["q"]), dev(x["k"]), dev(x["v"]), feature_map=name,
                    omega=dev(x["omega"]), decay=dev(x["decay"]),
                    causal=cfg.causal)
    torch.cuda.synchronize()
    out = out.cpu()
    errs = np.zeros((cfg.B, cfg.H))
    for b in range(cfg.B):
        sl = slice(b, b + 1)
        ref = oracle.forward(f64(x["q"][sl]), f64(x["k"][sl]),
                             f64(x["v"][sl]), cfg.mapk, f64(x["omega"]),
                             f64(x["decay"]), cfg.causal)
        got = out[sl].double().numpy()
        assert np.all(np.isfinite(got)), f"non-finite output, batch {b}"
        for h in range(cfg.H):
            r = ref[0, h]
            errs[b, h] = np.max(np.abs(got[0, h] - r)) / np.max(np.abs(r))
        del ref, got
    return errs


@pytest.mark.parametrize("cfg", [I.ELU1_CAUSAL, I.PERFORMER, I.DECAYED],
                         ids=lambda c: c.name)
def test_forward_full_size_every_unit(cfg):
    """Every one of the B*H units at the full workload size, element by
    element: the block-to-unit mapping, the per-unit synchronisation lines
    and the per-head decay all depend on the unit."""
    errs = full_size_errors(cfg, seed=0)
    worst = np.unravel_index(np.argmax(errs), errs.shape)
    print(f"{cfg.name}: max per-unit rel err {errs.max():.3e} at "
          f"(b, h) = {worst}", flush=True)
    assert errs.max() <= 1e-2


# --------------------------------------------------------------------------
# Properties
# --------------------------------------------------------------------------

def test_forward_is_deterministic():
    x = I.make_prefill(I.ELU1_CAUSAL.replace(B=2, n=2048), 4)
    args = [x["q"].cuda(), x["k"].cuda(), x["v"].cuda()]
    a = K.forward(*args)
    b = K.forward(*args)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_segmentation_invariance():
    """The same unit alone (one segment per chunk) and inside a big batch
    (fewer, longer segments) agrees to rounding."""
    cfg = I.ELU1_CAUSAL.replace(B=8, H=8, n=2048, decay=(-3.0, -1.0))
    x = I.make_prefill(cfg, 6)
    dec = x["decay"].cuda()
    big = K.forward(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), decay=dec)
    one = K.forward(x["q"][:1, :1].cuda().contiguous(),
                    x["k"][:1, :1].cuda().contiguous(),
                    x["v"][:1, :1].cuda().contiguous(), decay=dec[:1])
    torch.cuda.synchronize()
    a, b = big[:1, :1].float(), one.float()
    assert (a - b).abs().max().item() <= 1e-2 * b.abs().max().item()


def test_workspace_shared_across_shapes():
    """One workspace serves segmented calls of different shapes in turn: the
    scratch one shape leaves behind never reads as another shape's flags."""
    shapes = [(1, 2, 2048), (4, 8, 1024), (1, 1, 4096), (2, 4, 700)]
    cfgs = [I.ELU1_CAUSAL.replace(B=b, H=h, n=n) for b, h, n in shapes]
    need = max(K.forward_workspace_bytes(c.B, c.H, c.n, c.d, c.d_feat)
               for c in cfgs)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for i, cfg in enumerate(cfgs):
            x = I.make_prefill(cfg, 20 + i)
            out = K.forward(dev(x["q"]), dev(x["k"]), dev(x["v"]),
                            workspace=ws)
            torch.cuda.synchronize()
            ref = oracle.forward(f64(x["q"]), f64(x["k"]), f64(x["v"]),
                                 cfg.mapk, None, None, True)
            assert rel(out, ref) <= TOL[torch.bfloat16], (rep, cfg)


# Bytes of the synchronisation area at the start of a segmented forward's
# workspace: 64 header words, then one 32-word line per unit for up to 512.
SYNC_BYTES = 4 * (64 + 512 * 32)
TIMEOUT_WORD = 8


@pytest.mark.parametrize("cfg", [
    I.ELU1_CAUSAL,
    I.ELU1_CAUSAL.replace(causal=False),
    I.ELU1_CAUSAL.replace(B=1, H=2, n=4096, decay=(-3.0, -1.0)),
    I.PERFORMER.replace(n=2048),
    # 5 segments in a grid of 5: the segments run on different XCDs, so the
    # aggregates go through the coherence point
    I.ELU1_CAUSAL.replace(B=1, H=1, n=300),
    I.ELU1_CAUSAL.replace(B=1, H=1, n=300, causal=False),
], ids=["elu1", "noncausal", "decayed", "performer", "cross_xcd",
        "cross_xcd_noncausal"])
def test_exchange_never_times_out_and_leaves_area_zero(cfg):
    """Segmented calls: every wait for another segment's aggregate ends
    because the flag was seen (the timeout word stays 0), the last
    workgroup of each unit clears its line (the whole area reads 0), and
    every repeat gives bitwise the same output (the exchange and the
    overlapped staging around it leave no race)."""
    name = I.MAP_NAMES[cfg.mapk]
    need = K.forward_workspace_bytes(cfg.B, cfg.H, cfg.n, cfg.d, cfg.d_feat,
                                     name, cfg.dtype, cfg.causal)
    assert need > SYNC_BYTES, "the case must be split into segments"
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    x = I.make_prefill(cfg, 31)
    args = [dev(x["q"]), dev(x["k"]), dev(x["v"]), name]
    kw = dict(omega=dev(x["omega"]), decay=dev(x["decay"]),
              causal=cfg.causal, workspace=ws)
    first = K.forward(*args, **kw)
    for _ in range(40):
        again = K.forward(*args, **kw)
        assert torch.equal(first, again)
    torch.cuda.synchronize()
    sync = ws[:SYNC_BYTES].view(torch.int32).cpu()
    assert sync[TIMEOUT_WORD].item() == 0, "a wait gave up"
    assert torch.count_nonzero(sync).item() == 0
    K.workspace_check(ws)             # the library reports no failure either


def test_exchange_give_up_is_reported_and_poisons_outputs():
    """A wait that gives up is reported by la_workspace_check and turns the
    outputs that depend on the missing partial sums into NaN.  The host
    forces it with a spin limit of one poll: the last causal segment skips
    phase 1 and waits at once for fifteen segments that each still have 64
    chunks of phase 1 to go.  Every kernel still ends normally, the
    synchronisation area is zero again afterwards, and with the default
    limit restored the same call matches the oracle."""
    cfg = I.ELU1_CAUSAL.replace(B=1, H=1, n=65536)
    need = K.forward_workspace_bytes(cfg.B, cfg.H, cfg.n, cfg.d, cfg.d_feat)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    x = I.make_prefill(cfg, 5)
    args = [dev(x["q"]), dev(x["k"]), dev(x["v"])]
    seg_len = 4096                  # 16 segments of 64 chunks
    try:
        K.set_exchange_spin_limit(1)
        out = K.forward(*args, workspace=ws)
        torch.cuda.synchronize()
    finally:
        K.set_exchange_spin_limit(0)
    with pytest.raises(K.LinAttnError) as err:
        K.workspace_check(ws)
    assert err.value.status == K._binding.LA_ERR_EXCHANGE
    assert "gave up" in str(err.value)
    assert torch.isnan(out[0, 0, cfg.n - seg_len:].float()).all()
    assert torch.count_nonzero(ws[:SYNC_BYTES]).item() == 0
    K.workspace_check(ws)           # the status was cleared by the check
    out = K.forward(*args, workspace=ws)
    torch.cuda.synchronize()
    K.workspace_check(ws)
    ref = oracle.forward(f64(x["q"]), f64(x["k"]), f64(x["v"]), cfg.mapk,
                         None, None, True)
    assert rel(out, ref) <= TOL[torch.bfloat16]


def test_shared_workspace_after_unfused_performer():
    """One workspace serves calls of different sizes: an unfused Performer
    call without segments (fp32 storage) writes its q', k' features into the
    workspace, and a segmented call after it must still find the
    synchronisation area zero."""
    pf = I.PrefillConfig("pf_f32", B=1, H=2, n=17, d=32, dtype=torch.float32,
                         mapk=I.MAP_PERFORMER, m=128, decay=(-3.0, -1.0),
                         qk_std=0.5)
    seg = I.PrefillConfig("seg_bf16", B=2, H=2, n=65, d=32)
    need = max(K.forward_workspace_bytes(c.B, c.H, c.n, c.d, c.d_feat,
                                         I.MAP_NAMES[c.mapk], c.dtype, c.causal)
               for c in (pf, seg))
    assert need > SYNC_BYTES
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    x = I.make_prefill(pf, 11)
    K.forward(dev(x["q"]), dev(x["k"]), dev(x["v"]), "performer",
              omega=dev(x["omega"]), decay=dev(x["decay"]), workspace=ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws[:SYNC_BYTES]).item() == 0
    y = I.make_prefill(seg, 12)
    out = K.forward(dev(y["q"]), dev(y["k"]), dev(y["v"]), "elu1",
                    workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.forward(f64(y["q"]), f64(y["k"]), f64(y["v"]), oracle.MAP_ELU1,
                         None, None, True)
    assert rel(out, ref) <= TOL[torch.bfloat16]


def test_padded_features_many_segments():
    """d' = 16 features (padded to 32 columns in LDS) over many segmented
    units: the padding columns of every tile set must stay zero for the
    whole kernel (scratch written there once turned outputs into NaN)."""
    cfg = I.PrefillConfig("pad16", B=16, H=2, n=5000, d=128, m=16,
                          mapk=I.MAP_IDENTITY)
    q, k, v, dec = _identity_inputs(cfg, 4)
    out = K.forward(q.cuda(), k.cuda(), v.cuda(), "identity", causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    for b, h in [(0, 0), (cfg.B - 1, cfg.H - 1)]:
        ref = oracle.forward(f64(q[b:b + 1, h:h + 1]), f64(k[b:b + 1, h:h + 1]),
                             f64(v[b:b + 1, h:h + 1]), oracle.MAP_IDENTITY,
                             None, None, True)
        assert rel(out[b:b + 1, h:h + 1], ref) <= TOL[torch.bfloat16]


def test_random_shapes_share_one_workspace():
    """32 random shapes (maps, d, d', n with ragged tails, B, H, decay,
    causal, storage type; seed fixed) in one sequence, all through the
    binding's cached workspace, so each call also runs after calls of other
    sizes on the same memory.  Sampled units against the oracle."""
    import random
    rng = random.Random(777)
    fails = []
    for it in range(32):
        mapk = rng.choice([I.MAP_ELU1, I.MAP_ELU1, I.MAP_PERFORMER,
                           I.MAP_IDENTITY])
        d = (rng.choice([16, 32, 64, 64, 128]) if mapk != I.MAP_PERFORMER
             else rng.choice([32, 64]))
        m = (rng.choice([32, 64, 128, 256]) if mapk == I.MAP_PERFORMER else
             rng.choice([16, 32, 64, 128, 256]) if mapk == I.MAP_IDENTITY
             else 0)
        dtype = rng.choice([torch.bfloat16, torch.bfloat16, torch.float32])
        B, H = rng.choice([1, 2, 3, 4, 16]), rng.choice([1, 2, 5, 8, 16])
        n = rng.choice([1, 17, 63, 64, 65, 500, 1000, 2049, 4096, 5000])
        decay = rng.choice([None, (-3.0, -1.0)])
        causal = rng.random() < 0.8
        cfg = I.PrefillConfig(f"rand{it}", B=B, H=H, n=n, d=d, dtype=dtype,
                              mapk=mapk, m=m, decay=decay, causal=causal,
                              qk_std=0.5 if mapk == I.MAP_PERFORMER else 1.0)
        units = [(0, 0), (B - 1, H - 1)]
        try:
            if mapk == I.MAP_IDENTITY:
                q, k, v, dec = _identity_inputs(cfg, it)
                out = K.forward(q.cuda(), k.cuda(), v.cuda(), "identity",
                                decay=dev(dec), causal=causal)
                torch.cuda.synchronize()
                err = 0.0
                for b, h in units:
                    dd = None if dec is None else f64(dec[h:h + 1])
                    ref = oracle.forward(
                        f64(q[b:b + 1, h:h + 1]), f64(k[b:b + 1, h:h + 1]),
                        f64(v[b:b + 1, h:h + 1]), oracle.MAP_IDENTITY, None,
                        dd, causal)
                    err = max(err, rel(out[b:b + 1, h:h + 1], ref))
            else:
                err = run_forward(cfg, seed=it, units=units)
        except K.LinAttnError as e:
            if e.status == K._binding.LA_ERR_UNSUPPORTED:
                continue  # a combination not built (LDS limit)
            raise
        except AssertionError as e:
            fails.append((cfg, str(e)))
            continue
        if err > TOL[dtype]:
            fails.append((cfg, err))
    assert not fails, fails


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_constant_v_gives_constant_output(dtype):
    cfg = I.ELU1_CAUSAL.replace(B=1, H=4, n=3000, dtype=dtype,
                                decay=(-3.0, -1.0))
    x = I.make_prefill(cfg, 7)
    c = torch.linspace(-2, 2, 64).to(dtype)
    v = c.expand(1, 4, 3000, 64).contiguous()
    out = K.forward(x["q"].cuda(), x["k"].cuda(), v.cuda(),
                    decay=x["decay"].cuda())
    torch.cuda.synchronize()
    err = (out.float().cpu() - c.float()).abs().max().item()
    assert err <= TOL[dtype] * 2.0


def test_decay_zero_returns_v_exactly():
    """a = 0: each position attends only to itself, out = v bit for bit."""
    cfg = I.ELU1_CAUSAL.replace(B=1, H=2, n=700)
    x = I.make_prefill(cfg, 8)
    out = K.forward(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(),
                    decay=torch.zeros(2, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), x["v"])


# --------------------------------------------------------------------------
# Decode
# --------------------------------------------------------------------------

def run_decode(cfg: I.DecodeConfig, seed=0):
    x = I.make_decode(cfg, seed)
    mu, nu = x["mu"].cuda(), x["nu"].cuda()
    out = K.decode_step(mu, nu, x["q"].cuda(), x["k"].cuda(), x["v"].cuda(),
                        I.MAP_NAMES[cfg.mapk], omega=dev(x["omega"]),
                        decay=dev(x["decay"]))
    torch.cuda.synchronize()
    ro, rmu, rnu = oracle.decode(f64(x["mu"]), f64(x["nu"]), f64(x["q"]),
                                 f64(x["k"]), f64(x["v"]), cfg.mapk,
                                 f64(x["omega"]), f64(x["decay"]))
    return rel(out, ro), rel(mu, rmu), rel(nu, rnu)


# --------------------------------------------------------------------------
# Prefill -> decode hand-off: the state after the last position
# --------------------------------------------------------------------------

def _oracle_state(x, cfg):
    """mu_n, nu_n by the oracle's decode step applied to every position from
    a zero state (the literal eqs 7-8 / 10-11)."""
    B, H, n, d = x["v"].shape
    mu = np.zeros((B, H, cfg.d_feat, d))
    nu = np.zeros((B, H, cfg.d_feat))
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    for j in range(n):
        _, mu, nu = oracle.decode(mu, nu, q[:, :, j], k[:, :, j], v[:, :, j],
                                  cfg.mapk, f64(x["omega"]), f64(x["decay"]))
    return mu, nu


STATE_CASES = {
    # several segments per unit (the last one hands the state out)
    "elu1_segmented": I.ELU1_CAUSAL.replace(B=2, H=2, n=1000),
    "elu1_decay_d128": I.DECAYED.replace(B=1, H=2, n=700),
    "performer_fused": I.PERFORMER.replace(B=1, H=2, n=300, m=64),
    "fp32_decay_d32": I.ELU1_CAUSAL.replace(B=2, H=1, n=333, d=32,
                                            dtype=torch.float32,
                                            decay=(-2.0, -1.0)),
    "one_chunk": I.ELU1_CAUSAL.replace(B=1, H=3, n=40),
    "noncausal": I.ELU1_CAUSAL.replace(B=1, H=2, n=500, causal=False),
    # fp32, d = 128, d' = 256: two value halves each hand out their columns
    "fp32_split_values_df256": I.PrefillConfig(
        "fp32_split_values_df256", B=1, H=2, n=450, d=128,
        dtype=torch.float32, mapk=I.MAP_PERFORMER, m=256, qk_std=0.5,
        decay=(-2.0, -1.0)),
}


@pytest.mark.parametrize("name", sorted(STATE_CASES))
def test_forward_state_matches_oracle(name):
    cfg = STATE_CASES[name]
    x = I.make_prefill(cfg, 31)
    mu = torch.empty(cfg.B, cfg.H, cfg.d_feat, cfg.d, device="cuda")
    nu = torch.empty(cfg.B, cfg.H, cfg.d_feat, device="cuda")
    out = K.forward(dev(x["q"]), dev(x["k"]), dev(x["v"]),
                    I.MAP_NAMES[cfg.mapk], omega=dev(x["omega"]),
                    decay=dev(x["decay"]), causal=cfg.causal, mu_out=mu,
                    nu_out=nu)
    torch.cuda.synchronize()
    rmu, rnu = _oracle_state(x, cfg)
    ref = oracle.forward(f64(x["q"]), f64(x["k"]), f64(x["v"]), cfg.mapk,
                         f64(x["omega"]), f64(x["decay"]), cfg.causal)
    # the state is fp32, accumulated from features rounded to the storage type
    assert rel(out, ref) <= TOL[cfg.dtype]
    assert rel(mu, rmu) <= TOL[cfg.dtype]
    assert rel(nu, rnu) <= TOL[cfg.dtype]


def test_forward_state_empty_sequence_is_zero():
    mu = torch.full((2, 3, 64, 64), 7.0, device="cuda")
    nu = torch.full((2, 3, 64), 7.0, device="cuda")
    e = torch.empty(2, 3, 0, 64, dtype=torch.bfloat16, device="cuda")
    K.forward(e, e, e, mu_out=mu, nu_out=nu)
    torch.cuda.synchronize()
    assert mu.abs().max().item() == 0.0 and nu.abs().max().item() == 0.0


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("decay", [False, True])
def test_prefill_state_then_decode_continues(dtype, decay):
    """Prefill the first n0 positions with the state handed out, then decode
    the rest token by token: the outputs equal one forward over all n."""
    n, n0 = 600, 536
    cfg = I.ELU1_CAUSAL.replace(B=2, H=2, n=n, d=32, dtype=dtype,
                                decay=(-2.0, -1.0) if decay else None)
    x = I.make_prefill(cfg, 41)
    q, k, v, dec = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["decay"])
    full = K.forward(q, k, v, decay=dec)
    mu = torch.empty(2, 2, 32, 32, device="cuda")
    nu = torch.empty(2, 2, 32, device="cuda")
    K.forward(q[:, :, :n0].contiguous(), k[:, :, :n0].contiguous(),
              v[:, :, :n0].contiguous(), decay=dec, mu_out=mu, nu_out=nu)
    outs = [K.decode_step(mu, nu, q[:, :, j].contiguous(),
                          k[:, :, j].contiguous(), v[:, :, j].contiguous(),
                          decay=dec) for j in range(n0, n)]
    torch.cuda.synchronize()
    chain = torch.stack(outs, dim=2).float()
    tail = full[:, :, n0:].float()
    err = (chain - tail).abs().max().item() / tail.abs().max().item()
    assert err <= TOL[dtype]


@pytest.mark.parametrize("cfg", [
    I.DECODE.replace(name="dec_small", S=4, H=3),
    I.DECODE.replace(name="dec_d64_nodecay", S=3, H=5, d=64, a=None),
    I.DECODE.replace(name="dec_d16", S=2, H=2, d=16),
    I.DECODE.replace(name="dec_performer", S=3, H=2, d=64, m=256,
                     mapk=I.MAP_PERFORMER),
    I.DECODE.replace(name="dec_fp32", S=2, H=3, dtype=torch.float32),
], ids=lambda c: c.name)
def test_decode_small(cfg):
    eo, emu, enu = run_decode(cfg, 9)
    assert eo <= TOL[cfg.dtype] and emu <= 1e-4 and enu <= 1e-4


def test_decode_full_workload():
    """S=256 sequences x H=32 heads, d=d'=128, a=0.99: every unit checked."""
    eo, emu, enu = run_decode(I.DECODE, 0)
    assert eo <= 1e-2 and emu <= 1e-4 and enu <= 1e-4


@pytest.mark.parametrize("mapk", ["elu1", "identity"])
@pytest.mark.parametrize("decay", [False, True])
def test_decode_chain_reproduces_forward(mapk, decay):
    """Token-by-token decode from a zero fp32 state equals the prefill."""
    B, H, n, d = 2, 2, 80, 32
    g = torch.Generator().manual_seed(10)
    if mapk == "identity":
        q = torch.rand(B, H, n, d, generator=g) + 0.1
        k = torch.rand(B, H, n, d, generator=g) + 0.1
    else:
        q = torch.randn(B, H, n, d, generator=g)
        k = torch.randn(B, H, n, d, generator=g)
    v = torch.randn(B, H, n, d, generator=g)
    dec = torch.tensor([0.9, 0.97]) if decay else None
    fwd = K.forward(q.cuda(), k.cuda(), v.cuda(), mapk, decay=dev(dec))
    mu = torch.zeros(B, H, d, d, device="cuda")
    nu = torch.zeros(B, H, d, device="cuda")
    outs = []
    for j in range(n):
        outs.append(K.decode_step(mu, nu, q[:, :, j].contiguous().cuda(),
                                  k[:, :, j].contiguous().cuda(),
                                  v[:, :, j].contiguous().cuda(), mapk,
                                  decay=dev(dec)))
    chain = torch.stack(outs, dim=2)
    torch.cuda.synchronize()
    err = (chain - fwd).abs().max().item() / fwd.abs().max().item()
    assert err <= 1e-4
