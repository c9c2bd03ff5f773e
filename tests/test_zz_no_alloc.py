"""The allocation-free forward (la_forward_noalloc, static per-GPU scratch)
against la_forward with a workspace, through the C ABI: two calls in a row,
the second with a smaller input, plus a non-causal call and one whose
segment split is shrunk to fit the scratch.  Tolerance: 1e-2 relative
(bf16 storage), the same bar as the oracle parity tests."""
import numpy as np
import pytest
import torch

import kernelized_attention_scan_amd as K
from kernelized_attention_scan_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    K.load_library()
    torch.cuda.set_device(0)
    yield


def _dev(t):
    return None if t is None else t.cuda()


def _rel(a, b):
    a = a.float().cpu().double().numpy()
    b = b.float().cpu().double().numpy()
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b))
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


CASES = [
    # segmented decayed d=128 (the larger call), then a smaller elu1 call
    I.DECAYED.replace(name="noalloc_big", n=8192),
    I.ELU1_CAUSAL.replace(name="noalloc_small", B=1, H=2, n=1000),
    # non-causal: the two-launch form through the scratch
    I.ELU1_CAUSAL.replace(name="noalloc_noncausal", B=1, H=3, n=2000,
                          causal=False),
    # fused Performer, d' = 256: aggregates of 256 x 80 floats
    I.PERFORMER.replace(name="noalloc_performer", n=2048),
    # identity features d' = 256, d = 128 over 17 units x 16 segments would
    # need 40 MB of partial sums: the split is shrunk to fit the 32 MiB
    # scratch
    I.PrefillConfig("noalloc_shrunk", B=1, H=17, n=8192, d=128,
                    mapk=I.MAP_IDENTITY, m=256),
]


def _inputs(cfg, seed):
    if cfg.mapk != I.MAP_IDENTITY:
        return I.make_prefill(cfg, seed)
    g = torch.Generator().manual_seed(seed)      # positive features
    sh = (cfg.B, cfg.H, cfg.n, cfg.m)
    return {"q": (torch.rand(sh, generator=g) + 0.05).to(cfg.dtype),
            "k": (torch.rand(sh, generator=g) + 0.05).to(cfg.dtype),
            "v": torch.randn((cfg.B, cfg.H, cfg.n, cfg.d),
                             generator=g).to(cfg.dtype),
            "omega": None, "decay": None}


def test_noalloc_matches_forward_in_sequence():
    for cfg in CASES:
        x = _inputs(cfg, 3)
        name = I.MAP_NAMES[cfg.mapk]
        args = [_dev(x["q"]), _dev(x["k"]), _dev(x["v"]), name]
        kw = dict(omega=_dev(x["omega"]), decay=_dev(x["decay"]),
                  causal=cfg.causal)
        out = torch.empty_like(args[2])
        K.forward_noalloc(*args, out=out, **kw)
        ref = K.forward(*args, **kw)
        torch.cuda.synchronize()
        err = _rel(out, ref)
        print(f"{cfg.name}: rel diff {err:.2e}", flush=True)
        assert err <= 1e-2, (cfg.name, err)


def test_noalloc_rejects_unfused_performer():
    cfg = I.PERFORMER.replace(n=4096, dtype=torch.float32)
    x = I.make_prefill(cfg, 4)
    with pytest.raises(K.LinAttnError) as e:
        K.forward_noalloc(_dev(x["q"]), _dev(x["k"]), _dev(x["v"]),
                          "performer", omega=_dev(x["omega"]))
    assert e.value.status == K._binding.LA_ERR_UNSUPPORTED
