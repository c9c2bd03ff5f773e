"""Seeded synthetic inputs for the prefill and decode workloads.

This module draws random numbers and rounds them to the storage dtype; it
holds none of the method's arithmetic (no feature map, no state, no
readout).  It is the one piece of code that both the HIP path's callers
(tests, benchmark) and the fp64 oracle's callers use, so both sides see the
very same values.

Draw order per workload, all with ``torch.Generator('cpu').manual_seed(seed)``
and fp32 ``randn`` / ``rand``:

* prefill: Q, K, V (each [B, H, n, d], scaled by ``qk_std`` / ``v_std``),
  then omega [d, m] = randn / sqrt(d) (Performer only), then u [H] ~ U(0, 1)
  with the per-head decay a = 1 - 10^(lo + (hi - lo) u) (decayed only), then
  (gated only) u [H] ~ U(0, 1) with A_h = -10^(lo + (hi - lo) u) and z
  [B, H, n] ~ N(0, 1) with step delta = softplus(z): the per-position log
  decay is A_h * delta, the selective step of the Mamba section (a rate per
  head times an input-dependent step);
* decode: mu = |randn| * ctx, nu = |randn| * ctx, then q, k, v, then omega.

Tensors with bf16 storage are rounded once, fp32 -> bf16 round-to-nearest-even,
here; omega, decay, mu and nu stay fp32.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

MAP_IDENTITY, MAP_ELU1, MAP_PERFORMER = 0, 1, 2
MAP_NAMES = {MAP_IDENTITY: "identity", MAP_ELU1: "elu1",
             MAP_PERFORMER: "performer"}


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    H: int
    n: int
    d: int
    dtype: torch.dtype = torch.bfloat16
    mapk: int = MAP_ELU1
    m: int = 0                       # Performer feature count (d_feat)
    qk_std: float = 1.0
    v_std: float = 1.0
    decay: Optional[tuple] = None    # (lo, hi): 1 - a = 10^U(lo, hi)
    causal: bool = True
    gate: Optional[tuple] = None     # (lo, hi): log decay -10^U(lo,hi) * delta

    @property
    def d_feat(self) -> int:
        return self.m if self.mapk == MAP_PERFORMER else self.d

    @property
    def tokens(self) -> int:
        return self.B * self.H * self.n

    def replace(self, **kw) -> "PrefillConfig":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    S: int
    H: int
    d: int
    dtype: torch.dtype = torch.bfloat16
    mapk: int = MAP_ELU1
    m: int = 0
    ctx: float = 4096.0              # state magnitude ~ context length
    a: Optional[float] = 0.99        # one decay value for every head

    @property
    def d_feat(self) -> int:
        return self.m if self.mapk == MAP_PERFORMER else self.d

    def replace(self, **kw) -> "DecodeConfig":
        return dataclasses.replace(self, **kw)


# The five workloads of the method's hot path, by what they are.
TINY_FP32 = PrefillConfig("tiny_fp32_elu1_B1H1n256d16", B=1, H=1, n=256, d=16,
                          dtype=torch.float32)
ELU1_CAUSAL = PrefillConfig("elu1_causal_B4H8n4096d64", B=4, H=8, n=4096, d=64)
ELU1_NONCAUSAL = PrefillConfig("elu1_noncausal_B4H8n4096d64", B=4, H=8,
                               n=4096, d=64, causal=False)
DECAYED = PrefillConfig("decayed_elu1_B2H16n65536d128", B=2, H=16, n=65536,
                        d=128, decay=(-3.0, -1.0))
PERFORMER = PrefillConfig("performer_B4H8n8192d64m256", B=4, H=8, n=8192, d=64,
                          mapk=MAP_PERFORMER, m=256, qk_std=0.5)
# Input-dependent (per-position) decay at the decayed workload's sizes.
GATED = PrefillConfig("gated_elu1_B2H16n65536d128", B=2, H=16, n=65536,
                      d=128, gate=(-3.0, -1.0))
# A decay per state row (per channel, [H, d_feat]) at the same sizes; its
# log decays come from row_log_decay.
CHANNEL = PrefillConfig("channel_elu1_B2H16n65536d128", B=2, H=16, n=65536,
                        d=128)
DECODE = DecodeConfig("decode_S256H32d128_a0.99", S=256, H=32, d=128)
# the same step with a decay per state row (per channel, [H, d_feat])
DECODE_CHANNEL = DecodeConfig("decode_channel_S256H32d128", S=256, H=32,
                              d=128, a=None)

PREFILL_CONFIGS = {c.name: c for c in (TINY_FP32, ELU1_CAUSAL, ELU1_NONCAUSAL,
                                       DECAYED, PERFORMER, GATED, CHANNEL)}


def _round(x: torch.Tensor, dtype: torch.dtype) -> torch.Tensor:
    return x.to(dtype) if dtype != torch.float32 else x


def make_prefill(cfg: PrefillConfig, seed: int = 0) -> dict:
    """CPU tensors q, k, v (storage dtype), omega (fp32 or None),
    decay (fp32 [H] or None), log_decay (fp32 [B, H, n] or None)."""
    g = torch.Generator("cpu").manual_seed(seed)
    shape = (cfg.B, cfg.H, cfg.n, cfg.d)
    q = torch.randn(shape, generator=g) * cfg.qk_std
    k = torch.randn(shape, generator=g) * cfg.qk_std
    v = torch.randn(shape, generator=g) * cfg.v_std
    omega = None
    if cfg.mapk == MAP_PERFORMER:
        omega = torch.randn((cfg.d, cfg.m), generator=g) / (cfg.d ** 0.5)
    decay = None
    if cfg.decay is not None:
        lo, hi = cfg.decay
        u = torch.rand((cfg.H,), generator=g)
        decay = (1.0 - torch.pow(10.0, lo + (hi - lo) * u)).to(torch.float32)
    log_decay = None
    if cfg.gate is not None:
        lo, hi = cfg.gate
        u = torch.rand((cfg.H,), generator=g)
        rate = -torch.pow(10.0, lo + (hi - lo) * u)
        z = torch.randn((cfg.B, cfg.H, cfg.n), generator=g)
        step = torch.nn.functional.softplus(z)
        log_decay = (rate[None, :, None] * step).to(torch.float32).contiguous()
    return {"q": _round(q, cfg.dtype), "k": _round(k, cfg.dtype),
            "v": _round(v, cfg.dtype), "omega": omega, "decay": decay,
            "log_decay": log_decay}


def make_decode(cfg: DecodeConfig, seed: int = 0) -> dict:
    """CPU tensors mu [S,H,d_feat,d], nu [S,H,d_feat] (fp32); q, k, v [S,H,d]
    (storage dtype); omega; decay [H] fp32 or None."""
    g = torch.Generator("cpu").manual_seed(seed)
    df = cfg.d_feat
    mu = torch.randn((cfg.S, cfg.H, df, cfg.d), generator=g).abs() * cfg.ctx
    nu = torch.randn((cfg.S, cfg.H, df), generator=g).abs() * cfg.ctx
    q = torch.randn((cfg.S, cfg.H, cfg.d), generator=g)
    k = torch.randn((cfg.S, cfg.H, cfg.d), generator=g)
    v = torch.randn((cfg.S, cfg.H, cfg.d), generator=g)
    omega = None
    if cfg.mapk == MAP_PERFORMER:
        omega = torch.randn((cfg.d, cfg.m), generator=g) / (cfg.d ** 0.5)
    decay = None
    if cfg.a is not None:
        decay = torch.full((cfg.H,), float(cfg.a), dtype=torch.float32)
    return {"mu": mu, "nu": nu, "q": _round(q, cfg.dtype),
            "k": _round(k, cfg.dtype), "v": _round(v, cfg.dtype),
            "omega": omega, "decay": decay}


def decode_channel_log_decay(cfg: DecodeConfig, seed: int = 0) -> torch.Tensor:
    """Per-channel log decays [H, d_feat] (fp32) for the decode step: log(1 -
    10^U(-3, -1)), drawn from their own generator (seed + 101) so the other
    decode inputs of the same seed are unchanged."""
    g = torch.Generator("cpu").manual_seed(seed + 101)
    u = torch.rand((cfg.H, cfg.d_feat), generator=g)
    return torch.log1p(-(10.0 ** (-3.0 + 2.0 * u)))


def row_log_decay(cfg: PrefillConfig, seed: int = 0, layout: str = "channel",
                  lo: float = -3.0, hi: float = -1.0,
                  d_feat: Optional[int] = None) -> torch.Tensor:
    """Log decays per state row (fp32), from their own generator (seed + 202)
    so the other prefill inputs of the same seed are unchanged:
    "channel": [H, d_feat] = log(1 - 10^U(lo, hi));
    "both": [B, H, n, d_feat] = A * softplus(z) with a rate per head and row
    A = -10^U(lo, hi) [H, d_feat] and z [B, H, n, d_feat] ~ N(0, 1), the
    per-position recipe of make_prefill applied row by row.  d_feat
    overrides the config's feature width (features given directly)."""
    g = torch.Generator("cpu").manual_seed(seed + 202)
    df = d_feat or cfg.d_feat
    u = torch.rand((cfg.H, df), generator=g)
    if layout == "channel":
        return torch.log1p(-(10.0 ** (lo + (hi - lo) * u))).to(torch.float32)
    if layout != "both":
        raise ValueError(f"unknown layout {layout!r}")
    rate = -torch.pow(10.0, lo + (hi - lo) * u)
    z = torch.randn((cfg.B, cfg.H, cfg.n, df), generator=g)
    step = torch.nn.functional.softplus(z)
    return (rate[None, :, None, :] * step).to(torch.float32).contiguous()
