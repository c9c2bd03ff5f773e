#!/usr/bin/env python3
"""Throughput of causal kernelized linear attention on one MI355X.

One step = one la_forward call over one batch of synthetic, HBM-resident
input (all hot-path kernels).  Default workload: elu+1 causal, B=4, H=8,
n=4096, d=d'=64, bf16 storage.  The inputs (67 MB per set) fit in the 256 MB
MALL, so the timed loop rotates over enough distinct buffer sets (> 300 MB) that
every step reads from HBM.

Prints one JSON line:  tokens/s (B*H*n per second), the roofline of the hot
path (HBM bound: algorithmic bytes = read q, k, v and write out once), and
the fp64 CPU oracle timed on the host on a bounded sample.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal linear-attn fwd tokens/s (B·H·n/s) + % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
MALL_BYTES = 256 << 20


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "kernelized_attention_scan_amd",
                                           "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def workloads():
    from kernelized_attention_scan_amd import inputs as I
    return {"elu1": I.ELU1_CAUSAL, "decayed": I.DECAYED,
            "performer": I.PERFORMER, "tiny": I.TINY_FP32}


def algorithmic(cfg):
    """Bytes and flops the method itself must move / compute per step."""
    esz = 2 if "bfloat16" in str(cfg.dtype) else 4
    tokens = cfg.tokens
    byts = tokens * 4 * cfg.d * esz                 # read q, k, v; write out
    df = cfg.d_feat
    flops = tokens * (4 * df * cfg.d + 4 * df)      # state update + readout
    if cfg.mapk == 2:
        flops += tokens * 2 * 2 * cfg.d * cfg.m     # phi projection, q and k
    return byts, flops


def load_traffic(workload: str):
    """Counter-measured HBM bytes per step, if taken on the current kernels."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_src_sha") != kernel_source_hash():
        return None
    return t.get("traffic_bytes")


def cpu_baseline(cfg, seed: int, budget_s: float = 20.0):
    """The fp64 oracle on the host cores over a bounded sample of units."""
    import numpy as np
    import oracle
    from kernelized_attention_scan_amd import inputs as I
    x = I.make_prefill(cfg, seed)
    f64 = lambda t: None if t is None else t.double().numpy()
    q, k, v = x["q"], x["k"], x["v"]
    units = cfg.B * cfg.H
    # calibrate on one unit, then take as many units as fit the budget
    t0 = time.perf_counter()
    oracle.forward(f64(q[:1, :1]), f64(k[:1, :1]), f64(v[:1, :1]), cfg.mapk,
                   f64(x["omega"]),
                   None if x["decay"] is None else f64(x["decay"][:1]),
                   cfg.causal)
    one = time.perf_counter() - t0
    threads = oracle.num_threads()
    take = max(1, min(units, int(budget_s / max(one, 1e-9)) * threads // 1))
    take = min(take, units)
    flat = lambda t: t.reshape(units, 1, cfg.n, t.shape[-1])[:take]
    dec = None
    if x["decay"] is not None:
        dec = x["decay"].repeat(cfg.B)[:take]
    qs, ks, vs = flat(q), flat(k), flat(v)
    t0 = time.perf_counter()
    oracle.forward(f64(qs).reshape(1, take, cfg.n, -1),
                   f64(ks).reshape(1, take, cfg.n, -1),
                   f64(vs).reshape(1, take, cfg.n, -1), cfg.mapk,
                   f64(x["omega"]), None if dec is None else f64(dec),
                   cfg.causal)
    dt = time.perf_counter() - t0
    tokens = take * cfg.n
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{take} of {units} (batch, head) units x n={cfg.n} of "
                      f"workload {cfg.name}, fp64 literal recurrence, "
                      f"{dt:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="elu1", choices=sorted(workloads()))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not "
              "supported (the method shards over (batch, head) units with no "
              "exchange; see the design notes)", file=sys.stderr)
        return 2

    import torch
    import kernelized_attention_scan_amd as K
    from kernelized_attention_scan_amd import inputs as I

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    K.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = workloads()[args.workload]
    mapname = I.MAP_NAMES[cfg.mapk]
    byts, flops = algorithmic(cfg)

    # distinct buffer sets, together larger than the MALL
    set_bytes = byts + (cfg.d * cfg.m * 4 if cfg.mapk == 2 else 0)
    nsets = max(1, min(8, math.ceil(1.2 * MALL_BYTES / set_bytes)))
    sets = []
    for i in range(nsets):
        x = I.make_prefill(cfg, args.seed + i)
        sets.append({k: (None if t is None else t.to(dev)) for k, t in x.items()})
    outs = [torch.empty_like(s["v"]) for s in sets]
    ws = K.new_workspace(cfg.B, cfg.H, cfg.n, cfg.d, cfg.d_feat, mapname,
                         cfg.dtype, cfg.causal, device=dev)

    def step(i):
        s = sets[i % nsets]
        K.forward(s["q"], s["k"], s["v"], feature_map=mapname,
                  omega=s["omega"], decay=s["decay"], causal=cfg.causal,
                  out=outs[i % nsets], workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)   # the library launches here
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = ev0.elapsed_time(ev1) / args.steps

    tokens_per_s = cfg.tokens / (ms * 1e-3)
    achieved = byts / (ms * 1e-3) / 1e9
    traffic = load_traffic(cfg.name)
    line = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "n": cfg.n,
                   "d": cfg.d, "d_feat": cfg.d_feat, "map": mapname,
                   "decay": cfg.decay, "causal": cfg.causal,
                   "buffer_sets": nsets, "seed": args.seed},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "kernel": "la_forward (one call: all hot-path kernels)",
                     "algorithmic_bytes_per_launch": byts,
                     "algorithmic_flops_per_launch": flops,
                     "mfma_frac_algorithmic":
                         flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "wall_s_timed_region": t_wall,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.seed)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
