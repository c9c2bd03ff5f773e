#!/usr/bin/env python3
"""Throughput of causal kernelized linear attention on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic,
HBM-resident input:
  prefill workloads: one la_forward call (Performer: the two feature-map
    launches and the chunked forward it makes);
  decode: one la_decode_step over every (sequence, head) unit.
Default workload: the decayed recurrence (eqs 10-11), elu+1 causal, B=2,
H=16, n=65536, d=d'=128, bf16 storage, one decay value per head.  Its inputs
(2.1 GB) do not fit in the 256 MB MALL; workloads whose inputs do fit (elu1,
performer) rotate over enough distinct buffer sets (> 300 MB) that every step
reads from HBM.

Prints one JSON line: throughput (tokens/s = B*H*n per second; decode:
(sequence, head) units per second), the roofline of the dominant kernel
(HBM bound: algorithmic bytes per launch / its measured duration), and the
fp64 CPU oracle timed on the host cores over a bounded sample.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import re
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


# The sources each timed kernel is built from (device code and the host
# code that picks its launch shape); a change to any of them voids the
# counter-measured traffic taken on the old build.
KERNEL_SOURCES = {
    "forward": ["la_device.h", "la_internal.h", "la_forward.h",
                "la_forward_inst.h", "la_forward_bf16.hip",
                "la_forward_bf16_pf.hip", "la_forward_f32.hip",
                "la_api.cpp"],
    "decode": ["la_device.h", "la_internal.h", "la_decode.hip", "la_api.cpp"],
    "backward": ["la_device.h", "la_internal.h", "la_backward.hip",
                 "la_featmap.hip", "la_api.cpp"],
    "rows": ["la_device.h", "la_internal.h", "la_forward_rows.h",
             "la_forward_rows_inst.h", "la_forward_rows.hip",
             "la_forward_rows_bf16.hip", "la_forward_rows_f32.hip",
             "la_api.cpp"],
}


def kernel_kind(workload: str) -> str:
    if workload.startswith("decode"):
        return "decode"
    if workload == "channel":
        return "rows"
    return "backward" if workload.startswith("backward") else "forward"


def kernel_source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for name in sorted(KERNEL_SOURCES[kind]):
        with open(os.path.join(ROOT, "kernelized_attention_scan_amd", "csrc",
                               name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def workloads():
    from kernelized_attention_scan_amd import inputs as I
    return {"elu1": I.ELU1_CAUSAL, "decayed": I.DECAYED,
            "performer": I.PERFORMER, "tiny": I.TINY_FP32,
            "decode": I.DECODE, "noncausal": I.ELU1_NONCAUSAL,
            "gated": I.GATED, "backward": I.DECAYED, "channel": I.CHANNEL,
            "decode_channel": I.DECODE_CHANNEL,
            "backward_performer": I.PERFORMER, "backward_gated": I.GATED}


def esize(dtype) -> int:
    return 2 if "bfloat16" in str(dtype) else 4


def prefill_algorithmic(cfg, channel: bool = False):
    """Bytes and flops the method itself must move / compute per step: read
    q, k, v and write out once (with a decay per channel, read its [H,
    d_feat] log decays once too); 4 d' d + 4 d' flops per token (state
    update and readout), plus the Performer projection of q and k."""
    byts = cfg.tokens * 4 * cfg.d * esize(cfg.dtype)
    if channel:
        byts += cfg.H * cfg.d_feat * 4
    df = cfg.d_feat
    flops = cfg.tokens * (4 * df * cfg.d + 4 * df)
    if cfg.mapk == 2:
        flops += cfg.tokens * 2 * 2 * cfg.d * cfg.m
    return byts, flops


def decode_algorithmic(cfg, channel: bool = False):
    """Per step: read and write mu, nu (fp32) once; read q, k, v and write
    out (storage dtype); with a decay per channel, read the [H, d_feat] log
    decays once."""
    units = cfg.S * cfg.H
    df, d = cfg.d_feat, cfg.d
    byts = units * (2 * df * d * 4 + 2 * df * 4 + 4 * d * esize(cfg.dtype))
    if channel:
        byts += cfg.H * df * 4
    flops = units * (4 * df * d + 4 * df)
    return byts, flops


def load_traffic(workload: str):
    """Counter-measured HBM bytes per launch of the dominant kernel, if taken
    on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_src_sha") != kernel_source_hash(kernel_kind(workload)):
        return None
    return t.get("traffic_bytes")


def settle(torch, fn, ms: float):
    """Run fn(i) untimed until about `ms` milliseconds of GPU work have
    passed, so the timed steps run at the clocks a sustained load holds
    (the first tens of milliseconds of a fresh load run slower)."""
    if ms <= 0:
        return 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            fn(i)
            i += 1
        torch.cuda.synchronize()
    return i


def time_loop(torch, fn, steps: int, stream):
    """Average ms per call of fn(i) over `steps` calls, HIP events recorded on
    the stream the library launches on."""
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(steps):
        fn(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


# --------------------------------------------------------------------------
# CPU baselines: the fp64 oracle, as it stands, on a bounded sample
# --------------------------------------------------------------------------

def cpu_baseline_prefill(cfg, seed: int, budget_s: float = 20.0,
                         channel: bool = False):
    import oracle
    from kernelized_attention_scan_amd import inputs as I
    x = I.make_prefill(cfg, seed)
    # a decay per channel: [H, d_feat] per head, repeated for each batch row
    # of the flattened units
    chl = (I.row_log_decay(cfg, seed, "channel").repeat(cfg.B, 1)
           if channel else None)
    f64 = lambda t: None if t is None else t.double().numpy()
    units = cfg.B * cfg.H
    flat = lambda t: t.reshape(1, units, cfg.n, t.shape[-1])
    q, k, v = flat(x["q"]), flat(x["k"]), flat(x["v"])
    dec = None if x["decay"] is None else x["decay"].repeat(cfg.B)
    lam = (None if x["log_decay"] is None
           else x["log_decay"].reshape(1, units, cfg.n))
    om = f64(x["omega"])
    threads = oracle.num_threads()

    def run(take):
        sl = slice(0, take)
        if chl is not None:    # the gated recurrence, a decay per channel
            return oracle.forward_gated(
                f64(q[:, sl]), f64(k[:, sl]), f64(v[:, sl]), cfg.mapk, om,
                f64(chl[sl]), oracle.LD_CHANNEL, cfg.causal)
        if lam is not None:    # the gated recurrence, per-position decay
            return oracle.forward_gated(
                f64(q[:, sl]), f64(k[:, sl]), f64(v[:, sl]), cfg.mapk, om,
                f64(lam[:, sl]), oracle.LD_POSITION, cfg.causal)
        return oracle.forward(f64(q[:, sl]), f64(k[:, sl]), f64(v[:, sl]),
                              cfg.mapk, om,
                              None if dec is None else f64(dec[sl]),
                              cfg.causal)

    # calibrate on one unit per thread, then take as many units as fit
    probe = min(units, threads)
    t0 = time.perf_counter()
    run(probe)
    per_round = time.perf_counter() - t0
    take = int(budget_s / max(per_round, 1e-9)) * probe
    take = max(probe, min(units, take))
    reps, dt = 0, 0.0
    while reps == 0 or dt < 2.0:      # repeat a short sample for a stable time
        t0 = time.perf_counter()
        run(take)
        dt += time.perf_counter() - t0
        reps += 1
    return {"value": reps * take * cfg.n / dt, "unit": "tokens/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{take} of {units} (batch, head) units x n={cfg.n} of "
                      f"workload {cfg.name}, {reps} pass(es); fp64 literal "
                      f"recurrence, {dt:.1f} s"}


def cpu_baseline_decode(cfg, seed: int, budget_s: float = 10.0,
                        channel: bool = False):
    import oracle
    from kernelized_attention_scan_amd import inputs as I
    x = I.make_decode(cfg, seed)
    f64 = lambda t: None if t is None else t.double().numpy()
    lam = f64(I.decode_channel_log_decay(cfg, seed)) if channel else None
    threads = oracle.num_threads()
    S = cfg.S

    def run(take):
        a = (f64(x["mu"][:take]), f64(x["nu"][:take]), f64(x["q"][:take]),
             f64(x["k"][:take]), f64(x["v"][:take]), cfg.mapk,
             f64(x["omega"]))
        if channel:
            oracle.decode_gated(*a, lam, oracle.LD_CHANNEL)
        else:
            oracle.decode(*a, f64(x["decay"]))

    probe = max(1, min(S, threads))
    t0 = time.perf_counter()
    run(probe)
    per = time.perf_counter() - t0
    take = max(probe, min(S, int(budget_s / max(per, 1e-9)) * probe))
    t0 = time.perf_counter()
    run(take)
    dt = time.perf_counter() - t0
    return {"value": take * cfg.H / dt, "unit": "head-tokens/s",
            "cores": threads, "kind": "oracle",
            "sample": f"{take} of {S} sequences x H={cfg.H} of workload "
                      f"{cfg.name}; fp64 decode step (input conversion "
                      f"included), {dt:.2f} s"}


# --------------------------------------------------------------------------
# GPU legs
# --------------------------------------------------------------------------

def prefill_leg(torch, K, I, cfg, args, dev):
    mapname = I.MAP_NAMES[cfg.mapk]
    channel = args.workload == "channel"
    byts, flops = prefill_algorithmic(cfg, channel)
    set_bytes = byts + (cfg.d * cfg.m * 4 if cfg.mapk == 2 else 0)
    nsets = max(1, min(8, math.ceil(1.2 * MALL_BYTES / set_bytes)))
    sets = []
    for i in range(nsets):
        x = I.make_prefill(cfg, args.seed + i)
        if channel:
            x["row_log_decay"] = I.row_log_decay(cfg, args.seed + i, "channel")
        sets.append({k: (None if t is None else t.to(dev)) for k, t in x.items()})
    outs = [torch.empty_like(s["v"]) for s in sets]
    if channel:
        ws = torch.zeros(max(1, K.gated_workspace_bytes(
            cfg.B, cfg.H, cfg.n, cfg.d, cfg.d_feat, mapname, "channel",
            cfg.dtype, cfg.causal)), dtype=torch.uint8, device=dev)
    else:
        ws = K.new_workspace(cfg.B, cfg.H, cfg.n, cfg.d, cfg.d_feat, mapname,
                             cfg.dtype, cfg.causal, device=dev)
    stream = torch.cuda.current_stream(dev)   # the library launches here

    def step(i):
        s = sets[i % nsets]
        if channel:                      # a decay per channel
            K.forward_gated(s["q"], s["k"], s["v"], s["row_log_decay"],
                            "channel", feature_map=mapname, omega=s["omega"],
                            causal=cfg.causal, out=outs[i % nsets],
                            workspace=ws)
            return
        if s["log_decay"] is not None:   # per-position decay
            K.forward_gated(s["q"], s["k"], s["v"], s["log_decay"],
                            "position", feature_map=mapname, omega=s["omega"],
                            causal=cfg.causal, out=outs[i % nsets],
                            workspace=ws)
            return
        K.forward(s["q"], s["k"], s["v"], feature_map=mapname,
                  omega=s["omega"], decay=s["decay"], causal=cfg.causal,
                  out=outs[i % nsets], workspace=ws)

    settled = settle(torch, step, args.settle_ms)
    for i in range(args.warmup):
        step(i)
    t_wall = time.perf_counter()
    ms = time_loop(torch, step, args.steps, stream)
    t_wall = time.perf_counter() - t_wall

    esz = esize(cfg.dtype)
    # the library fuses the Performer map into the forward when it can (then
    # no q', k' features go through the workspace)
    fused = cfg.mapk == 2 and K.forward_workspace_bytes(
        cfg.B, cfg.H, cfg.n, cfg.d, cfg.m, "performer", cfg.dtype,
        cfg.causal) < 2 * cfg.tokens * cfg.m * esz
    if channel:
        # one call per step: three launches -- the segment aggregates, the
        # carry scan and the readout -- timed together
        kern = {"kernel": "la_fwd_rows_kernel (aggregates) + "
                          "la_fwd_rows_carry_kernel + la_fwd_rows_kernel "
                          "(readout) per step",
                "ms": ms, "bytes": byts, "flops": flops}
    elif cfg.mapk != 2 or fused:
        # one kernel per step: the chunked forward (Performer: map fused)
        kern = {"kernel": "la_fwd_kernel (chunked "
                          + ("causal" if cfg.causal else
                             "non-causal: aggregates, then readout") + " forward"
                          + (", Performer map fused)" if fused else ")"),
                "ms": ms, "bytes": byts, "flops": flops}
    else:
        # Performer: the same two kinds of launch la_forward makes, timed
        # apart -- the feature map (x -> phi(x), per call one of q, k) and the
        # chunked forward over the features.
        rows = cfg.tokens
        feats = [torch.empty(cfg.B, cfg.H, cfg.n, cfg.m, dtype=cfg.dtype,
                             device=dev) for _ in range(2)]
        fws = K.new_workspace(cfg.B, cfg.H, cfg.n, cfg.d, cfg.m, "identity",
                              cfg.dtype, cfg.causal, device=dev)

        def fmap(i):
            s = sets[i % nsets]
            K.featmap(s["q"], "performer", omega=s["omega"], out=feats[0])

        def fwd_feat(i):
            s = sets[i % nsets]
            K.forward(feats[0], feats[1], s["v"], feature_map="identity",
                      causal=cfg.causal, out=outs[i % nsets], workspace=fws)

        fmap(0)
        K.featmap(sets[0]["k"], "performer", omega=sets[0]["omega"],
                  out=feats[1])
        for i in range(3):
            fwd_feat(i)
        ms_f = time_loop(torch, fmap, args.steps, stream)
        ms_w = time_loop(torch, fwd_feat, args.steps, stream)
        f_bytes = rows * (cfg.d + cfg.m) * esz
        w_bytes = cfg.tokens * (2 * cfg.m + 2 * cfg.d) * esz
        w_flops = cfg.tokens * (4 * cfg.m * cfg.d + 4 * cfg.m)
        if ms_w >= ms_f:
            kern = {"kernel": "la_fwd_kernel over Performer features "
                              "(d_feat = m)",
                    "ms": ms_w, "bytes": w_bytes, "flops": w_flops}
        else:
            kern = {"kernel": "la_featmap_performer (one of q, k)",
                    "ms": ms_f, "bytes": f_bytes,
                    "flops": rows * 2 * cfg.d * cfg.m}
        kern["other_launches_ms"] = {"featmap_one_of_q_k": ms_f,
                                     "forward_over_features": ms_w}
    return {"ms": ms, "t_wall": t_wall, "items": cfg.tokens,
            "unit": "tokens/s", "bytes": byts, "flops": flops,
            "kern": kern, "nsets": nsets, "settle_steps": settled,
            "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H,
                       "n": cfg.n, "d": cfg.d, "d_feat": cfg.d_feat,
                       "map": mapname, "decay": cfg.decay, "gate": cfg.gate,
                       "channel_decay": ("log(1 - 10^U(-3,-1)) [H, d_feat]"
                                         if channel else None),
                       "causal": cfg.causal, "buffer_sets": nsets,
                       "seed": args.seed}}


def backward_algorithmic(cfg):
    """Per step of the backward: read q, k, v, out, dout and den (and a
    decay per position, fp32) once, write dq, dk, dv once; flops of the
    three unnormalised linear attentions it is made of (dq' and dk': widths
    d + 1 and d'; dv: d' and d), 4 x width x width per token each."""
    d, df = cfg.d, cfg.d_feat
    byts = cfg.tokens * (8 * d * esize(cfg.dtype) + 4 +
                         (4 if cfg.gate is not None else 0))
    flops = cfg.tokens * (2 * 4 * (d + 1) * df + 4 * df * d)
    return byts, flops


def backward_leg(torch, K, I, cfg, args, dev):
    """One step = la_backward over the whole workload (the training forward
    that produces out and den runs once, before the timed region)."""
    mapname = I.MAP_NAMES[cfg.mapk]
    byts, flops = backward_algorithmic(cfg)
    x = I.make_prefill(cfg, args.seed)
    s = {k: (None if t is None else t.to(dev)) for k, t in x.items()}
    g = torch.Generator("cpu").manual_seed(args.seed + 7)
    dout = torch.randn(cfg.B, cfg.H, cfg.n, cfg.d, generator=g).to(
        cfg.dtype).to(dev)
    out, den = K.forward_train(s["q"], s["k"], s["v"], mapname,
                               decay=s["decay"], omega=s["omega"],
                               log_decay=s["log_decay"])
    grads = [torch.empty_like(s["q"]) for _ in range(3)]
    stream = torch.cuda.current_stream(dev)

    def step(i):
        K.backward(s["q"], s["k"], s["v"], out, den, dout, mapname,
                   decay=s["decay"], dq=grads[0], dk=grads[1], dv=grads[2],
                   omega=s["omega"], log_decay=s["log_decay"])

    settled = settle(torch, step, args.settle_ms)
    for i in range(args.warmup):
        step(i)
    t_wall = time.perf_counter()
    ms = time_loop(torch, step, args.steps, stream)
    t_wall = time.perf_counter() - t_wall
    return {"ms": ms, "t_wall": t_wall, "items": cfg.tokens,
            "unit": "tokens/s", "bytes": byts, "flops": flops,
            "kern": {"kernel": ("la_featmap_performer_kernel x2 + "
                                "la_bwd_prep_kernel + la_bwd_kernel + "
                                "la_bwd_pf_grad_kernel x2 per step")
                               if cfg.mapk == I.MAP_PERFORMER else
                               "la_bwd_prep_kernel + la_bwd_kernel "
                               "(column-block roles) per step"
                               if cfg.gate is not None else
                               "la_bwd_prep_kernel + la_bwd_seg_kernel "
                               "(aggregates, then readout) per step",
                     "ms": ms, "bytes": byts, "flops": flops},
            "nsets": 1, "settle_steps": settled,
            "config": {"workload": "backward_" + cfg.name, "B": cfg.B,
                       "H": cfg.H, "n": cfg.n, "d": cfg.d,
                       "d_feat": cfg.d_feat, "map": mapname,
                       "decay": cfg.decay, "gate": cfg.gate, "causal": True,
                       "seed": args.seed}}


def cpu_baseline_backward(cfg, seed: int, budget_s: float = 15.0):
    import oracle
    from kernelized_attention_scan_amd import inputs as I
    x = I.make_prefill(cfg, seed)
    f64 = lambda t: None if t is None else t.double().numpy()
    g = __import__("torch").Generator("cpu").manual_seed(seed + 7)
    dout = __import__("torch").randn(cfg.B, cfg.H, cfg.n, cfg.d, generator=g)
    units = cfg.B * cfg.H
    flat = lambda t: t.reshape(1, units, cfg.n, t.shape[-1])
    q, k, v, do = flat(x["q"]), flat(x["k"]), flat(x["v"]), flat(dout)
    dec = None if x["decay"] is None else x["decay"].repeat(cfg.B)
    lam = (None if x["log_decay"] is None
           else x["log_decay"].reshape(1, units, cfg.n))
    threads = oracle.num_threads()

    def run(take):
        sl = slice(0, take)
        if lam is not None:
            return oracle.backward_gated(
                f64(q[:, sl]), f64(k[:, sl]), f64(v[:, sl]), f64(do[:, sl]),
                cfg.mapk, f64(x["omega"]), f64(lam[:, sl]),
                oracle.LD_POSITION)
        return oracle.backward(f64(q[:, sl]), f64(k[:, sl]), f64(v[:, sl]),
                               f64(do[:, sl]), cfg.mapk, f64(x["omega"]),
                               None if dec is None else f64(dec[sl]))

    probe = min(units, threads)
    t0 = time.perf_counter()
    run(probe)
    per = time.perf_counter() - t0
    take = max(probe, min(units, int(budget_s / max(per, 1e-9)) * probe))
    t0 = time.perf_counter()
    run(take)
    dt = time.perf_counter() - t0
    return {"value": take * cfg.n / dt, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{take} of {units} (batch, head) units x n={cfg.n} of "
                      f"workload {cfg.name}; fp64 adjoint recurrence "
                      f"(gradients), {dt:.1f} s"}


def decode_leg(torch, K, I, cfg, args, dev):
    mapname = I.MAP_NAMES[cfg.mapk]
    channel = args.workload == "decode_channel"
    byts, flops = decode_algorithmic(cfg, channel)
    x = I.make_decode(cfg, args.seed)
    s = {k: (None if t is None else t.to(dev)) for k, t in x.items()}
    lam = (I.decode_channel_log_decay(cfg, args.seed).to(dev) if channel
           else None)
    out = torch.empty_like(s["v"])
    stream = torch.cuda.current_stream(dev)

    def step(i):
        # mu, nu are updated in place: successive steps form a decode chain
        if channel:
            K.decode_step_gated(s["mu"], s["nu"], s["q"], s["k"], s["v"],
                                lam, "channel", mapname, omega=s["omega"],
                                out=out)
        else:
            K.decode_step(s["mu"], s["nu"], s["q"], s["k"], s["v"], mapname,
                          omega=s["omega"], decay=s["decay"], out=out)

    settled = settle(torch, step, args.settle_ms)
    for i in range(args.warmup):
        step(i)
    t_wall = time.perf_counter()
    ms = time_loop(torch, step, args.steps, stream)
    t_wall = time.perf_counter() - t_wall
    units = cfg.S * cfg.H
    return {"ms": ms, "t_wall": t_wall, "items": units,
            "unit": "head-tokens/s", "bytes": byts, "flops": flops,
            "kern": {"kernel": "la_decode_kernel (state streamed once)",
                     "ms": ms, "bytes": byts, "flops": flops},
            "nsets": 1, "settle_steps": settled,
            "config": {"workload": cfg.name, "S": cfg.S, "H": cfg.H,
                       "d": cfg.d, "d_feat": cfg.d_feat, "map": mapname,
                       "a": cfg.a,
                       "decay": ("per channel: log(1 - 10^U(-3,-1)) [H, "
                                 "d_feat]" if channel else "per head"),
                       "seed": args.seed}}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decayed",
                    choices=sorted(workloads()))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--n", type=int, default=0,
                    help="sequence length other than the workload's own "
                         "(prefill workloads; for length sweeps)")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed steps for this long before the warmup "
                         "steps, so clocks reach their sustained level")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-MiB buffer three times (a kernel of "
                         "known HBM traffic, to scale the profiler's byte "
                         "counters) and exit")
    ap.add_argument("--stream-rate", type=int, default=0, metavar="MIB",
                    help="only time plain streaming kernels over MIB-MiB "
                         "buffers (torch's elementwise add, which reads and "
                         "writes each byte once, and a device copy), print "
                         "their rates and exit: what a plain kernel reaches "
                         "on this GPU, beside the 8 TB/s peak")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not "
              "supported: this build runs on a single GPU (units of (batch, "
              "head) shard across GPUs with no exchange, see the design "
              "notes)", file=sys.stderr)
        return 2

    import torch
    import kernelized_attention_scan_amd as K
    from kernelized_attention_scan_amd import inputs as I

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": nbytes,
                          "copy_calibration_bytes_written": nbytes,
                          "launches": 3}), flush=True)
        return 0
    if args.stream_rate:
        n = (args.stream_rate << 20) // 2
        x = torch.ones(n, dtype=torch.bfloat16, device=dev)
        y = torch.empty_like(x)
        rates = {}
        for name, fn in (("add", lambda: torch.add(x, 1.0, out=y)),
                         ("copy", lambda: y.copy_(x))):
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            sec = e0.elapsed_time(e1) * 1e-3 / args.steps
            rates[f"{name}_TBps"] = round(2 * 2 * n / sec / 1e12, 3)
        print(json.dumps({"stream_rate_bytes_read": 2 * n,
                          "stream_rate_bytes_written": 2 * n,
                          "launches": args.steps, **rates}), flush=True)
        return 0
    K.load_library()
    cfg = workloads()[args.workload]
    if args.n:
        if args.workload.startswith("decode"):
            print("--n applies to prefill workloads only", file=sys.stderr)
            return 2
        cfg = cfg.replace(n=args.n,
                          name=re.sub(r"n\d+", f"n{args.n}", cfg.name, count=1))
    is_decode = args.workload.startswith("decode")
    is_bwd = args.workload.startswith("backward")
    leg = (decode_leg if is_decode else backward_leg if is_bwd
           else prefill_leg)(torch, K, I, cfg, args, dev)
    ms = leg["ms"]
    kern = leg["kern"]
    achieved = kern["bytes"] / (kern["ms"] * 1e-3) / 1e9
    if is_decode or cfg.dtype != torch.bfloat16:
        dtype = "f32"
    else:
        dtype = "bf16"
    line = {
        "metric": METRIC if not (is_decode or is_bwd) else
                  "linear-attn decode step head-tokens/s (S·H/s) + % of "
                  "HBM roofline" if is_decode else
                  "causal linear-attn backward tokens/s (B·H·n/s) + % of "
                  "HBM roofline",
        "value": leg["items"] / (ms * 1e-3),
        "unit": leg["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": leg["config"],
        "roofline": {"bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": load_traffic(args.workload),
                     "kernel": kern["kernel"],
                     "kernel_ms_per_launch": kern["ms"],
                     "algorithmic_bytes_per_launch": kern["bytes"],
                     "algorithmic_flops_per_launch": kern["flops"],
                     "algorithmic_TFLOPs":
                         kern["flops"] / (kern["ms"] * 1e-3) / 1e12,
                     "mfma_frac_algorithmic":
                         kern["flops"] / (kern["ms"] * 1e-3) / 1e12
                         / BF16_PEAK_TFLOPS},
        "step_algorithmic_GBs": leg["bytes"] / (ms * 1e-3) / 1e9,
        "settle": {"ms": args.settle_ms, "untimed_steps": leg["settle_steps"]},
        "wall_s_timed_region": leg["t_wall"],
    }
    if "other_launches_ms" in kern:
        line["roofline"]["launches_ms"] = kern["other_launches_ms"]
    if not args.no_cpu_baseline:
        if is_decode:
            line["cpu_baseline"] = cpu_baseline_decode(
                cfg, args.seed, channel=args.workload == "decode_channel")
        else:
            line["cpu_baseline"] = (
                cpu_baseline_backward(cfg, args.seed) if is_bwd else
                cpu_baseline_prefill(cfg, args.seed,
                                     channel=args.workload == "channel"))
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
