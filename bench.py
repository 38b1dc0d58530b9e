#!/usr/bin/env python3
"""Benchmark of the action-expert denoise loop on one MI355X.

One "step" is one full denoise call: 10 flow-matching Euler steps of the
pi0.5-shaped expert (18 layers, width 1024, 8 query heads + 1 KV head of
dim 256, GeGLU 4096, 50 action tokens of dim 32, state 32, prefix KV of 560
tokens, bf16 weights and activations) at batch 1, on synthetic seeded
inputs already resident in HBM. Prints one JSON line.

Roofline: the path streams every per-step GEMM weight plus the prefix KV from
HBM once per Euler step (the modulation parameters are folded into a
create-time table and are not counted); achieved GB/s = those algorithmic
bytes per launch / the measured launch time, against 8 TB/s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
# dense MFMA peaks (TFLOP/s) of the type each weight format's GEMMs multiply in
MFMA_PEAK_TFLOPS = {"fp32": 157.3, "bf16": 2500.0, "fp8": 5000.0, "w4a16": 2500.0, "w8a16": 2500.0, "w4a8": 5000.0}
from vla_flow_matching_pi0_amd.profsum import source_digest as kernel_source_digest  # noqa: E402


def measured_traffic(workload: str, mode: str):
    """HBM bytes per launch of the timed kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain streaming kernel of
    known size), or None when there is none for this code and workload."""
    kernel = {"persistent": "k_persistent", "stream": "k_stream"}.get(mode)
    if kernel is None:
        return None
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.startswith("- `"):
                k, v = line[3:].split("`", 1)[0], line.split(":", 1)[1].strip().strip("`")
                vals[k] = v
    if vals.get("kernel_source_sha256") != kernel_source_digest(kernel):
        return None
    try:
        return int(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_bytes_per_step(cfg) -> int:
    """Bytes the method must read from HBM per Euler step: the per-step GEMM
    weights (q/k/v/o/gate/up/down of every layer, in/out projections) plus
    every layer's prefix K and V. The state projection is applied once per
    call (algorithmic_bytes_per_launch)."""
    W, F, d, L = cfg.width, cfg.mlp_dim, cfg.head_dim, cfg.num_layers
    qkv = W * (cfg.num_q_heads + 2 * cfg.num_kv_heads) * d
    o = cfg.num_q_heads * d * W
    per_layer = qkv + o + 2 * W * F + F * W
    small = cfg.action_dim * W + W * cfg.action_dim
    if getattr(cfg, "variant", "pi05") == "pi0":
        small += W * W              # pi0: the time-MLP output GEMM of every step
    prefix = 2 * L * cfg.batch * cfg.prefix_len * cfg.num_kv_heads * d
    act_b = 4 if cfg.weight_precision == "fp32" else 2
    if cfg.weight_precision == "fp8":
        gemm = L * per_layer                                  # one byte per weight
    elif cfg.weight_precision in ("w4a16", "w4a8"):
        gemm = L * per_layer // 2 + L * per_layer // cfg.w4_group * 2   # nibbles + fp16 group scales
    elif cfg.weight_precision == "w8a16":
        cols = (cfg.num_q_heads + 2 * cfg.num_kv_heads) * d + W + 2 * F + W
        gemm = L * per_layer + L * cols * 4                            # int8 codes + fp32 column scales
    else:
        gemm = L * per_layer * act_b
    return gemm + small * act_b + prefix * act_b


def algorithmic_bytes_per_launch(cfg) -> int:
    """One call: num_steps Euler steps plus the state projection, read once."""
    act_b = 4 if cfg.weight_precision == "fp32" else 2
    return algorithmic_bytes_per_step(cfg) * cfg.num_steps + cfg.state_dim * cfg.width * act_b


def resolved_mode(cfg, mode: str) -> str:
    """The launch the library takes for `mode` (its 'auto' rule: graph launch
    for bf16 weights and at least 256 rows, else the persistent kernel)."""
    if mode != "auto":
        return mode
    T = cfg.action_horizon + (1 if getattr(cfg, "variant", "pi05") == "pi0" else 0)
    return "graph" if cfg.weight_precision == "bf16" and cfg.batch * T >= 256 else "persistent"


def roofline_bound(cfg) -> str:
    """'hbm' or 'mfma': whichever of the weight stream and the arithmetic
    (dense MFMA peak of the type the GEMMs multiply in) takes longer at peak."""
    t_hbm = algorithmic_bytes_per_launch(cfg) / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops_per_chunk(cfg) / (MFMA_PEAK_TFLOPS[cfg.weight_precision] * 1e12)
    return "mfma" if t_mfma > t_hbm else "hbm"


def flops_per_chunk(cfg) -> float:
    """Multiply-adds x 2 of the GEMMs and attention of one chunk (pi0: one
    state token more per sample, plus the time-MLP output GEMM)."""
    pi0 = getattr(cfg, "variant", "pi05") == "pi0"
    T = cfg.action_horizon + (1 if pi0 else 0)
    M = cfg.batch * T
    W, F, d, L = cfg.width, cfg.mlp_dim, cfg.head_dim, cfg.num_layers
    qkv = W * (cfg.num_q_heads + 2 * cfg.num_kv_heads) * d
    gemm = M * (L * (qkv + cfg.num_q_heads * d * W + 3 * W * F) + 2 * cfg.action_dim * W + (W * W if pi0 else 0))
    attn = L * cfg.batch * cfg.num_q_heads * T * (cfg.prefix_len + T) * d * 2
    return 2.0 * (gemm + attn) * cfg.num_steps


def prefix_flops(cfg) -> float:
    """Multiply-adds x 2 of one prefix pass: every layer's fused QKV, o,
    gate/up and down GEMMs and bidirectional attention over its P tokens; the
    last layer only projects its keys and values."""
    M = cfg.batch * cfg.prefix_len
    W, F, d, L = cfg.width, cfg.mlp_dim, cfg.head_dim, cfg.num_layers
    qd, kd = cfg.num_q_heads * d, cfg.num_kv_heads * d
    layer = M * (W * (qd + 2 * kd) + qd * W + 3 * W * F) + 2 * cfg.batch * cfg.num_q_heads * cfg.prefix_len ** 2 * d
    return 2.0 * ((L - 1) * layer + M * W * 2 * kd)


def bench_prefix(name: str, reps: int, stream, expert=None, expert_bufs=None):
    """Time the prefix producer on random-init weights of the workload's shape
    (N(0, 0.02^2) bf16, drawn on the device) and N(0, 1) embeddings; with an
    expert of matching shape, also the observation-to-actions chain (prefix
    pass writing the expert's bound K/V buffers, then one denoise call)."""
    import torch
    from synth import PREFIX_CONFIGS, prefix_param_specs
    from vla_flow_matching_pi0_amd import vfm
    cfg = PREFIX_CONFIGS[name]
    gen = torch.Generator(device="cuda").manual_seed(cfg.seed)
    w = {n: (torch.randn(s, generator=gen, device="cuda") * cfg.weight_std).to(torch.bfloat16)
         for n, s in prefix_param_specs(cfg)}
    pre = vfm.PrefixProducer(cfg, w)
    del w
    emb = torch.randn((cfg.batch, cfg.prefix_len, cfg.width), generator=gen, device="cuda").to(torch.bfloat16)
    shape = (cfg.num_layers, cfg.batch, cfg.prefix_len, cfg.num_kv_heads, cfg.head_dim)
    chain = expert is not None and tuple(expert_bufs["prefix_k"].shape) == shape
    pk = expert_bufs["prefix_k"] if chain else torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    pv = expert_bufs["prefix_v"] if chain else torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        pre.run(emb, pk, pv, stream)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        pre.run(emb, pk, pv, stream)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    fl = prefix_flops(cfg)
    tf = fl / (ms * 1e-3) / 1e12
    out = {"workload": cfg.name, "ms_per_pass": round(ms, 4), "flop_per_pass": fl,
           "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4)}}
    if chain:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(reps):
            pre.run(emb, pk, pv, stream)
            expert.denoise(stream=stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        expert.check(stream)
        out["chain_ms"] = round(ev[0].elapsed_time(ev[1]) / reps, 4)
        out["plan"] = bench_plan(pre, emb, pk, pv, expert, stream, ticks=max(5, reps // 5 * 5))
    pre.close()
    return out


def bench_plan(pre, emb, pk, pv, expert, stream, ticks: int, every: int = 5):
    """A control loop as a plan: the prefix stage refreshes the K/V every
    `every` ticks, the expert denoises on every tick (selective refresh).
    Mean ms per tick over `ticks` ticks, against the same sequence of calls
    issued directly on one stream."""
    import torch
    from vla_flow_matching_pi0_amd import vfm
    plan = vfm.Plan()
    plan.add_prefix(pre, emb, pk, pv, every=every)
    plan.add_denoise(expert)
    for t in range(every):
        plan.run(t, stream)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record(stream)
    for t in range(ticks):
        plan.run(t, stream)
    ev[1].record(stream)
    ev[2].record(stream)
    for t in range(ticks):
        if t % every == 0:
            pre.run(emb, pk, pv, stream)
        expert.denoise(stream=stream)
    ev[3].record(stream)
    torch.cuda.synchronize()
    expert.check(stream)
    plan.close()
    return {"prefix_every": every, "ticks": ticks, "ms_per_tick": round(ev[0].elapsed_time(ev[1]) / ticks, 4),
            "direct_ms_per_tick": round(ev[2].elapsed_time(ev[3]) / ticks, 4)}


def cpu_baseline(cfg, params, pk, pv, noise, state, steps: int, min_seconds: float = 10.0):
    """The oracle, untuned, timed on the host cores on a bounded sample:
    `steps` Euler steps of the same chunk, repeated until `min_seconds` have
    passed, scaled to the full chunk."""
    from oracle import denoise as O
    from oracle import pi0 as P0
    run = P0.denoise_pi0 if getattr(cfg, "variant", "pi05") == "pi0" else O.denoise
    from threadpoolctl import threadpool_info, threadpool_limits
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    affinity = len(os.sched_getaffinity(0))
    p64 = O.to_f64(params)

    def leg(seconds: float):
        reps, dt = 0, 0.0
        while dt < seconds:
            t0 = time.perf_counter()
            run(p64, noise, state, pk, pv, cfg, num_steps=steps)
            dt += time.perf_counter() - t0
            reps += 1
        return dt * 1e3 * cfg.num_steps / (steps * reps), reps, dt

    per_chunk_ms, reps, dt = leg(min_seconds)
    with threadpool_limits(limits=1):
        one_ms, one_reps, one_dt = leg(min_seconds)
    return {"value": round(per_chunk_ms, 1), "unit": "ms/chunk", "cores": int(blas), "kind": "oracle",
            "sample": f"{reps} x {steps} of {cfg.num_steps} Euler steps of the {cfg.name} chunk (float64 numpy, "
                      f"BLAS on {blas} threads), scaled to {cfg.num_steps} steps; {dt:.1f} s measured",
            "affinity_cores": affinity, "blas_threads": int(blas),
            "single_thread": {"value": round(one_ms, 1), "unit": "ms/chunk", "cores": 1,
                              "sample": f"{one_reps} x {steps} Euler steps with BLAS limited to one thread, "
                                        f"{one_dt:.1f} s measured"}}


def phase_breakdown(t, nb, N, L, fused, pi0, merged=True):
    """Mean (work, wait) in microseconds of each phase of a middle layer, from
    workgroup 0's (arrive, release) stamps: work runs from the previous
    release to this arrival, wait from arrival to release."""
    if pi0 or L < 3:
        return None
    names = (["qkv_attn", "o", "gu", "down"] if fused
             else ["rn_attn", "qkv_attn", "o", "rn_mlp", "gu", "down"] if merged
             else ["rn_attn", "qkv", "attn", "combine", "o", "rn_mlp", "gu", "down"])
    per_step = len(names) * L + 1 if fused else len(names) * L
    # barrier index i ends the phase that ran before it; the first layer-l
    # phase of step k (k >= 0) follows barrier 1 + k * per_step + (l * len(names) - (0 if fused else 1))
    out = {n: [0.0, 0.0] for n in names}
    cnt = 0
    for k in range(N):
        for l in range(1, L - 1):
            base = 1 + k * per_step + l * len(names) - (0 if fused else 1)
            for j, n in enumerate(names):
                i = base + j
                if i + 1 > nb:
                    continue
                out[n][0] += t[i + 1, 0] - t[i, 1]
                out[n][1] += t[i + 1, 1] - t[i + 1, 0]
            cnt += 1
    return {n: [round(a / cnt, 2), round(b / cnt, 2)] for n, (a, b) in out.items()} if cnt else None


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed denoise calls (chunks)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="pi05_bf16_b1")
    ap.add_argument("--mode", default="persistent", choices=["persistent", "graph", "eager", "auto", "stream"],
                    help="launch mode; 'auto' is the library default (graph launch of the large-batch kernels for "
                         "bf16 experts with at least 256 rows, else the persistent kernel); 'stream' is the "
                         "batch-1 kernel whose weights stream into LDS ahead of use (bf16 pi0.5 shapes)")
    ap.add_argument("--large-m-tiles", default="auto", choices=["auto", "narrow", "wide"],
                    help="graph / eager launch with many rows: the large-M GEMM tile plan")
    ap.add_argument("--persistent-launch", default="cooperative", choices=["cooperative", "plain"],
                    help="launch API of the persistent kernel (plain: for profilers that cannot follow "
                         "cooperative launches)")
    ap.add_argument("--cpu-steps", type=int, default=10, help="Euler steps of the oracle CPU sample (0: skip)")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="between timed calls, stream this many MiB through the caches (cold-cache timing: "
                         "the weights of a quantised expert otherwise stay in the 256 MB last-level cache); "
                         "value is then the mean per-call time")
    ap.add_argument("--prefix", default="prefix_gemma2b_p560",
                    help="prefix-producer workload timed after the expert ('none': skip)")
    ap.add_argument("--prefix-reps", type=int, default=20)
    ap.add_argument("--calib-mib", type=int, default=0,
                    help="after the timed region, run a plain streaming kernel (negation) over this many MiB "
                         "of float32, the reference for scaling HBM counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the denoise loop at batch 1 is "
              "not sharded; a batch would split across GPUs by samples with no communication.", file=sys.stderr)
        return 2

    import torch
    from synth import CONFIGS, make_calibration_inputs, make_inputs
    from vla_flow_matching_pi0_amd import vfm

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1
    cfg = CONFIGS[args.workload]
    print(f"[bench] workload {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    params, pk, pv, noise, state = make_inputs(cfg)
    wdt = torch.float32 if cfg.weight_precision == "fp32" else torch.bfloat16   # masters / activations
    dev = {k: torch.from_numpy(v).to("cuda").to(wdt) for k, v in params.items()}
    ex = vfm.Expert(cfg, dev)
    del dev
    ex.set_option("launch_mode", args.mode)
    ex.set_option("persistent_launch", args.persistent_launch)
    ex.set_option("large_m_tiles", args.large_m_tiles)
    bufs = {"prefix_k": torch.from_numpy(pk).to("cuda").to(wdt), "prefix_v": torch.from_numpy(pv).to("cuda").to(wdt),
            "noise": torch.from_numpy(noise).to("cuda"), "actions": torch.empty(noise.shape, device="cuda")}
    if cfg.state_dim:
        bufs["state"] = torch.from_numpy(state).to("cuda")
    stream = torch.cuda.current_stream()
    if cfg.weight_precision in ("fp8", "w4a8"):
        # activation scales from one calibration pass over a separate draw
        cpk, cpv, cnoise, cstate = make_calibration_inputs(cfg)
        cal = {"prefix_k": torch.from_numpy(cpk).to("cuda").to(wdt), "prefix_v": torch.from_numpy(cpv).to("cuda").to(wdt),
               "noise": torch.from_numpy(cnoise).to("cuda"), "actions": torch.empty(cnoise.shape, device="cuda")}
        if cfg.state_dim:
            cal["state"] = torch.from_numpy(cstate).to("cuda")
        for k, v in cal.items():
            ex.bind(k, v)
        print("[bench] FP8 calibration pass", file=sys.stderr, flush=True)
        ex.calibrate(stream)
    for k, v in bufs.items():
        ex.bind(k, v)
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        ex.denoise(stream=stream)
    ex.check(stream)
    torch.cuda.synchronize()

    # timed region: HIP events on the launch stream around the whole run of
    # back-to-back calls (a timing event recorded between two calls costs
    # about 5 us of idle device time itself); with --flush-mib every call is
    # bracketed instead, so that the flush kernel between calls stays out
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    flush = None
    if args.flush_mib > 0:
        flush = torch.ones(args.flush_mib * (1 << 20) // 4, device="cuda")

    def bracketed(n):
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(n):
            starts[i].record(stream)
            ex.denoise(stream=stream)
            ends[i].record(stream)
            if flush is not None:
                flush.neg_()
        torch.cuda.synchronize()
        ex.check(stream)
        return np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])

    if flush is not None:
        per = bracketed(args.steps)
        total_ms = float(np.sum(per))
    else:
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(args.steps):
            ex.denoise(stream=stream)
        t1.record(stream)
        torch.cuda.synchronize()
        ex.check(stream)
        total_ms = t0.elapsed_time(t1)
        # the per-call distribution from a separate, shorter bracketed run
        per = bracketed(min(args.steps, 50))
    med = float(np.median(per))
    mean = float(np.mean(per))
    ms_chunk = mean if flush is not None else total_ms / args.steps
    del flush

    # in-kernel synchronisation: one more (untimed) call with the phase timeline on; the share of the call that
    # workgroup 0 spends between arriving at a device-wide barrier and its release
    sync = None
    if args.mode == "persistent":
        L, N = cfg.num_layers, cfg.num_steps
        plan = ex.persistent_plan()
        ex.set_option("trace", "1")
        ex.denoise(stream=stream)
        ex.check(stream)
        pi0 = 1 if cfg.variant == "pi0" else 0   # pi0: the time-MLP GEMM and layer 0's norm add 2 per step
        t = ex.export("trace", (2 * (N * (8 * L + 1 + 2 * pi0) + 4),)).reshape(-1, 2).astype(np.float64)
        ex.set_option("trace", "0")
        nb = plan["barriers"]
        span = t[nb, 1] - t[0, 1]
        stall = float(np.sum(t[1:nb + 1, 1] - t[1:nb + 1, 0]))
        sync = {"barriers_per_call": nb, "fused_norms": plan["fused_norms"], "stall_us": round(stall, 1),
                "span_us": round(float(span), 1), "stall_frac": round(stall / span, 4) if span > 0 else None,
                "per_layer_us": phase_breakdown(t, nb, N, L, plan["fused_norms"], pi0, plan["attn_merge"])}
    elif args.mode == "stream":
        # (arrive, counters complete, workgroup ready) per barrier: the stall is
        # arrival to ready (the device-wide wait plus any wait for weights)
        L, N = cfg.num_layers, cfg.num_steps
        nb = N * (5 * L + 2) - 1
        words = max(2 * (N * (8 * L + 1) + 4), 3 * (nb + 2))
        ex.set_option("trace", "1")
        ex.denoise(stream=stream)
        ex.check(stream)
        t = ex.export("trace", (words,))[: 3 * (nb + 1)].reshape(-1, 3).astype(np.float64)
        ex.set_option("trace", "0")
        span = t[nb, 2] - t[0, 2]
        stall = float(np.sum(t[1:, 2] - t[1:, 0]))
        weight_wait = float(np.sum(t[1:, 2] - t[1:, 1]))
        sync = {"barriers_per_call": nb, "stall_us": round(stall, 1), "weight_wait_us": round(weight_wait, 1),
                "span_us": round(float(span), 1), "stall_frac": round(stall / span, 4) if span > 0 else None}
    # execution-state capsule of the bound buffers: snapshot and restore, each a set of device-to-device copies
    cap = ex.capsule()
    reps = 20
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record(stream)
    for _ in range(reps):
        cap.save(ex, stream)
    ev[1].record(stream)
    for _ in range(reps):
        cap.restore(ex, stream)
    ev[2].record(stream)
    torch.cuda.synchronize()
    save_us = ev[0].elapsed_time(ev[1]) * 1e3 / reps
    restore_us = ev[1].elapsed_time(ev[2]) * 1e3 / reps
    capsule = {"bytes": cap.nbytes, "save_us": round(save_us, 2), "restore_us": round(restore_us, 2),
               "restore_GBps": round(2 * cap.nbytes / (restore_us * 1e3), 1)}
    cap.close()
    prefix = None
    if args.prefix != "none":
        print(f"[bench] prefix producer {args.prefix}", file=sys.stderr, flush=True)
        prefix = bench_prefix(args.prefix, args.prefix_reps, stream, ex, bufs)
    if args.calib_mib > 0:
        n = args.calib_mib * (1 << 20) // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        # the same bytes copied with plain and with device-scope (sc1) loads,
        # to check the counter scale on the load policy the kernels also use
        for policy in (0, 16):
            for _ in range(3):
                vfm.copy_probe(src, dst, policy, stream)
        torch.cuda.synchronize()
        del src, dst

    bytes_launch = algorithmic_bytes_per_launch(cfg)
    achieved = bytes_launch / (mean * 1e-3) / 1e9
    tflops = flops_per_chunk(cfg) / (mean * 1e-3) / 1e12
    mfma_peak = MFMA_PEAK_TFLOPS[cfg.weight_precision]
    t_hbm = bytes_launch / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops_per_chunk(cfg) / (mfma_peak * 1e12)
    if roofline_bound(cfg) == "mfma":
        roofline = {"bound": "mfma", "achieved": round(tflops, 1), "peak": mfma_peak, "unit": "TFLOP/s",
                    "frac": round(tflops / mfma_peak, 4), "traffic": None}
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(cfg.name, args.mode)}
    cpu = None
    if args.cpu_steps > 0:
        print(f"[bench] oracle CPU sample ({args.cpu_steps} steps)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, params, pk, pv, noise, state, args.cpu_steps)
    line = {
        "metric": "ms per 10-step action chunk @ batch 1; % of HBM weight-stream roofline",
        "value": round(ms_chunk, 4),
        "unit": "ms/chunk",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_chunk, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp32": "f32", "bf16": "bf16", "fp8": "fp8e4m3", "w4a16": "int4/bf16",
                  "w8a16": "int8/bf16", "w4a8": "int4/fp8e4m3"}[cfg.weight_precision],
        "data": "synthetic",
        "config": {"workload": cfg.name, "layers": cfg.num_layers, "width": cfg.width, "heads": f"{cfg.num_q_heads}q/{cfg.num_kv_heads}kv",
                   "head_dim": cfg.head_dim, "mlp": cfg.mlp_dim, "horizon": cfg.action_horizon,
                   "action_dim": cfg.action_dim, "state_dim": cfg.state_dim, "prefix": cfg.prefix_len,
                   "batch": cfg.batch, "euler_steps": cfg.num_steps, "launch_mode": resolved_mode(cfg, args.mode),
                   "persistent_launch": args.persistent_launch},
        "chunks_per_s": round(cfg.batch * 1e3 / ms_chunk, 2),
        "ms_per_launch_mean": round(mean, 4),
        "ms_per_chunk_median": round(med, 4),
        "ms_per_chunk_p99": round(float(np.percentile(per, 99)), 4),
        "roofline_ms_per_chunk": round(max(t_hbm, t_mfma) * 1e3, 4),
        "algorithmic_bytes_per_launch": int(bytes_launch),
        "achieved_tflops": round(tflops, 2),
        "sync": sync,
        "capsule": capsule,
        "prefix_producer": prefix,
        "flush_mib": args.flush_mib,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    ex.close()
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
