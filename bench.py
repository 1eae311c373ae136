#!/usr/bin/env python3
"""Throughput of the quantized MoE expert path on one MI355X.

Metric: expert-path tokens/s and achieved HBM GB/s on quantized expert
weight bytes (fraction of the 8 TB/s peak), hidden 4096, 512 experts.

Workloads (seeded synthetic data; real weights and prompts are not used):
  decode_4bit    one decode layer, top-3 + 1 shared, 4-bit, 1 token/step;
                 a step is one token through one layer instance, rotating
                 over --instances resident layer instances so every
                 expert byte comes from HBM (cold weights)
  decode_2bit    same with 2-bit experts, top-4 + 1 shared
  batch16_top10  16 tokens/step, top-10 + 1 shared, 4-bit, cold rotation

Prints ONE JSON line.  Inputs are resident in HBM before timing starts.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode_4bit",
                   choices=["decode_4bit", "decode_2bit", "batch16_top10"])
    p.add_argument("--instances", type=int, default=8, help="layer instances for cold rotation")
    p.add_argument("--tokens-pool", type=int, default=64, help="distinct token vectors")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample budget")
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args()


def gate_up_bytes(cfg) -> int:
    q = cfg.hidden * cfg.inter * cfg.bits // 8
    sb = cfg.hidden * cfg.inter // cfg.group * 4
    return 2 * (q + sb)


def cpu_baseline(cfg, seconds: float):
    """The fp64 oracle, as it stands, on a bounded sample of the workload."""
    import oracle
    import synth

    ncores = len(os.sched_getaffinity(0))
    T = max(1, ncores)                        # the oracle threads over tokens
    x = synth.bf16_to_f64(synth.tokens(synth.with_changes(cfg, tokens=T), 1000, T))
    cache = {}
    oracle.run_layer(cfg, 0, x[:1], want_intermediates=False, blob_cache=cache)   # warm blob cache
    done, t0 = 0, time.perf_counter()
    while True:
        oracle.run_layer(cfg, 0, x, want_intermediates=False, blob_cache=cache)
        done += T
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return dict(value=done / el, unit="tokens/s", cores=min(T, ncores), kind="oracle",
                sample=f"{done} tokens of one {cfg.name} layer (batches of {T} tokens, "
                       f"{el:.1f} s, expert blobs pre-generated)")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(this build measures the single-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_expert_gemv_router_amd as q
    import synth

    cfg = synth.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    shape = q.Shape.of(cfg)
    stride = (cfg.expert_bytes + 255) // 256 * 256
    T, K = cfg.tokens, cfg.top_k
    n_inst = args.instances
    stream = torch.cuda.Stream(device=dev)

    log(f"[bench] {cfg.name}: filling {n_inst} layer instances "
        f"({n_inst * cfg.n_slots * stride / 1e9:.1f} GB) on device")
    arenas = []
    for l in range(n_inst):
        a = torch.empty(cfg.n_slots * stride, dtype=torch.uint8, device=dev)
        synth.device_fill_experts(cfg, l, a.data_ptr(), stride, stream=stream.cuda_stream)
        arenas.append(a)
    table = q.ExpertTable(shape, arenas, stride, device=dev)
    bf16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    routers = [bf16(synth.router(cfg, l)) for l in range(n_inst)]
    pool = bf16(np.stack([synth.tokens(cfg, 100 + i, T) for i in range(args.tokens_pool)]))
    ws = q.new_workspace(shape, T, K, dev)
    total = args.warmup + args.steps
    idx_all = torch.empty((total, T, K), dtype=torch.int32, device=dev)
    w = torch.empty((T, K), dtype=torch.float32, device=dev)
    sw = torch.empty((T,), dtype=torch.float32, device=dev)
    gu = torch.empty((T, K + cfg.n_shared, 2, cfg.inter), dtype=torch.float32, device=dev)
    y = torch.empty((T, cfg.hidden), dtype=torch.float32, device=dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()

    def step(s, timed_slot=None):
        l = s % n_inst
        x = pool[s % args.tokens_pool]
        idx = idx_all[s]
        q.moe_router_topk(shape, x, routers[l], K, 0, None, ws, out=(idx, w, sw), stream=stream)
        if timed_slot is not None:
            ev[timed_slot][0].record(stream)
        q.moe_q4_expert_gemv(shape, table, l, x, idx, K, 0, ws, gu, stream=stream)
        if timed_slot is not None:
            ev[timed_slot][1].record(stream)
        q.moe_swiglu_down_combine(shape, table, l, gu, idx, w, sw, x, K, ws, y, stream=stream)

    with torch.cuda.stream(stream):
        for s in range(args.warmup):
            step(s)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for i in range(args.steps):
            step(args.warmup + i, timed_slot=i)
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    elapsed_ms = start.elapsed_time(end)
    gemv_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))

    idx_np = idx_all[args.warmup:].cpu().numpy()
    distinct = np.array([len(np.unique(i)) for i in idx_np]) + cfg.n_shared
    expert_bytes_steps = distinct * cfg.expert_bytes
    router_bytes = cfg.n_experts * cfg.hidden * 2
    ms_per_step = elapsed_ms / args.steps
    tokens_per_s = args.steps * T / (elapsed_ms / 1e3)
    gbps_expert = expert_bytes_steps.sum() / (elapsed_ms / 1e3) / 1e9
    gbps_all = (expert_bytes_steps.sum() + args.steps * router_bytes) / (elapsed_ms / 1e3) / 1e9
    gemv_bytes = float(np.mean(distinct)) * gate_up_bytes(cfg)
    achieved = gemv_bytes / (gemv_ms / 1e3) / 1e9

    rec = {
        "metric": "expert-path tokens/sec & achieved HBM GB/s (% of peak), hidden 4096 E=512",
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"q{cfg.bits}_affine/f16xf32acc",
        "data": "synthetic (seeded SplitMix64 weights and tokens, cold layer rotation)",
        "config": {"workload": cfg.name, "hidden": cfg.hidden, "n_experts": cfg.n_experts,
                   "inter": cfg.inter, "top_k": K, "n_shared": cfg.n_shared, "tokens_per_step": T,
                   "bits": cfg.bits, "layers_per_step": 1, "layer_instances": n_inst},
        "gbps_expert": round(gbps_expert, 1),
        "gbps_all_bytes": round(gbps_all, 1),
        "frac_hbm_peak": round(gbps_expert / HBM_PEAK_GBS, 4),
        "expert_layers_per_s": round(tokens_per_s, 2),
        "distinct_experts_per_step": round(float(np.mean(distinct)), 2),
        "wall_s_timed": round(wall, 4),
        "roofline": {"kernel": "gemv_kernel (gate/up dequant GEMV)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "avg_launch_us": round(gemv_ms * 1e3, 3),
                     "bytes_per_launch": int(gemv_bytes)},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle sample")
        rec["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
