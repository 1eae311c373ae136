#!/usr/bin/env python3
"""Throughput of the quantized MoE expert path on one MI355X.

Metric: expert-path tokens/s and achieved HBM GB/s on quantized expert
weight bytes (fraction of the 8 TB/s peak), hidden 4096, 512 experts.

Default workload (stack60_decode): one decode token through 60 resident
MoE layers (60 x 513 experts of hidden 4096, intermediate 1024, 4-bit
group-64 affine, top-3 + 1 shared, unit-weight RMS norm between layers) --
a step is one token through all 60 layers, one persistent launch.  The
whole 218 GB expert set is resident in HBM before timing; every step's
expert bytes come from HBM (the set is far larger than the caches).

Other workloads (--workload): decode_4bit, decode_2bit, batch16_top10 --
one layer per step, rotating over --instances resident layer instances so
every expert byte is read from HBM; stack60_prefill -- 2048 tokens through
the same 60 resident layers per step (top-10 + shared, grouped
dequant-GEMMs on MFMA).

Inputs are seeded synthetic data (SplitMix64 streams); no trained weights
or prompts.  Prints ONE JSON line on stdout; progress goes to stderr.
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
METRIC = "expert-path tokens/sec & achieved HBM GB/s (% of peak), hidden 4096 E=512"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=64)
    p.add_argument("--warmup", type=int, default=8)
    p.add_argument("--workload", default="stack60_decode",
                   choices=["stack60_decode", "decode_4bit", "decode_2bit", "batch16_top10", "stack60_prefill"])
    p.add_argument("--layerwise", action="store_true",
                   help="stack60_decode: per-layer launches instead of the persistent kernel")
    p.add_argument("--instances", type=int, default=8, help="layer instances for cold rotation")
    p.add_argument("--tokens-pool", type=int, default=64, help="distinct token vectors")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample budget")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB (counter calibration)")
    return p.parse_args()


def expert_gate_up_bytes(cfg) -> int:
    q = cfg.hidden * cfg.inter * cfg.bits // 8
    sb = cfg.hidden * cfg.inter // cfg.group * 4
    return 2 * (q + sb)


def cores():
    return len(os.sched_getaffinity(0))


# ------------------------------------------------------------ CPU baseline

def cpu_baseline_layer(cfg, seconds: float):
    """The fp64 oracle, as it stands, on a bounded sample of one layer."""
    import oracle
    import synth

    n = cores()
    T = max(1, n)                         # the oracle threads over tokens
    x = synth.bf16_to_f64(synth.tokens(synth.with_changes(cfg, tokens=T), 1000, T))
    cache = {}
    oracle.run_layer(cfg, 0, x, want_intermediates=False, blob_cache=cache)   # generate blobs once
    done, busy = 0, 0.0
    while busy < seconds:
        t0 = time.perf_counter()
        oracle.run_layer(cfg, 0, x, want_intermediates=False, blob_cache=cache)
        busy += time.perf_counter() - t0
        done += T
    return dict(value=round(done / busy, 3), unit="tokens/s", cores=min(T, n), kind="oracle",
                sample=f"{done} tokens through one {cfg.name} layer in batches of {T} "
                       f"({busy:.1f} s of oracle time; expert blobs generated beforehand)")


def cpu_baseline_stack(cfg, seconds: float):
    """The fp64 oracle on a bounded sample of the 60-layer decode: a batch of
    tokens (one per host core) through as many layers as the budget allows;
    tokens/s is scaled to 60 layers from the measured per-token-layer time."""
    import oracle
    import synth

    n = cores()
    T = max(1, n)
    h = synth.bf16_to_f64(synth.tokens(synth.with_changes(cfg, tokens=T), 2000, T))
    shape = oracle.shape_of(cfg)
    busy, layers = 0.0, 0
    for l in range(cfg.layers):
        wr = synth.router(cfg, l)
        _, idx, _, _ = oracle.route(shape, wr, h, cfg.top_k, oracle.layer_flags(cfg))
        need = set(int(e) for e in np.unique(idx)) | set(range(cfg.n_experts, cfg.n_slots))
        blobs = {e: synth.expert_blob(cfg, l, e) for e in need}
        t0 = time.perf_counter()
        out = oracle.moe_layer(shape, blobs, wr, h, cfg.top_k, oracle.layer_flags(cfg),
                               want_intermediates=False)
        busy += time.perf_counter() - t0
        h = out["y"]
        layers += 1
        if busy >= seconds:
            break
    per_token_layer = busy / (layers * T)
    return dict(value=round(1.0 / (per_token_layer * cfg.layers), 4), unit="tokens/s",
                cores=min(T, n), kind="oracle",
                sample=f"{T} tokens through {layers} of {cfg.layers} layers ({busy:.1f} s of oracle "
                       f"time, blob generation excluded); tokens/s = 1 / (60 x measured "
                       f"per-token-layer time)")


# -------------------------------------------------------------- workloads

def recorded_stack_traffic():
    """HBM bytes per launch of the persistent stack kernel from the committed
    rocprofv3 counter summary, or None when the kernel's sources changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "stack_kernel_stack60_decode_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in ("stack_decode.hip", "moeq_device.hpp", "topk.hpp", "moeq_internal.hpp"):
        with open(os.path.join(ROOT, "quantized_expert_gemv_router_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if rec.get("source_sha256_16") != h.hexdigest()[:16] or "traffic_bytes_per_launch" not in rec:
        return None
    return int(rec["traffic_bytes_per_launch"])


def setup_layers(cfg, n_layers, dev, stream):
    import torch
    import quantized_expert_gemv_router_amd as q
    import synth

    shape = q.Shape.of(cfg)
    stride = (cfg.expert_bytes + 255) // 256 * 256
    log(f"[bench] {cfg.name}: filling {n_layers} layers x {cfg.n_slots} experts "
        f"({n_layers * cfg.n_slots * stride / 1e9:.1f} GB) in HBM")
    arenas = []
    for l in range(n_layers):
        a = torch.empty(cfg.n_slots * stride, dtype=torch.uint8, device=dev)
        synth.device_fill_experts(cfg, l, a.data_ptr(), stride, stream=stream.cuda_stream)
        arenas.append(a)
    table = q.ExpertTable(shape, arenas, stride, device=dev)
    bf16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    routers = [bf16(synth.router(cfg, l)) for l in range(n_layers)]
    torch.cuda.synchronize()
    return shape, table, routers, bf16


def run_stack(args, cfg, dev, stream):
    import torch
    import quantized_expert_gemv_router_amd as q
    import synth

    shape, table, routers, _ = setup_layers(cfg, cfg.layers, dev, stream)
    rt = q.RouterTable(routers, device=dev)
    K = cfg.top_k
    pool = torch.from_numpy(np.stack([synth.bf16_to_f64(synth.tokens(cfg, 100 + i, 1)).astype(np.float32)
                                      for i in range(args.tokens_pool)])).to(dev)
    total = args.warmup + args.steps
    hs = [pool[s % args.tokens_pool].clone() for s in range(total)]
    tks = torch.empty((total, cfg.layers, 1, K), dtype=torch.int32, device=dev)
    ws = q.new_workspace(shape, 1, K, dev)
    flags = q.F_STACK_LAYERWISE if args.layerwise else 0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()

    def step(s, slot=None):
        if slot is not None:
            ev[slot][0].record(stream)
        import ctypes
        rc = q.lib().moe_expert_stack_decode(ctypes.byref(shape), table.view(), rt.ptr(), 0, cfg.layers,
                                             1, K, flags, hs[s].data_ptr(), tks[s].data_ptr(), None,
                                             ws.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(q.moeq_last_error())
        if slot is not None:
            ev[slot][1].record(stream)

    with torch.cuda.stream(stream):
        for s in range(args.warmup):
            step(s)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(stream)
        for i in range(args.steps):
            step(args.warmup + i, slot=i)
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    status = q.moe_read_device_status(ws, stream)
    if status != 0:
        raise RuntimeError(f"device status {status} after the timed region")
    elapsed_ms = start.elapsed_time(end)
    launch_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    idx = tks[args.warmup:].cpu().numpy()
    distinct = np.array([[len(np.unique(idx[s, l])) for l in range(cfg.layers)]
                         for s in range(args.steps)]) + cfg.n_shared
    expert_bytes = distinct.sum(axis=1) * cfg.expert_bytes          # per step
    router_bytes = cfg.layers * cfg.n_experts * cfg.hidden * 2
    per_launch = float(expert_bytes.mean())
    sec = elapsed_ms / 1e3
    rec = base_record(args, cfg, steps_tokens=args.steps, elapsed_ms=elapsed_ms, wall=wall)
    rec.update({
        "gbps_expert": round(expert_bytes.sum() / sec / 1e9, 1),
        "gbps_all_bytes": round((expert_bytes.sum() + args.steps * router_bytes) / sec / 1e9, 1),
        "frac_hbm_peak": round(expert_bytes.sum() / sec / 1e9 / HBM_PEAK_GBS, 4),
        "expert_layers_per_s": round(args.steps * cfg.layers / sec, 1),
        "path": "persistent" if q.moeq_last_stack_path() == 1 else "per-layer",
        "roofline": {"kernel": "stack_kernel (persistent 60-layer decode, one launch per token)"
                     if q.moeq_last_stack_path() == 1 else "per-layer launches (3 per layer)",
                     "bound": "hbm", "achieved": round(per_launch / (launch_ms / 1e3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(per_launch / (launch_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": recorded_stack_traffic() if q.moeq_last_stack_path() == 1 else None,
                     "avg_launch_us": round(launch_ms * 1e3, 2),
                     "bytes_per_launch": int(per_launch),
                     "router_bytes_per_launch": router_bytes},
    })
    rec["config"].update(layers_per_step=cfg.layers, resident_gb=round(
        cfg.layers * cfg.n_slots * cfg.expert_bytes / 1e9, 1))
    return rec


def run_prefill(args, cfg, dev, stream):
    """T-token prefill through all resident layers per step (grouped
    dequant-GEMMs on MFMA); per-kernel times from HIP events on the stream."""
    import torch
    import quantized_expert_gemv_router_amd as q
    import synth

    shape, table, routers, _ = setup_layers(cfg, cfg.layers, dev, stream)
    rt = q.RouterTable(routers, device=dev)
    T, K = cfg.tokens, cfg.top_k
    total = args.warmup + args.steps
    sets = [torch.from_numpy(synth.bf16_to_f64(synth.tokens(cfg, 3000 + i, T)).astype(np.float32)).to(dev)
            for i in range(min(total, 4))]
    hs = [sets[s % len(sets)].clone() for s in range(total)]
    ws = q.new_prefill_workspace(shape, T, K, dev)
    tk = torch.empty((cfg.layers, T, K), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    def step(s, trace=None):
        import ctypes
        rc = q.lib().moe_expert_stack_prefill(ctypes.byref(shape), table.view(), rt.ptr(), 0, cfg.layers, T, K,
                                              0, hs[s].data_ptr(), None if trace is None else trace.data_ptr(),
                                              ws.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(q.moeq_last_error())

    with torch.cuda.stream(stream):
        for s in range(args.warmup):
            step(s, tk if s == args.warmup - 1 else None)
        torch.cuda.synchronize()
        q.moeq_prefill_timing(True)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(stream)
        for i in range(args.steps):
            # the routing of the last warm-up step gives the bytes per step; with
            # no warm-up, the first timed step records it (80 KB per layer)
            step(args.warmup + i, tk if (args.warmup == 0 and i == 0) else None)
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    kt = q.moeq_prefill_timing_read()
    q.moeq_prefill_timing(False)
    status = q.moe_read_device_status(ws, stream)
    if status != 0:
        raise RuntimeError(f"device status {status} after the timed region")
    elapsed_ms = start.elapsed_time(end)
    idx = tk.cpu().numpy()
    touched = np.array([np.count_nonzero(np.bincount(idx[l].ravel(), minlength=cfg.n_experts))
                        for l in range(cfg.layers)]) + cfg.n_shared
    expert_bytes = int(touched.sum()) * cfg.expert_bytes          # per step (the warm-up's routing)
    router_bytes = cfg.layers * cfg.n_experts * cfg.hidden * 2
    sec = elapsed_ms / 1e3
    # dominant kernel: the gate/up GEMM (2/3 of the weight bytes)
    gu_ms, gu_n = kt["gate_up"]
    gu_bytes = expert_bytes * 2 // 3 // cfg.layers               # per launch (one layer)
    gu_gbs = gu_bytes / (gu_ms / gu_n / 1e3) / 1e9
    pairs = T * (K + cfg.n_shared)
    gu_flop = 2.0 * pairs * 2 * cfg.inter * cfg.hidden            # per launch
    rec = base_record(args, cfg, steps_tokens=args.steps * T, elapsed_ms=elapsed_ms, wall=wall)
    rec.update({
        "gbps_expert": round(expert_bytes * args.steps / sec / 1e9, 1),
        "gbps_all_bytes": round((expert_bytes + router_bytes) * args.steps / sec / 1e9, 1),
        "frac_hbm_peak": round(expert_bytes * args.steps / sec / 1e9 / HBM_PEAK_GBS, 4),
        "expert_layers_per_s": round(args.steps * T * cfg.layers / sec, 1),
        "kernel_ms_per_layer": {k: round(v[0] / max(v[1], 1), 4) for k, v in kt.items()},
        "roofline": {"kernel": "gemm_kernel<gate/up> (grouped dequant-GEMM, fp16 MFMA)", "bound": "hbm",
                     "achieved": round(gu_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "avg_launch_us": round(gu_ms / gu_n * 1e3, 2), "bytes_per_launch": int(gu_bytes),
                     "mfma_tflops": round(gu_flop / (gu_ms / gu_n / 1e3) / 1e12, 1),
                     "mfma_peak_tflops": 2500.0},
    })
    rec["config"].update(layers_per_step=cfg.layers, experts_touched_per_layer=float(touched.mean()),
                         resident_gb=round(cfg.layers * cfg.n_slots * cfg.expert_bytes / 1e9, 1))
    return rec


def run_layer_workload(args, cfg, dev, stream):
    import torch
    import quantized_expert_gemv_router_amd as q
    import synth

    n_inst = args.instances
    shape, table, routers, bf16 = setup_layers(cfg, n_inst, dev, stream)
    T, K = cfg.tokens, cfg.top_k
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

    def step(s, slot=None):
        l = s % n_inst
        x = pool[s % args.tokens_pool]
        idx = idx_all[s]
        q.moe_router_topk(shape, x, routers[l], K, 0, None, ws, out=(idx, w, sw), stream=stream)
        if slot is not None:
            ev[slot][0].record(stream)
        q.moe_q4_expert_gemv(shape, table, l, x, idx, K, 0, ws, gu, stream=stream)
        if slot is not None:
            ev[slot][1].record(stream)
        q.moe_swiglu_down_combine(shape, table, l, gu, idx, w, sw, x, K, ws, y, stream=stream)

    with torch.cuda.stream(stream):
        for s in range(args.warmup):
            step(s)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(stream)
        for i in range(args.steps):
            step(args.warmup + i, slot=i)
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    elapsed_ms = start.elapsed_time(end)
    gemv_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    idx_np = idx_all[args.warmup:].cpu().numpy()
    distinct = np.array([len(np.unique(i)) for i in idx_np]) + cfg.n_shared
    expert_bytes = distinct * cfg.expert_bytes
    router_bytes = cfg.n_experts * cfg.hidden * 2
    sec = elapsed_ms / 1e3
    gemv_bytes = float(np.mean(distinct)) * expert_gate_up_bytes(cfg)
    rec = base_record(args, cfg, steps_tokens=args.steps * T, elapsed_ms=elapsed_ms, wall=wall)
    rec.update({
        "gbps_expert": round(expert_bytes.sum() / sec / 1e9, 1),
        "gbps_all_bytes": round((expert_bytes.sum() + args.steps * router_bytes) / sec / 1e9, 1),
        "frac_hbm_peak": round(expert_bytes.sum() / sec / 1e9 / HBM_PEAK_GBS, 4),
        "expert_layers_per_s": round(args.steps * T / sec, 1),
        "distinct_experts_per_step": round(float(np.mean(distinct)), 2),
        "roofline": {"kernel": ("gemv_kernel (gate/up dequant GEMV, one token)" if T == 1 else
                                "gemv_batch_kernel (gate/up dequant GEMV, several tokens)"), "bound": "hbm",
                     "achieved": round(gemv_bytes / (gemv_ms / 1e3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gemv_bytes / (gemv_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None, "avg_launch_us": round(gemv_ms * 1e3, 3),
                     "bytes_per_launch": int(gemv_bytes)},
    })
    rec["config"].update(layers_per_step=1, layer_instances=n_inst)
    return rec


def base_record(args, cfg, steps_tokens, elapsed_ms, wall):
    return {
        "metric": METRIC,
        "value": round(steps_tokens / (elapsed_ms / 1e3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed_ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"q{cfg.bits}_affine_bf16sb/f16xf32acc+f64router",
        "data": "synthetic: seeded SplitMix64 expert blobs, bf16 N(0,0.02) routers, N(0,1) tokens",
        "config": {"workload": cfg.name, "hidden": cfg.hidden, "n_experts": cfg.n_experts,
                   "inter": cfg.inter, "top_k": cfg.top_k, "n_shared": cfg.n_shared,
                   "tokens_per_step": cfg.tokens, "bits": cfg.bits, "group": cfg.group},
        "wall_s_timed": round(wall, 4),
    }


def calibrate_copy(mib, dev):
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n, "launches": 5}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(the multi-GPU layout is described, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, dev)
        return
    cfg = synth.CONFIGS[args.workload]
    stream = torch.cuda.Stream(device=dev)
    if cfg.layers > 1 and cfg.tokens > 1:
        rec = run_prefill(args, cfg, dev, stream)
    elif cfg.layers > 1:
        rec = run_stack(args, cfg, dev, stream)
    else:
        rec = run_layer_workload(args, cfg, dev, stream)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle sample")
        rec["cpu_baseline"] = (cpu_baseline_stack if cfg.layers > 1 else cpu_baseline_layer)(
            cfg, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
