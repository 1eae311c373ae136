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
every expert byte is read from HBM; stack60_prefill (_4k, _8k) -- 2048
(4096, 8192) tokens through the same 60 resident layers per step (top-10 +
shared, grouped dequant-GEMMs on MFMA).

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
MFMA_FP16_PEAK_TFLOPS = 2500.0   # dense fp16 matrix-core peak
METRIC = "expert-path tokens/sec & achieved HBM GB/s (% of peak), hidden 4096 E=512"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=64)
    p.add_argument("--warmup", type=int, default=8)
    p.add_argument("--workload", default="stack60_decode",
                   choices=["stack60_decode", "decode_4bit", "decode_2bit", "batch16_top10", "stack60_prefill",
                            "stack60_prefill_4k", "stack60_prefill_8k", "pool_decode", "decode_3bit"])
    p.add_argument("--layerwise", action="store_true",
                   help="stack60_decode: per-layer launches instead of the persistent kernel")
    p.add_argument("--layer-calls", action="store_true",
                   help="one-token layer workloads: the three calls per layer (router, gate/up, down/combine) "
                        "instead of one persistent launch per layer")
    p.add_argument("--eager", action="store_true",
                   help="one-token layer workloads: launch every call from Python instead of replaying "
                        "the steps captured in a HIP graph")
    p.add_argument("--warm", action="store_true",
                   help="one-token and batch layer workloads: the same layer instance and token every step "
                        "(its experts stay in the caches) instead of the cold rotation")
    p.add_argument("--instances", type=int, default=8, help="layer instances for cold rotation")
    p.add_argument("--tokens-pool", type=int, default=64, help="distinct token vectors")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample budget")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--pool-layers", type=int, default=16,
                   help="pool_decode: layers held in pinned host memory (7.08 MB x 513 per layer)")
    p.add_argument("--pool-slots", default="8,20,64,513", help="pool_decode: slots per layer to sweep")
    p.add_argument("--pool-streams", default="1,4", help="pool_decode: copy streams to sweep")
    p.add_argument("--pool-reuse", default="0,0.6,0.9",
                   help="pool_decode: token correlation a (token t+1 = a token t + sqrt(1-a^2) fresh) to sweep, "
                        "with and without prefetch of the previous token's experts")
    p.add_argument("--probe-handoff", action="store_true",
                   help="only run the cross-workgroup hand-off latency probe sweep (diagnostic)")
    p.add_argument("--block-timeline", type=int, default=0, metavar="L",
                   help="only run the per-workgroup clock trace of the persistent decode over L layers "
                        "(diagnostic: hand-off latencies and skew)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB (counter calibration)")
    return p.parse_args()


def expert_gate_up_bytes(cfg) -> int:
    q = cfg.hidden * cfg.inter * cfg.bits // 8
    sb = cfg.hidden * cfg.inter // cfg.group * 4
    return 2 * (q + sb)


def cores():
    return len(os.sched_getaffinity(0))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class OracleThreads:
    """Sets the OpenMP thread count of the oracle library (libgomp is shared,
    so omp_set_num_threads reaches the oracle's parallel loops)."""

    def __init__(self, n):
        import ctypes
        self.n = n
        self.gomp = ctypes.CDLL("libgomp.so.1")

    def __enter__(self):
        self.prev = self.gomp.omp_get_max_threads()
        self.gomp.omp_set_num_threads(self.n)
        return self

    def __exit__(self, *exc):
        self.gomp.omp_set_num_threads(self.prev)


TOL = 2e-3   # max |gpu - oracle| <= TOL * max |oracle|


class ParityError(RuntimeError):
    pass


def topk_matches(idx, ref_idx, ref_logits, rel=2.0 ** -35):
    """The persistent decode's top-K against the oracle's: equal, except that
    a rank may hold another expert whose oracle logit differs from the
    oracle's pick by a nonzero amount at most rel * max|logit| (the kernel
    hands logits over rounded to a 36-bit significand, so such a pair can
    tie there and go to the lower index); exact ties must match exactly."""
    idx, ref_idx = np.asarray(idx), np.asarray(ref_idx)
    if np.array_equal(idx, ref_idx):
        return True
    if len(set(idx.tolist())) != idx.size:
        return False
    tol = rel * np.abs(ref_logits).max()
    for g, o in zip(idx.tolist(), ref_idx.tolist()):
        if g != o and not (0 <= g < ref_logits.size and 0.0 < abs(ref_logits[g] - ref_logits[o]) <= tol):
            return False
    return True


def rel_err(gpu, ref) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(gpu - ref).max() / np.abs(ref).max())


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
    # the same oracle on one thread, one token at a time
    x1 = x[:1]
    done1, busy1 = 0, 0.0
    with OracleThreads(1):
        while busy1 < min(4.0, seconds / 3):
            t0 = time.perf_counter()
            oracle.run_layer(cfg, 0, x1, want_intermediates=False, blob_cache=cache)
            busy1 += time.perf_counter() - t0
            done1 += 1
    return dict(value=round(done / busy, 3), unit="tokens/s", cores=min(T, n), kind="oracle",
                cpu_model=cpu_model(), one_thread_value=round(done1 / busy1, 3),
                sample=f"{done} tokens through one {cfg.name} layer in batches of {T} "
                       f"({busy:.1f} s of oracle time; expert blobs generated beforehand); "
                       f"one_thread_value: {done1} tokens one at a time on 1 thread ({busy1:.1f} s)")


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
    # one thread, one token, first layers of the stack
    h1 = h[:1]
    busy1, layers1 = 0.0, 0
    with OracleThreads(1):
        for l in range(cfg.layers):
            wr = synth.router(cfg, l)
            _, idx, _, _ = oracle.route(shape, wr, h1, cfg.top_k, oracle.layer_flags(cfg))
            need = set(int(e) for e in np.unique(idx)) | set(range(cfg.n_experts, cfg.n_slots))
            blobs = {e: synth.expert_blob(cfg, l, e) for e in need}
            t0 = time.perf_counter()
            out = oracle.moe_layer(shape, blobs, wr, h1, cfg.top_k, oracle.layer_flags(cfg),
                                   want_intermediates=False)
            busy1 += time.perf_counter() - t0
            h1 = out["y"]
            layers1 += 1
            if busy1 >= min(4.0, seconds / 3):
                break
    return dict(value=round(1.0 / (per_token_layer * cfg.layers), 4), unit="tokens/s",
                cores=min(T, n), kind="oracle", cpu_model=cpu_model(),
                one_thread_value=round(1.0 / (busy1 / layers1 * cfg.layers), 4),
                sample=f"{T} tokens through {layers} of {cfg.layers} layers ({busy:.1f} s of oracle "
                       f"time, blob generation excluded); tokens/s = 1 / (60 x measured "
                       f"per-token-layer time); one_thread_value: 1 token through {layers1} layers "
                       f"on 1 thread ({busy1:.1f} s), scaled the same way")


# -------------------------------------------------------------- workloads

def recorded_traffic(profile, sources):
    """HBM bytes per launch of a kernel from its committed rocprofv3 counter
    summary, or None when the kernel's sources changed since the counters
    were taken (the summary records the sha256 of the sources)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "quantized_expert_gemv_router_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if rec.get("source_sha256_16") != h.hexdigest()[:16] or "traffic_bytes_per_launch" not in rec:
        return None
    return int(rec["traffic_bytes_per_launch"])


def recorded_stack_traffic():
    return recorded_traffic("stack_kernel_stack60_decode_traffic.txt",
                            ("stack_decode.hip", "moeq_device.hpp", "topk.hpp", "moeq_internal.hpp"))


def recorded_prefill_traffic():
    """The 2048-token workload's gate/up GEMM (the counters were taken on it)."""
    return recorded_traffic("prefill_gemm_counters_stack60_prefill.txt",
                            ("prefill.hip", "moeq_device.hpp", "moeq_internal.hpp"))


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


def parity_stack(cfg, shape, table, rt, ws, h0, stream):
    """One token through all layers with traces, checked against the fp64
    oracle teacher-forced on the GPU's own layer inputs: top-K exact at every
    layer, outputs within TOL on a spread of layers."""
    import ctypes
    import torch
    import oracle
    import quantized_expert_gemv_router_amd as q

    L, K, H = cfg.layers, cfg.top_k, cfg.hidden
    h = h0.clone()
    tk = torch.empty((L, 1, K), dtype=torch.int32, device=h.device)
    hk = torch.empty((L, 1, H), dtype=torch.float32, device=h.device)
    rc = q.lib().moe_expert_stack_decode(ctypes.byref(shape), table.view(), rt.ptr(), 0, L, 1, K, 0,
                                         h.data_ptr(), tk.data_ptr(), hk.data_ptr(), ws.data_ptr(),
                                         stream.cuda_stream)
    if rc != 0:
        raise RuntimeError(q.moeq_last_error())
    status = q.moe_read_device_status(ws, stream)
    if status != 0:
        raise ParityError(f"device status {status} in the parity run")
    idx = tk.cpu().numpy()[:, 0, :]
    hs = hk.cpu().numpy()[:, 0, :].astype(np.float64)
    outs = [hs[l + 1] for l in range(L - 1)] + [h.cpu().numpy()[0].astype(np.float64)]
    sh = oracle.shape_of(cfg)
    flags = oracle.layer_flags(cfg)
    import synth
    for l in range(L):
        ref_lg, ref_idx, _, _ = oracle.route(sh, synth.router(cfg, l), hs[l][None, :], K, flags)
        if not topk_matches(idx[l], ref_idx[0], ref_lg[0]):
            raise ParityError(f"layer {l}: GPU top-K {idx[l].tolist()} != oracle {ref_idx[0].tolist()}")
    checked = sorted(set([0, 1, L // 4, L // 2, 3 * L // 4, L - 2, L - 1]))
    worst = 0.0
    for l in checked:
        exp = oracle.run_layer(cfg, l, hs[l][None, :], want_intermediates=False)
        e = rel_err(outs[l], exp["y"][0])
        worst = max(worst, e)
        if not e <= TOL:
            raise ParityError(f"layer {l}: output rel err {e:.3e} > {TOL}")
    return {"topk_exact_layers": L, "layers": L, "outputs_checked_layers": checked,
            "max_rel_err": float(f"{worst:.3e}"), "tol": TOL,
            "reference": "fp64 oracle, teacher-forced on the GPU's layer inputs"}


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
    log("[bench] parity: one token through all layers against the fp64 oracle")
    parity = parity_stack(cfg, shape, table, rt, ws, pool[0], stream)
    log(f"[bench] parity ok: {parity}")
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
    rec["parity"] = parity
    return rec


def parity_prefill(cfg, shape, table, rt, stream, n_sample=16):
    """Layer 0 of the prefill on its own: top-K of every token against the
    fp64 oracle router, outputs of a seeded token sample against the oracle
    layer."""
    import torch
    import oracle
    import quantized_expert_gemv_router_amd as q
    import synth

    T, K = cfg.tokens, cfg.top_k
    x64 = synth.bf16_to_f64(synth.tokens(cfg, 3000, T))
    h = torch.from_numpy(x64.astype(np.float32)).to("cuda")
    ws = q.new_prefill_workspace(shape, T, K, h.device)
    tk = q.moe_expert_stack_prefill(shape, table, rt, h, K, layer0=0, L=1, workspace=ws, trace=True,
                                    stream=stream)
    status = q.moe_read_device_status(ws, stream)
    if status != 0:
        raise ParityError(f"device status {status} in the prefill parity run")
    idx = tk.cpu().numpy()[0]
    y = h.cpu().numpy().astype(np.float64)
    sh = oracle.shape_of(cfg)
    _, ref_idx, _, _ = oracle.route(sh, synth.router(cfg, 0), x64, K, oracle.layer_flags(cfg))
    bad = np.flatnonzero(~np.all(ref_idx == idx, axis=1))
    if bad.size:
        raise ParityError(f"prefill layer 0: top-K differs on {bad.size} tokens (first {bad[:5].tolist()})")
    rng = np.random.default_rng(0)
    sample = np.sort(rng.choice(T, size=min(n_sample, T), replace=False))
    exp = oracle.run_layer(cfg, 0, x64[sample], want_intermediates=False)
    e = rel_err(y[sample], exp["y"])
    if not e <= TOL:
        raise ParityError(f"prefill layer 0: output rel err {e:.3e} > {TOL}")
    del ws
    return {"topk_exact_tokens": int(T), "layer": 0, "outputs_checked_tokens": sample.tolist(),
            "max_rel_err": float(f"{e:.3e}"), "tol": TOL, "reference": "fp64 oracle"}


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
    log("[bench] parity: prefill layer 0 against the fp64 oracle")
    parity = parity_prefill(cfg, shape, table, rt, stream)
    log(f"[bench] parity ok: {parity}")
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
    gu_s = gu_ms / gu_n / 1e3
    gu_tflops = gu_flop / gu_s / 1e12
    # the gate/up GEMM's bound: HBM while its flop per weight byte is below
    # the fp16 MFMA ridge (2.5 PFLOP/s / 8 TB/s = 312), the matrix cores above
    mfma_bound = gu_flop / (MFMA_FP16_PEAK_TFLOPS * 1e12) > gu_bytes / (HBM_PEAK_GBS * 1e9)
    roof = {"kernel": "gemm_kernel<gate/up> (grouped dequant-GEMM, fp16 MFMA)",
            "avg_launch_us": round(gu_ms / gu_n * 1e3, 2), "bytes_per_launch": int(gu_bytes),
            "flop_per_launch": gu_flop, "hbm_gbs": round(gu_gbs, 1), "hbm_frac": round(gu_gbs / HBM_PEAK_GBS, 4),
            "mfma_tflops": round(gu_tflops, 1), "mfma_frac": round(gu_tflops / MFMA_FP16_PEAK_TFLOPS, 4),
            "traffic": recorded_prefill_traffic() if cfg.name == "stack60_prefill" else None}
    if mfma_bound:
        roof.update(bound="mfma", achieved=round(gu_tflops, 1), peak=MFMA_FP16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(gu_tflops / MFMA_FP16_PEAK_TFLOPS, 4))
    else:
        roof.update(bound="hbm", achieved=round(gu_gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(gu_gbs / HBM_PEAK_GBS, 4))
    rec.update({
        "gbps_expert": round(expert_bytes * args.steps / sec / 1e9, 1),
        "gbps_all_bytes": round((expert_bytes + router_bytes) * args.steps / sec / 1e9, 1),
        "frac_hbm_peak": round(expert_bytes * args.steps / sec / 1e9 / HBM_PEAK_GBS, 4),
        "expert_layers_per_s": round(args.steps * T * cfg.layers / sec, 1),
        "kernel_ms_per_layer": {k: round(v[0] / max(v[1], 1), 4) for k, v in kt.items()},
        "roofline": roof,
    })
    rec["config"].update(layers_per_step=cfg.layers, experts_touched_per_layer=float(touched.mean()),
                         resident_gb=round(cfg.layers * cfg.n_slots * cfg.expert_bytes / 1e9, 1))
    rec["parity"] = parity
    return rec


def run_layer_fused(args, cfg, dev, stream):
    """One decode token through one layer per step as a single persistent
    launch (router, top-K, gate/up, SwiGLU, down and combine in one kernel,
    the layer input taken as is: MOEQ_F_STACK_NO_NORM), rotating over
    --instances resident layer instances so the expert bytes come from HBM."""
    import ctypes
    import torch
    import quantized_expert_gemv_router_amd as q
    import synth
    import oracle

    if args.warm:
        args.instances, args.tokens_pool = 1, 1
    n_inst = args.instances
    shape, table, routers, bf16 = setup_layers(cfg, n_inst, dev, stream)
    rt = q.RouterTable(routers, device=dev)
    K = cfg.top_k
    ws = q.new_workspace(shape, 1, K, dev)
    total = args.warmup + args.steps
    tok = [torch.from_numpy(synth.bf16_to_f64(synth.tokens(cfg, 100 + i, 1)).astype(np.float32)).to(dev)
           for i in range(args.tokens_pool)]
    hs = [tok[s % args.tokens_pool].clone() for s in range(total)]
    tks = torch.empty((total, 1, 1, K), dtype=torch.int32, device=dev)
    flags = q.F_STACK_NO_NORM
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

    def step(s, slot=None):
        l = s % n_inst
        if slot is not None:
            ev[slot][0].record(stream)
        rc = q.lib().moe_expert_stack_decode(ctypes.byref(shape), table.view(), rt.ptr(), l, 1, 1, K, flags,
                                             hs[s].data_ptr(), tks[s].data_ptr(), None, ws.data_ptr(),
                                             stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(q.moeq_last_error())
        if slot is not None:
            ev[slot][1].record(stream)

    # parity: instance 0, token 0 against the fp64 oracle
    log("[bench] parity: one fused layer against the fp64 oracle")
    h0 = tok[0].clone()
    tk0 = torch.empty((1, 1, K), dtype=torch.int32, device=dev)
    rc = q.lib().moe_expert_stack_decode(ctypes.byref(shape), table.view(), rt.ptr(), 0, 1, 1, K, flags,
                                         h0.data_ptr(), tk0.data_ptr(), None, ws.data_ptr(), stream.cuda_stream)
    if rc != 0:
        raise RuntimeError(q.moeq_last_error())
    status = q.moe_read_device_status(ws, stream)
    if status != 0:
        raise ParityError(f"device status {status} in the parity run")
    path = q.moeq_last_stack_path()
    exp = oracle.run_layer(cfg, 0, synth.bf16_to_f64(synth.tokens(cfg, 100, 1)), want_intermediates=False)
    if not topk_matches(tk0.cpu().numpy()[0, 0], exp["idx"][0], exp["logits"][0]):
        raise ParityError("top-K differs from the oracle")
    e = rel_err(h0.cpu().numpy(), exp["y"])
    if not e <= TOL:
        raise ParityError(f"output rel err {e:.3e} > {TOL}")
    parity = {"topk_exact_tokens": 1, "max_rel_err": float(f"{e:.3e}"), "tol": TOL, "reference": "fp64 oracle"}
    log(f"[bench] parity ok: {parity}")

    with torch.cuda.stream(stream):
        for s in range(args.warmup):
            step(s)
    torch.cuda.synchronize()
    if args.eager:
        with torch.cuda.stream(stream):
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            start.record(stream)
            for i in range(args.steps):
                step(args.warmup + i, slot=i)
            end.record(stream)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        elapsed_ms = start.elapsed_time(end)
        launch_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        launch = "eager (one Python call per launch)"
    else:
        # the timed steps captured in one HIP graph (one kernel node each);
        # an untimed replay is checked bit for bit against the last step
        # launched eagerly on the same input, then the inputs are restored
        base = args.warmup
        h_in = [hs[base + i].clone() for i in range(args.steps)]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(args.steps):
                step(base + i)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
            torch.cuda.synchronize()
            last = base + args.steps - 1
            h_chk = h_in[-1].clone()
            rc = q.lib().moe_expert_stack_decode(ctypes.byref(shape), table.view(), rt.ptr(), last % n_inst, 1, 1,
                                                 K, flags, h_chk.data_ptr(), None, None, ws.data_ptr(),
                                                 stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(q.moeq_last_error())
            torch.cuda.synchronize()
            if not torch.equal(h_chk, hs[last]):
                raise ParityError("the graph replay's output differs from the same step launched eagerly")
            log("[bench] graph replay output equals the eager launch")
            for i in range(args.steps):
                hs[base + i].copy_(h_in[i])
            torch.cuda.synchronize()
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            start.record(stream)
            g.replay()
            end.record(stream)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        elapsed_ms = start.elapsed_time(end)
        launch_ms = elapsed_ms / args.steps
        launch = f"HIP graph of {args.steps} steps (one launch each), replayed"
    status = q.moe_read_device_status(ws, stream)
    if status != 0:
        raise RuntimeError(f"device status {status} after the timed region")
    idx = tks[args.warmup:].cpu().numpy()
    distinct = np.array([len(np.unique(idx[s])) for s in range(args.steps)]) + cfg.n_shared
    expert_bytes = distinct * cfg.expert_bytes
    router_bytes = cfg.n_experts * cfg.hidden * 2
    per_launch = float(expert_bytes.mean())
    sec = elapsed_ms / 1e3
    rec = base_record(args, cfg, steps_tokens=args.steps, elapsed_ms=elapsed_ms, wall=wall)
    path_name = "persistent" if path == 1 else "per-layer"
    rec.update({
        "gbps_expert": round(expert_bytes.sum() / sec / 1e9, 1),
        "gbps_all_bytes": round((expert_bytes.sum() + args.steps * router_bytes) / sec / 1e9, 1),
        "frac_hbm_peak": round(expert_bytes.sum() / sec / 1e9 / HBM_PEAK_GBS, 4),
        "expert_layers_per_s": round(args.steps / sec, 1),
        "path": path_name,
        "roofline": {"kernel": "stack_kernel (one layer, one persistent launch)" if path == 1
                     else "per-layer launches (3)", "bound": "hbm",
                     "achieved": round(per_launch / (launch_ms / 1e3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(per_launch / (launch_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None, "avg_launch_us": round(launch_ms * 1e3, 3),
                     "bytes_per_launch": int(per_launch), "router_bytes_per_launch": router_bytes},
        "parity": parity,
    })
    rec["config"].update(layers_per_step=1, layer_instances=n_inst, launch=launch,
                         weights=("warm: one layer instance and one token every step, the same experts"
                                  if args.warm else
                                  f"cold: {n_inst} layer instances x {args.tokens_pool} tokens rotating, "
                                  "far more expert bytes than the 256 MB of last-level cache"))
    return rec


def run_layer_workload(args, cfg, dev, stream):
    import torch
    import quantized_expert_gemv_router_amd as q
    import synth

    if args.warm:
        args.instances, args.tokens_pool = 1, 1
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

    # parity: instance 0, token set 0, through the same three calls
    import oracle
    log("[bench] parity: one step against the fp64 oracle")
    x0 = pool[0]
    q.moe_router_topk(shape, x0, routers[0], K, 0, None, ws, out=(idx_all[0], w, sw), stream=stream)
    q.moe_q4_expert_gemv(shape, table, 0, x0, idx_all[0], K, 0, ws, gu, stream=stream)
    q.moe_swiglu_down_combine(shape, table, 0, gu, idx_all[0], w, sw, x0, K, ws, y, stream=stream)
    status = q.moe_read_device_status(ws, stream)
    if status != 0:
        raise ParityError(f"device status {status} in the parity run")
    x64 = synth.bf16_to_f64(synth.tokens(cfg, 100, T))
    exp = oracle.run_layer(cfg, 0, x64, want_intermediates=False)
    if not np.array_equal(idx_all[0].cpu().numpy(), exp["idx"]):
        raise ParityError("top-K differs from the oracle")
    e = rel_err(y.cpu().numpy(), exp["y"])
    if not e <= TOL:
        raise ParityError(f"output rel err {e:.3e} > {TOL}")
    parity = {"topk_exact_tokens": T, "max_rel_err": float(f"{e:.3e}"), "tol": TOL,
              "reference": "fp64 oracle, same inputs"}
    log(f"[bench] parity ok: {parity}")

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

    if args.eager:
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
        launch = "eager (one Python call per kernel)"
    else:
        elapsed_ms, gemv_ms, wall = time_layer_graph(args, step, stream, shape, table, pool, idx_all, ws, gu, y, K)
        launch = f"HIP graph of {args.steps} steps (3 launches each), replayed"
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
    rec["config"].update(layers_per_step=1, layer_instances=n_inst, launch=launch,
                         weights=("warm: one layer instance and one token every step, the same experts"
                                  if args.warm else
                                  f"cold: {n_inst} layer instances x {args.tokens_pool} tokens rotating, "
                                  "far more expert bytes than the 256 MB of last-level cache"))
    rec["parity"] = parity
    return rec


def time_layer_graph(args, step, stream, shape, table, pool, idx_all, ws, gu, y, K):
    """The timed steps captured in one HIP graph (three kernel nodes per
    step), replayed once after an untimed replay; the gate/up call alone is
    captured the same way for its per-launch time.  The graph's last output
    is checked bit for bit against the same step launched eagerly."""
    import torch
    import quantized_expert_gemv_router_amd as q

    with torch.cuda.stream(stream):
        for s in range(args.warmup):
            step(s)
    torch.cuda.synchronize()
    base = args.warmup
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(args.steps):
            step(base + i)
    gg = torch.cuda.CUDAGraph()   # the gate/up launches of the same steps
    with torch.cuda.graph(gg, stream=stream):
        for i in range(args.steps):
            s = base + i
            q.moe_q4_expert_gemv(shape, table, s % args.instances, pool[s % args.tokens_pool], idx_all[s], K, 0,
                                 ws, gu, stream=stream)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        g.replay()   # untimed
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(stream)
        g.replay()
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        y_graph = y.clone()
        gs, ge = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gg.replay()
        gs.record(stream)
        gg.replay()
        ge.record(stream)
        torch.cuda.synchronize()
        step(base + args.steps - 1)   # the last step again, launched eagerly
        torch.cuda.synchronize()
    if not torch.equal(y_graph, y):
        raise ParityError("the graph replay's output differs from the same step launched eagerly")
    log("[bench] graph replay output equals the eager launch")
    return start.elapsed_time(end), gs.elapsed_time(ge) / args.steps, wall


def run_pool(args, cfg, dev, stream):
    """Decode through a bounded expert pool (the paged mode of the pages):
    the 60-layer model's expert shapes, L layers of 513 experts held in
    pinned host memory, slots_per_layer * L device slots, least recently used
    slot evicted.  Per layer and token: router on the GPU, the K ids to the
    host, pool acquire (misses copied host -> HBM on the copy streams),
    gate/up and down/combine through the pool's pointer table, release.
    Every step is a new N(0,1) token: the routing is the synthetic model's
    own (uniform over experts at layer 0; later layers concentrate, as the
    layer outputs share a component across tokens), not the pages' text."""
    import torch
    import quantized_expert_gemv_router_amd as q
    import synth
    import oracle

    L = args.pool_layers
    cfg = synth.with_changes(cfg, layers=L)
    shape = q.Shape.of(cfg)
    P, K, E, H = cfg.n_slots, cfg.top_k, cfg.n_experts, cfg.hidden
    stride = (cfg.expert_bytes + 255) // 256 * 256
    host_gb = L * P * stride / 1e9
    log(f"[bench] pool_decode: {L} layers x {P} experts in pinned host memory ({host_gb:.1f} GB)")
    gen = torch.empty(P * stride, dtype=torch.uint8, device=dev)
    host = []
    for l in range(L):
        synth.device_fill_experts(cfg, l, gen.data_ptr(), stride, stream=stream.cuda_stream)
        stream.synchronize()
        t = torch.empty(P * stride, dtype=torch.uint8, pin_memory=True)
        t.copy_(gen)
        host.append(t)
    del gen
    bf16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    routers = [bf16(synth.router(cfg, l)) for l in range(L)]
    def fresh(i):   # token i of a stream of distinct tokens (independent routings)
        return torch.from_numpy(synth.bf16_to_f64(synth.tokens(cfg, 100 + i, 1)).astype(np.float32)).to(dev)

    ws = q.new_workspace(shape, 1, K, dev)
    idx = torch.empty((1, K), dtype=torch.int32, device=dev)
    w = torch.empty((1, K), dtype=torch.float32, device=dev)
    sw = torch.empty((1,), dtype=torch.float32, device=dev)
    gu = torch.empty((1, K + cfg.n_shared, 2, cfg.inter), dtype=torch.float32, device=dev)
    ids_host = torch.empty((1, K), dtype=torch.int32, pin_memory=True)
    copies = [torch.cuda.Stream(device=dev) for _ in range(max(int(c) for c in args.pool_streams.split(",")))]

    def token(pool, h, trace=None, prev=None, prefetch=False):
        for l in range(L):
            if trace is not None:
                trace.append(h.clone())
            if prefetch and prev is not None and prev[l] is not None:
                # before this layer's routing resolves: the previous token's
                # experts of the layer start their copies
                pool.prefetch(l, prev[l])
            q.moe_router_topk(shape, h, routers[l], K, q.F_RMSNORM, None, ws, out=(idx, w, sw), stream=stream)
            ids_host.copy_(idx, non_blocking=True)
            stream.synchronize()
            sel = ids_host[0].tolist()
            if prev is not None:
                if prev[l] is not None:
                    token.reused += len(set(sel) & set(prev[l]))
                    token.routed += len(sel)
                prev[l] = sel
            view = pool.acquire(l, sel + list(range(E, P)), stream=stream)
            q.moe_q4_expert_gemv(shape, view, l, h, idx, K, q.F_RMSNORM, ws, gu, stream=stream)
            q.moe_swiglu_down_combine(shape, view, l, gu, idx, w, sw, h, K, ws, h, stream=stream)
            pool.release(l, stream=stream)

    def make_pool(slots, n_streams):
        arena = torch.empty(L * slots * stride, dtype=torch.uint8, device=dev)
        table = torch.zeros(L * P, dtype=torch.int64, device=dev)
        pool = q.Pool(shape, L, arena, L * slots, stride, host, table, copies[:n_streams])
        return pool, arena, table

    # raw host -> HBM copy rate of one expert blob per copy, for the PCIe bound
    NCP = 256
    dst = torch.empty(64 * stride, dtype=torch.uint8, device=dev)
    raw = {}
    for ns in sorted(set(int(c) for c in args.pool_streams.split(","))):
        for rep_ in range(2):   # the first pass warms the copy paths up
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(NCP):
                e = (i * 37) % P
                with torch.cuda.stream(copies[i % ns]):
                    dst[(i % 64) * stride:(i % 64 + 1) * stride].copy_(
                        host[i % L][e * stride:e * stride + stride], non_blocking=True)
            torch.cuda.synchronize()
            raw[ns] = round(NCP * stride / (time.perf_counter() - t0) / 1e9, 2)
    del dst
    log(f"[bench] raw pinned host -> HBM copy rate (GB/s) by copy streams: {raw}")

    # parity: one token through the pool (fewest slots, most streams) is
    # bit-identical to the resident per-layer path, whose top-K equals the
    # fp64 oracle's on the GPU's own layer inputs
    log("[bench] parity: pooled token vs resident per-layer path and the fp64 oracle")
    slots_list = [int(x) for x in args.pool_slots.split(",")]
    streams_list = [int(x) for x in args.pool_streams.split(",")]
    pool, arena, table = make_pool(min(slots_list), max(streams_list))
    h_pool = fresh(0)
    trace = []
    with torch.cuda.stream(stream):
        token(pool, h_pool, trace)
    pool.destroy()
    del pool, arena, table
    res = [torch.empty(P * stride, dtype=torch.uint8, device=dev) for _ in range(L)]
    for l in range(L):
        res[l].copy_(host[l])
    table_r = q.ExpertTable(shape, res, stride, device=dev)
    rt = q.RouterTable(routers, device=dev)
    h_res = fresh(0)
    ws_r = q.new_workspace(shape, 1, K, dev)
    tk, hk = q.moe_expert_stack_decode(shape, table_r, rt, h_res, K, flags=q.F_STACK_LAYERWISE, workspace=ws_r,
                                       trace=True, stream=stream)
    torch.cuda.synchronize()
    if not torch.equal(h_res, h_pool):
        raise ParityError("pooled decode differs from the resident per-layer path")
    for l in range(L):
        if not torch.equal(hk[l], trace[l]):
            raise ParityError(f"layer {l}: pooled layer input differs from the resident path")
        _, ridx, _, _ = oracle.route(oracle.shape_of(cfg), synth.router(cfg, l),
                                     trace[l].cpu().numpy().astype(np.float64), K, oracle.layer_flags(cfg))
        if not np.array_equal(ridx[0], tk[l, 0].cpu().numpy()):
            raise ParityError(f"layer {l}: top-K differs from the oracle")
    ref = oracle.run_layer(cfg, 0, trace[0].cpu().numpy().astype(np.float64), want_intermediates=False)
    e0 = rel_err(trace[1].cpu().numpy(), ref["y"]) if L > 1 else rel_err(h_pool.cpu().numpy(), ref["y"])
    if not e0 <= TOL:
        raise ParityError(f"layer 0 output rel err {e0:.3e} > {TOL}")
    parity = {"pooled_equals_resident_bitwise": True, "topk_exact_layers": L, "layer0_rel_err": float(f"{e0:.3e}"),
              "tol": TOL, "reference": "resident per-layer path (bitwise) and the fp64 oracle"}
    del res, table_r, rt, ws_r, tk, hk
    log(f"[bench] parity ok: {parity}")

    curve = []
    for slots in slots_list:
        for ns in streams_list:
            pool, arena, table = make_pool(slots, ns)
            resident = slots >= P
            if resident:
                pool.make_resident(stream=stream)
            n_warm = args.warmup if resident else max(args.warmup, 64)
            with torch.cuda.stream(stream):
                for i in range(n_warm):
                    token(pool, fresh(10000 + i))
            torch.cuda.synchronize()
            st0 = pool.stats()
            hs = [fresh(20000 + i) for i in range(args.steps)]
            t0 = time.perf_counter()
            with torch.cuda.stream(stream):
                for i in range(args.steps):
                    token(pool, hs[i])
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            st = pool.stats()
            hits, misses = st["hits"] - st0["hits"], st["misses"] - st0["misses"]
            copied = st["bytes_copied"] - st0["bytes_copied"]
            curve.append({"slots_per_layer": slots, "copy_streams": ns, "resident": resident,
                          "tokens_per_s": round(args.steps / dt, 2), "ms_per_token": round(dt / args.steps * 1e3, 3),
                          "hit_rate": round(hits / max(hits + misses, 1), 4),
                          "misses_per_token_layer": round(misses / (args.steps * L), 3),
                          "h2d_gbs": round(copied / dt / 1e9, 2),
                          "slot_gb": round(L * slots * stride / 1e9, 2)})
            log(f"[bench] {curve[-1]}")
            pool.destroy()
            del pool, arena, table
            torch.cuda.empty_cache()
    at20 = [c for c in curve if c["slots_per_layer"] == 20] or curve
    head = max(at20, key=lambda c: c["tokens_per_s"])

    # temporal reuse (a stand-in for correlated text, labelled as such): a
    # chain of tokens x_{t+1} = a x_t + sqrt(1 - a^2) z_{t+1}, with and
    # without prefetching the previous token's experts of each layer before
    # its router runs; fewest slots, one copy stream
    reuse_curve = []
    slots_r = min(slots_list)
    for alpha in [float(v) for v in args.pool_reuse.split(",")]:
        beta = float(np.sqrt(max(0.0, 1.0 - alpha * alpha)))
        for pf in (False, True):
            pool, arena, table = make_pool(slots_r, 1)
            prev = [None] * L
            x = fresh(30000)
            token.reused = token.routed = 0
            with torch.cuda.stream(stream):
                for i in range(max(args.warmup, 32)):
                    x = alpha * x + beta * fresh(30001 + i)
                    token(pool, x.clone(), prev=prev, prefetch=pf)
            torch.cuda.synchronize()
            st0 = pool.stats()
            token.reused = token.routed = 0
            chain = []
            for i in range(args.steps):
                x = alpha * x + beta * fresh(40000 + i)
                chain.append(x.clone())
            t0 = time.perf_counter()
            with torch.cuda.stream(stream):
                for i in range(args.steps):
                    token(pool, chain[i], prev=prev, prefetch=pf)
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            st = pool.stats()
            hits, misses = st["hits"] - st0["hits"], st["misses"] - st0["misses"]
            reuse_curve.append({"correlation_a": alpha, "prefetch": pf, "slots_per_layer": slots_r,
                                "measured_reuse": round(token.reused / max(token.routed, 1), 4),
                                "tokens_per_s": round(args.steps / dt, 2), "hit_rate": round(hits / max(hits + misses, 1), 4),
                                "h2d_gbs": round((st["bytes_copied"] - st0["bytes_copied"]) / dt / 1e9, 2)})
            log(f"[bench] {reuse_curve[-1]}")
            pool.destroy()
            del pool, arena, table
            torch.cuda.empty_cache()
    sec = head["ms_per_token"] / 1e3
    rec = base_record(args, cfg, steps_tokens=args.steps, elapsed_ms=sec * args.steps * 1e3, wall=sec * args.steps)
    rec.update({
        "expert_layers_per_s": round(L / sec, 1),
        "roofline": {"kernel": "host -> HBM expert copies (hipMemcpyAsync from pinned host)", "bound": "pcie",
                     "achieved": head["h2d_gbs"], "peak": 64.0, "unit": "GB/s",
                     "frac": round(head["h2d_gbs"] / 64.0, 4), "traffic": None,
                     "raw_copy_gbs_by_streams": raw},
        "curve": curve,
        "reuse_curve": reuse_curve,
        "parity": parity,
    })
    rec["config"].update(layers_per_step=L, slots_per_layer=head["slots_per_layer"],
                         copy_streams=head["copy_streams"], host_pinned_gb=round(host_gb, 1),
                         routing="synthetic model's own: distinct N(0,1) tokens, uniform at layer 0, "
                                 "concentrating in later layers")
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


def probe_handoff():
    """Hand-off latency sweep: one JSON line per (pattern, words, layout, back-off)."""
    import quantized_expert_gemv_router_amd as q
    names = {0: "tagged all-gather", 1: "flag + payload", 2: "ping-pong", 3: "counter barrier",
             4: "gather to one + broadcast", 5: "gather to one + broadcast + one data read",
             6: "tagged all-gather, pipelined polls", 7: "fixed-point atomic reduction"}
    cases = [(6, w, w, s, d) for w in (1, 4, 8) for s in (0, 1, 2) for d in (2, 4)]
    cases += [(0, w, w, s, 1) for w in (1, 4, 8) for s in (0, 1)]
    cases += [(2, 1, 1, s, p) for s in (0, 1) for p in (1, 8)]
    cases += [(3, 1, 1, s, 1) for s in (0, 1)]
    cases += [(0, w, w, s, 1) for w in (1, 2, 4, 8, 16, 32) for s in (0, 1)]
    cases += [(0, w, st, 1, 1) for w in (1, 4, 16) for st in (16, 64, 512)]
    cases += [(1, w, w, 1, 1) for w in (1, 4, 16)]
    cases += [(4, w, w, 1, c) for w in (1, 4, 16) for c in (1, 8, 32)]
    cases += [(5, w, w, 1, c) for w in (4, 16) for c in (8, 32)]
    cases += [(7, w, 2 * w, s, 1) for w in (1, 2, 4) for s in (0, 1)]
    xcc_logged = False
    for mode, w, stride, s, peer in cases:
        if stride < w:
            continue
        rounds = 2000
        try:
            q.moeq_probe_handoff(mode, w, 50, s, peer, stride=stride)            # warm-up
            r = q.moeq_probe_handoff(mode, w, rounds, s, peer, stride=stride)
        except q.MoeqError as e:
            print(json.dumps({"probe": names[mode], "mode": mode, "words_per_block": w, "sleep": s,
                              "error": str(e)}), flush=True)
            if e.code != q.E_UNSUPPORTED:
                break          # a wait gave up: stop the sweep
            continue
        rec = {"probe": names[mode], "mode": mode, "words_per_block": w, "stride_words": stride, "sleep": s,
               "us_per_round": round(r["ticks"] * 0.01 / rounds, 3), "stale_words": r["stale"]}
        if mode in (4, 5):
            rec["go_copies"] = peer
        if mode == 6:
            rec["loads_in_flight"] = peer
        if mode == 2:
            rec["peer"] = peer
            rec["us_one_way"] = round(r["ticks"] * 0.01 / rounds / 2, 3)
        if not xcc_logged:
            rec["xcc_of_workgroup"] = r["xcc"]
            xcc_logged = True
        print(json.dumps(rec), flush=True)


def block_timeline(L, dev, stream):
    """Per-workgroup clock trace of the persistent decode (one token through
    L layers of the 60-layer configuration, six traced launches after five
    untraced ones): when each workgroup reached each phase, relative to the
    last workgroup's h publish of the previous layer, and the poll rounds of
    each hand-off.  Printed as text."""
    import torch
    import quantized_expert_gemv_router_amd as q
    import synth

    cfg = synth.with_changes(synth.CONFIGS["stack60_decode"], layers=L)
    shape, table, routers, _ = setup_layers(cfg, L, dev, stream)
    rt = q.RouterTable(routers, device=dev)
    ws = q.new_workspace(shape, 1, cfg.top_k, dev)
    x = torch.from_numpy(synth.bf16_to_f64(synth.tokens(cfg, 0, 1)).astype(np.float32)).to(dev)
    for _ in range(5):
        h = x.clone()
        q.moe_expert_stack_decode(shape, table, rt, h, cfg.top_k, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    NB = torch.cuda.get_device_properties(dev).multi_processor_count
    EV = 16
    reps = []
    for _ in range(6):
        clk = torch.zeros((NB, L, EV), dtype=torch.int64, device=dev)
        if q.moeq_stack_block_clock_trace(clk) != EV:
            raise RuntimeError("unexpected clock-trace width")
        h = x.clone()
        q.moe_expert_stack_decode(shape, table, rt, h, cfg.top_k, workspace=ws, stream=stream)
        torch.cuda.synchronize()
        reps.append(clk.cpu().numpy())
    if q.moe_read_device_status(ws, stream) != 0:
        raise RuntimeError("device status set during the traced launches")
    tick_us = 0.01   # the 100 MHz constant clock
    names = {0: "start", 1: "h polled", 2: "lg pub", 3: "lg polled", 7: "topk w0", 4: "topk", 14: "gu issued",
             15: "shared pub", 5: "gu dots", 6: "a pub", 8: "a polled", 9: "h pub"}
    rows, per = [], []
    for c in reps:
        t = c.astype(np.float64) * tick_us
        for l in range(2, L - 1):
            rows.append(t[:, l, :] - t[:, l - 1, 9].max())
        per.append(np.median(np.diff(t[:, :, 0].min(axis=0))))
    R = np.stack(rows)
    print(f"stack decode block timeline: {L} layers, {NB} workgroups, 6 launches; layer period "
          f"(median of min-over-workgroups start differences) {np.median(per):.2f} us")
    print("times after the last workgroup's h publish of the previous layer (us), medians over layers:")
    print(f"{'event':10s} {'min':>7s} {'median':>7s} {'p90':>7s} {'max':>7s}   (over workgroups)")
    for ev in names:   # in phase order
        v = R[:, :, ev]
        print(f"{names[ev]:10s} {np.median(v.min(1)):7.2f} {np.median(np.median(v, 1)):7.2f} "
              f"{np.median(np.percentile(v, 90, axis=1)):7.2f} {np.median(v.max(1)):7.2f}")
    for nm, pub, poll in (("logits", 2, 3), ("activations", 6, 8)):
        lp = R[:, :, pub].max(1)
        print(f"{nm}: last publish {np.median(lp):.2f}; polled min {np.median(R[:, :, poll].min(1) - lp):.2f} "
              f"median {np.median(np.median(R[:, :, poll], 1) - lp):.2f} max {np.median(R[:, :, poll].max(1) - lp):.2f}"
              " after it")
    for ev, nm in ((2, "lg pub"), (5, "gu dots"), (6, "a pub"), (9, "h pub")):
        v = np.median(R[:, :, ev], axis=0)
        print(f"{nm:8s} median by XCD (workgroup mod 8):", " ".join(f"{np.median(v[x::8]):.2f}" for x in range(8)))
    raw = np.stack(reps)
    for ev, nm in ((10, "h"), (11, "logits"), (12, "shared acts"), (13, "routed acts")):
        v = raw[:, :, 2:L - 1, ev]
        print(f"poll rounds {nm:12s}: median {np.median(v):.0f}  p90 {np.percentile(v, 90):.0f}  max {v.max():.0f}")


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
    if args.probe_handoff:
        probe_handoff()
        return
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, dev)
        return
    stream = torch.cuda.Stream(device=dev)
    if args.block_timeline:
        block_timeline(args.block_timeline, dev, stream)
        return
    if args.workload == "pool_decode":
        rec = run_pool(args, synth.CONFIGS["stack60_decode"], dev, stream)
        print(json.dumps(rec), flush=True)
        return
    cfg = synth.CONFIGS[args.workload]
    if cfg.layers > 1 and cfg.tokens > 1:
        rec = run_prefill(args, cfg, dev, stream)
    elif cfg.layers > 1:
        rec = run_stack(args, cfg, dev, stream)
    elif cfg.tokens == 1 and cfg.bits in (2, 3, 4) and not args.layer_calls:
        # widths with a persistent instantiation: the whole layer in one launch
        rec = run_layer_fused(args, cfg, dev, stream)
    else:
        rec = run_layer_workload(args, cfg, dev, stream)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle sample")
        rec["cpu_baseline"] = (cpu_baseline_stack if cfg.layers > 1 else cpu_baseline_layer)(
            cfg, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
