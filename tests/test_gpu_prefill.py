"""GPU parity of the prefill path (moe_expert_stack_prefill) against the
fp64 oracle.

Tokens are independent (no attention), so each prefill layer must give, per
token, the decode layer's result: the oracle runs the same layer on the
GPU's own input h_l (fp32, exact in fp64; teacher forcing), top-K must be
bit-exact and h_{l+1} within max|gpu - oracle| <= 2e-3 * max|oracle|.  The
expert GEMMs use fp16 operands (activations and dequantised weights, one
rounding each) with fp32 accumulation, which stays well inside that bar.

At the full workload size (2048 tokens, 512 experts, top-10 + shared, 60
resident layers): layer 0 is checked for every token (top-K and output), a
seeded 32-token sample through all 60 layers, and the 4096- and 8192-token
prefills on layer 0 (every token's top-K) and a token sample over four
layers.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import quantized_expert_gemv_router_amd as q
import synth
from tests.gpu_util import assert_close, bf16_dev, say, slot_stride

pytestmark = pytest.mark.gpu


def build(cfg, L):
    shape = q.Shape.of(cfg)
    stride = slot_stride(cfg)
    arenas = []
    for l in range(L):
        a = torch.empty(cfg.n_slots * stride, dtype=torch.uint8, device="cuda")
        synth.device_fill_experts(cfg, l, a.data_ptr(), stride)
        arenas.append(a)
    routers = q.RouterTable([bf16_dev(synth.router(cfg, l)) for l in range(L)])
    torch.cuda.synchronize()
    return shape, q.ExpertTable(shape, arenas, stride), routers


def tokens_f32(cfg, token_set, T):
    return torch.from_numpy(synth.bf16_to_f64(synth.tokens(cfg, token_set, T)).astype(np.float32)).cuda()


def check_layer(cfg, layer, h_in, h_out, idx, rows=None, renorm=True, tag=""):
    """Oracle layer on the GPU's input rows; exact top-K, output within tolerance."""
    rows = np.arange(h_in.shape[0]) if rows is None else rows
    x = h_in[rows].astype(np.float64)
    ref = oracle.run_layer(synth.with_changes(cfg, rmsnorm=True), layer, x, want_intermediates=False,
                           renorm=renorm)
    srt = -np.sort(-ref["logits"], axis=1)
    gap = (srt[:, cfg.top_k - 1] - srt[:, cfg.top_k]).min()
    bad = np.flatnonzero((idx[rows] != ref["idx"]).any(axis=1))
    assert bad.size == 0, f"{tag} layer {layer}: top-K differs at tokens {rows[bad][:8]} (min gap {gap:.2e})"
    e = assert_close(h_out[rows], ref["y"], f"{tag} layer {layer} output")
    return e, gap


SMALL = {
    # ragged tiles: ~75 pairs per routed expert, 300 for the shared one
    "h256_e8_k2_t300": (synth.with_changes(synth.CONFIGS["stack60_prefill"], name="pf_tiny", hidden=256,
                                           inter=128, n_experts=8, top_k=2, layers=3), 300),
    # more experts than tokens per expert; T not a multiple of anything
    "h1024_e64_k6_t513": (synth.with_changes(synth.CONFIGS["stack60_prefill"], name="pf_mid", hidden=1024,
                                             inter=256, n_experts=64, top_k=6, layers=2), 513),
    # a single token through the prefill path
    "h512_e16_k3_t1": (synth.with_changes(synth.CONFIGS["stack60_prefill"], name="pf_one", hidden=512,
                                          inter=128, n_experts=16, top_k=3, layers=2), 1),
    # the boundary's maximum: 4096 routed experts and top-16 (most experts get
    # zero to two pairs, so nearly every row tile is a ragged one)
    "h256_e4096_k16_t200": (synth.with_changes(synth.CONFIGS["stack60_prefill"], name="pf_emax", hidden=256,
                                               inter=128, n_experts=4096, top_k=16, layers=1), 200),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_prefill_small_layer_by_layer(name):
    cfg, T = SMALL[name]
    say(f"[prefill] {name}")
    shape, ex, rt = build(cfg, cfg.layers)
    h = tokens_f32(cfg, 7, T)
    ws = q.new_prefill_workspace(shape, T, cfg.top_k)
    for l in range(cfg.layers):
        h_in = h.cpu().numpy().copy()
        tk = q.moe_expert_stack_prefill(shape, ex, rt, h, cfg.top_k, layer0=l, L=1, workspace=ws, trace=True)
        e, gap = check_layer(cfg, l, h_in, h.cpu().numpy(), tk[0].cpu().numpy(), tag=name)
        say(f"  layer {l}: {T} tokens exact top-K (min gap {gap:.2e}), output rel err {e:.2e}")
    assert q.moe_read_device_status(ws) == 0


def test_prefill_multi_layer_call_matches_layer_by_layer():
    cfg, T = SMALL["h256_e8_k2_t300"]
    shape, ex, rt = build(cfg, cfg.layers)
    ws = q.new_prefill_workspace(shape, T, cfg.top_k)
    h1 = tokens_f32(cfg, 3, T)
    h2 = h1.clone()
    tk = q.moe_expert_stack_prefill(shape, ex, rt, h1, cfg.top_k, workspace=ws, trace=True)
    for l in range(cfg.layers):
        t2 = q.moe_expert_stack_prefill(shape, ex, rt, h2, cfg.top_k, layer0=l, L=1, workspace=ws, trace=True)
        assert torch.equal(tk[l], t2[0])
    assert torch.equal(h1, h2)


def test_prefill_batch_invariance_and_reproducible():
    """A token's result does not depend on the other tokens of the batch."""
    cfg, T = SMALL["h1024_e64_k6_t513"]
    shape, ex, rt = build(cfg, 1)
    x = tokens_f32(cfg, 11, T)
    full = x.clone()
    q.moe_expert_stack_prefill(shape, ex, rt, full, cfg.top_k, L=1)
    again = x.clone()
    q.moe_expert_stack_prefill(shape, ex, rt, again, cfg.top_k, L=1)
    assert torch.equal(full, again)
    parts = [x[:200].clone(), x[200:201].clone(), x[201:].clone()]
    for p in parts:
        q.moe_expert_stack_prefill(shape, ex, rt, p, cfg.top_k, L=1)
    assert torch.equal(torch.cat(parts), full)


def test_prefill_no_renorm():
    cfg, T = SMALL["h256_e8_k2_t300"]
    shape, ex, rt = build(cfg, 1)
    h = tokens_f32(cfg, 5, T)
    h_in = h.cpu().numpy().copy()
    tk = q.moe_expert_stack_prefill(shape, ex, rt, h, cfg.top_k, L=1, flags=q.F_NO_RENORM, trace=True)
    check_layer(cfg, 0, h_in, h.cpu().numpy(), tk[0].cpu().numpy(), renorm=False, tag="no-renorm")


def test_prefill_refuses_unsupported():
    cfg, T = SMALL["h256_e8_k2_t300"]
    shape, ex, rt = build(cfg, 1)
    h = tokens_f32(cfg, 5, 4)
    two = q.Shape(256, 128, 8, 1, 2, 64)
    with pytest.raises(q.MoeqError) as ei:
        q.moe_expert_stack_prefill(two, ex, rt, h, 2, L=1, workspace=torch.zeros(1 << 20, dtype=torch.uint8,
                                                                                  device="cuda"))
    assert ei.value.code == q._binding.E_UNSUPPORTED
    odd = q.Shape(192, 128, 8, 1, 4, 64)
    with pytest.raises(q.MoeqError) as ei:
        q.moe_expert_stack_prefill(odd, ex, rt, h, 2, L=1, workspace=torch.zeros(1 << 20, dtype=torch.uint8,
                                                                                  device="cuda"))
    assert ei.value.code == q._binding.E_UNSUPPORTED


def fill_blob_cache(cfg, layer, experts, cache):
    """Host blobs of (layer, e) for the experts the oracle will read, made by
    the seeded generator on a thread pool (the C generator runs without the
    interpreter lock)."""
    need = sorted(set(int(e) for e in experts) - {e for (l, e) in cache if l == layer})
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as pool:
        for e, blob in zip(need, pool.map(lambda e: synth.expert_blob(cfg, layer, e), need)):
            cache[(layer, e)] = blob


def oracle_layer(cfg, layer, x, cache):
    """The oracle layer on rows x (fp64), blobs from `cache` (filled first)."""
    sh = oracle.shape_of(cfg)
    _, idx, _, _ = oracle.route(sh, synth.router(cfg, layer), x, cfg.top_k, oracle.layer_flags(cfg))
    fill_blob_cache(cfg, layer, list(np.unique(idx)) + list(range(cfg.n_experts, cfg.n_slots)), cache)
    return oracle.run_layer(cfg, layer, x, want_intermediates=False, blob_cache=cache)


@pytest.fixture(scope="module")
def full():
    """The 60 resident layers of the prefill workload (218 GB)."""
    cfg = synth.CONFIGS["stack60_prefill"]
    say(f"[prefill] full size: E={cfg.n_experts} top-{cfg.top_k}+{cfg.n_shared}, {cfg.layers} layers resident")
    shape, ex, rt = build(cfg, cfg.layers)
    yield cfg, shape, ex, rt
    del ex
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_prefill_full_size_layer0_every_token(full):
    """Layer 0 of the 2048-token workload: top-K and output of every token
    against the fp64 oracle; layer 1 (on the GPU's layer-0 output): top-K of
    every token and the outputs of a seeded sample."""
    cfg, shape, ex, rt = full
    T = cfg.tokens
    ws = q.new_prefill_workspace(shape, T, cfg.top_k)
    h = tokens_f32(cfg, 0, T)
    cache = {}
    rng = np.random.default_rng(2024)
    for l in range(2):
        h_in = h.cpu().numpy().copy()
        tk = q.moe_expert_stack_prefill(shape, ex, rt, h, cfg.top_k, layer0=l, L=1, workspace=ws, trace=True)
        torch.cuda.synchronize()
        idx = tk[0].cpu().numpy()
        rows = np.arange(T) if l == 0 else np.sort(rng.choice(T, size=32, replace=False))
        x = h_in.astype(np.float64)
        logits, ridx, _, _ = oracle.route(oracle.shape_of(cfg), synth.router(cfg, l), x, cfg.top_k,
                                          oracle.layer_flags(cfg))
        bad = np.flatnonzero((idx != ridx).any(axis=1))
        assert bad.size == 0, f"layer {l}: top-K differs at {bad.size} tokens, first {bad[:8]}"
        ref = oracle_layer(cfg, l, x[rows], cache)
        e = assert_close(h.cpu().numpy()[rows], ref["y"], f"full layer {l} output")
        counts = np.bincount(idx.ravel(), minlength=cfg.n_experts)
        say(f"  layer {l}: all {T} tokens exact top-K; outputs of {rows.size} tokens rel err {e:.2e}; "
            f"pairs per expert {counts.min()}..{counts.max()}")
        cache.clear()
    assert q.moe_read_device_status(ws) == 0


@pytest.mark.timeout(900)
def test_prefill_full_size_60_layers_token_sample(full):
    """All 60 layers of the 2048-token prefill, one layer per call; a seeded
    sample of 32 tokens is checked at every layer against the fp64 oracle on
    the GPU's own layer input (teacher forcing): exact top-K, output within
    the bar."""
    cfg, shape, ex, rt = full
    T = cfg.tokens
    ws = q.new_prefill_workspace(shape, T, cfg.top_k)
    h = tokens_f32(cfg, 1, T)
    rows = np.sort(np.random.default_rng(60).choice(T, size=32, replace=False))
    rows_dev = torch.from_numpy(rows).cuda()
    ins, outs, idxs = [], [], []
    for l in range(cfg.layers):
        ins.append(h[rows_dev].cpu().numpy().astype(np.float64))
        tk = q.moe_expert_stack_prefill(shape, ex, rt, h, cfg.top_k, layer0=l, L=1, workspace=ws, trace=True)
        idxs.append(tk[0][rows_dev].cpu().numpy())
        outs.append(h[rows_dev].cpu().numpy().astype(np.float64))
    assert q.moe_read_device_status(ws) == 0
    worst, cache = 0.0, {}
    for l in range(cfg.layers):
        ref = oracle_layer(cfg, l, ins[l], cache)
        bad = np.flatnonzero((idxs[l] != ref["idx"]).any(axis=1))
        assert bad.size == 0, f"layer {l}: top-K differs at sampled tokens {rows[bad][:8]}"
        worst = max(worst, assert_close(outs[l], ref["y"], f"60-layer sample, layer {l} output"))
        cache.clear()
    say(f"  {rows.size} tokens x {cfg.layers} layers: exact top-K, worst output rel err {worst:.2e}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [4096, 8192])
def test_prefill_large_token_counts(full, T):
    """Prefill at 4096 and 8192 tokens (the MFMA-bound side of the roofline):
    layer 0 top-K of every token against the fp64 oracle router; layers 0..3
    through one multi-layer call on the same tokens must equal layer-by-layer
    calls, and a seeded token sample is checked at each of those layers
    against the oracle on the GPU's own input."""
    cfg, shape, ex, rt = full
    L = 4
    ws = q.new_prefill_workspace(shape, T, cfg.top_k)
    x = tokens_f32(cfg, 40 + T // 4096, T)
    h_all = x.clone()
    tk_all = q.moe_expert_stack_prefill(shape, ex, rt, h_all, cfg.top_k, layer0=0, L=L, workspace=ws, trace=True)
    rows = np.sort(np.random.default_rng(T).choice(T, size=24, replace=False))
    rows_dev = torch.from_numpy(rows).cuda()
    h = x.clone()
    cache = {}
    worst = 0.0
    for l in range(L):
        h_in = h.cpu().numpy().astype(np.float64)
        tk = q.moe_expert_stack_prefill(shape, ex, rt, h, cfg.top_k, layer0=l, L=1, workspace=ws, trace=True)
        assert torch.equal(tk[0], tk_all[l]), f"T={T} layer {l}: multi-layer call routes differently"
        idx = tk[0].cpu().numpy()
        if l == 0:
            _, ridx, _, _ = oracle.route(oracle.shape_of(cfg), synth.router(cfg, 0), h_in, cfg.top_k,
                                         oracle.layer_flags(cfg))
            bad = np.flatnonzero((idx != ridx).any(axis=1))
            assert bad.size == 0, f"T={T} layer 0: top-K differs at {bad.size} tokens, first {bad[:8]}"
        ref = oracle_layer(cfg, l, h_in[rows], cache)
        bad = np.flatnonzero((idx[rows] != ref["idx"]).any(axis=1))
        assert bad.size == 0, f"T={T} layer {l}: top-K differs at sampled tokens {rows[bad][:8]}"
        worst = max(worst, assert_close(h.cpu().numpy()[rows], ref["y"], f"T={T} layer {l} output"))
        cache.clear()
    assert torch.equal(h, h_all)
    assert q.moe_read_device_status(ws) == 0
    say(f"  T={T}: layer 0 every token exact top-K; {rows.size} tokens x {L} layers within the bar "
        f"(worst {worst:.2e}); multi-layer call bit-identical to layer-by-layer")
