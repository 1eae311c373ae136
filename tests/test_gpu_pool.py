"""The expert slot pool on the GPU (moe_pool_*): layers run through a pool
whose slots are filled from a pinned host image on router demand must give
bit-identical outputs to the same kernels reading fully resident experts
(same bytes, same kernels), with the hit/miss/eviction counts of the
host-side policy (moeq_poolsim_*) for the same request stream.  Misses,
evictions and the stream ordering between copies and kernels are
exercised with back-to-back acquires that are not synchronised on the host.
"""
import pytest
import torch

import quantized_expert_gemv_router_amd as q
import synth
from quantized_expert_gemv_router_amd import _binding as B
from tests.gpu_util import bf16_dev, say, slot_stride

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_4layers": synth.with_changes(synth.CONFIGS["tiny"], name="tiny_pool", layers=4),
    # real expert size (7,077,888 B), fewer experts so the host image stays small
    "h4096_e16": synth.with_changes(synth.CONFIGS["decode_4bit"], name="pool16", n_experts=16, layers=3),
}


class Setup:
    def __init__(self, cfg):
        self.cfg = cfg
        self.shape = q.Shape.of(cfg)
        self.stride = slot_stride(cfg)
        P, L = cfg.n_slots, cfg.layers
        self.host = torch.empty(L * P * self.stride, dtype=torch.uint8, pin_memory=True)
        hv = self.host.numpy().reshape(L, P, self.stride)
        for l in range(L):
            hv[l] = synth.layer_blobs(cfg, l, self.stride)
        self.resident = q.ExpertTable(self.shape, [torch.from_numpy(hv[l].reshape(-1)).cuda() for l in range(L)],
                                      self.stride)
        self.routers = [bf16_dev(synth.router(cfg, l)) for l in range(L)]
        self.copy = torch.cuda.Stream()
        self.copies = [self.copy] + [torch.cuda.Stream() for _ in range(3)]
        # the same blobs as separate pinned allocations, one per layer
        self.host_layers = []
        for l in range(L):
            t = torch.empty(P * self.stride, dtype=torch.uint8, pin_memory=True)
            t.copy_(self.host[l * P * self.stride:(l + 1) * P * self.stride])
            self.host_layers.append(t)

    def pool(self, n_slots, streams=1):
        P, L = self.cfg.n_slots, self.cfg.layers
        arena = torch.empty(n_slots * self.stride, dtype=torch.uint8, device="cuda")
        table = torch.zeros(L * P, dtype=torch.int64, device="cuda")
        if streams == 1:   # one contiguous host image, one copy stream
            return q.Pool(self.shape, L, arena, n_slots, self.stride, self.host, table, self.copy)
        # per-layer host allocations, misses spread over several copy streams
        return q.Pool(self.shape, L, arena, n_slots, self.stride, self.host_layers, table, self.copies[:streams])

    def token(self, i):
        return bf16_dev(synth.tokens(self.cfg, 500 + i, 1))


@pytest.fixture(scope="module", params=sorted(CASES))
def setup(request):
    say(f"[pool] building {request.param}")
    return Setup(CASES[request.param])


def run_layer(S, experts, layer, x, ws):
    cfg = S.cfg
    idx, w, sw, _ = q.moe_router_topk(S.shape, x, S.routers[layer], cfg.top_k, workspace=ws)
    gu = q.moe_q4_expert_gemv(S.shape, experts, layer, x, idx, cfg.top_k, workspace=ws)
    y = q.moe_swiglu_down_combine(S.shape, experts, layer, gu, idx, w, sw, x, cfg.top_k, workspace=ws)
    return idx, gu, y


@pytest.mark.parametrize("streams", [1, 4])
@pytest.mark.parametrize("extra_layers", [-1, 1])
def test_pool_matches_resident_and_policy(setup, extra_layers, streams):
    S, cfg = setup, setup.cfg
    # two layers' worth of slots forces evictions on every layer; one layer
    # more than the stack keeps recently used experts around (hits)
    n_slots = (2 if extra_layers < 0 else cfg.layers + extra_layers) * (cfg.top_k + cfg.n_shared)
    say(f"[pool] {cfg.name}: {n_slots} slots for {cfg.layers} x {cfg.n_slots} experts, {streams} copy streams")
    pool = S.pool(n_slots, streams)
    sim = q.PoolSim(cfg.layers, cfg.n_slots, n_slots)
    ws = q.new_workspace(S.shape, 1, cfg.top_k)
    ws_r = q.new_workspace(S.shape, 1, cfg.top_k)
    requests = []
    for step in range(6):
        for l in range(cfg.layers):
            x = S.token(step * cfg.layers + l)
            idx_r, gu_r, y_r = run_layer(S, S.resident, l, x, ws_r)
            ids = idx_r.cpu().numpy()[0].tolist() + [cfg.n_experts] * cfg.n_shared
            view = pool.acquire(l, ids)
            sim.acquire(l, ids)
            idx, gu, y = run_layer(S, view, l, x, ws)
            pool.release(l)
            sim.release(l)
            requests.append((l, ids, x, y_r))
            assert torch.equal(idx, idx_r)
            assert torch.equal(gu, gu_r), f"step {step} layer {l}: gate/up differ"
            assert torch.equal(y, y_r), f"step {step} layer {l}: outputs differ"
    st, ss = pool.stats(), sim.stats()
    say(f"  stats {st}")
    assert (st["hits"], st["misses"], st["evictions"]) == (ss["hits"], ss["misses"], ss["evictions"])
    assert st["bytes_copied"] == st["misses"] * cfg.expert_bytes
    assert st["evictions"] > 0 if extra_layers < 0 else st["hits"] > 0
    assert q.moe_read_device_status(ws) == 0

    # the same requests again, acquired and released back to back with no
    # host synchronisation: copies into reused slots must wait for the
    # kernels of the layers that used them
    pool2 = S.pool(n_slots, streams)
    outs = []
    for l, ids, x, _ in requests:
        view = pool2.acquire(l, ids)
        outs.append(run_layer(S, view, l, x, ws)[2].clone())
        pool2.release(l)
    torch.cuda.synchronize()
    for (l, ids, x, y_r), y in zip(requests, outs):
        assert torch.equal(y, y_r), f"unsynchronised replay differs at layer {l}"
    assert pool2.stats() == st
    pool.destroy()
    pool2.destroy()


def test_prefetch_keeps_outputs_bit_identical(setup):
    """Prefetching the previous step's experts of each layer before its
    routing (temporal prefetch) changes which copies happen when, never the
    results: every layer output equals the resident experts' bit for bit,
    and prefetched experts turn into hits."""
    S, cfg = setup, setup.cfg
    n_slots = 2 * (cfg.top_k + cfg.n_shared) + 2
    pool = S.pool(n_slots)
    ws = q.new_workspace(S.shape, 1, cfg.top_k)
    ws_r = q.new_workspace(S.shape, 1, cfg.top_k)
    prev = [None] * cfg.layers
    hits_from_prefetch = 0
    for step in range(5):
        for l in range(cfg.layers):
            x = S.token(700 + step * cfg.layers + l)
            if prev[l] is not None:
                pool.prefetch(l, prev[l])
            idx_r, _, y_r = run_layer(S, S.resident, l, x, ws_r)
            ids = idx_r.cpu().numpy()[0].tolist() + [cfg.n_experts] * cfg.n_shared
            before = pool.stats()["hits"]
            view = pool.acquire(l, ids)
            hits_from_prefetch += pool.stats()["hits"] - before
            _, _, y = run_layer(S, view, l, x, ws)
            pool.release(l)
            assert torch.equal(y, y_r), f"step {step} layer {l}: prefetched pool output differs"
            prev[l] = ids
    torch.cuda.synchronize()
    assert hits_from_prefetch > 0
    pool.destroy()


def test_pool_resident_and_exhausted(setup):
    S, cfg = setup, setup.cfg
    ws = q.new_workspace(S.shape, 1, cfg.top_k)
    pool = S.pool(cfg.layers * cfg.n_slots)
    pool.make_resident()
    for l in range(cfg.layers):
        x = S.token(900 + l)
        _, _, y_r = run_layer(S, S.resident, l, x, ws)
        view = pool.acquire(l, list(range(cfg.n_slots)))
        _, _, y = run_layer(S, view, l, x, ws)
        pool.release(l)
        assert torch.equal(y, y_r)
    st = pool.stats()
    assert st["misses"] == 0 and st["hits"] == cfg.layers * cfg.n_slots
    pool.destroy()

    small = S.pool(cfg.top_k)                        # one short of a layer's experts
    with pytest.raises(q.MoeqError) as ei:
        small.acquire(0, list(range(cfg.top_k)) + [cfg.n_experts])
    assert ei.value.code == B.E_POOL_EXHAUSTED
    assert small.stats()["misses"] == 0
    small.destroy()


def test_pool_refuses_pageable_host_image(setup):
    S, cfg = setup, setup.cfg
    pageable = torch.empty(cfg.layers * cfg.n_slots * S.stride, dtype=torch.uint8)
    arena = torch.empty(4 * S.stride, dtype=torch.uint8, device="cuda")
    table = torch.zeros(cfg.layers * cfg.n_slots, dtype=torch.int64, device="cuda")
    with pytest.raises(q.MoeqError) as ei:
        q.Pool(S.shape, cfg.layers, arena, 4, S.stride, pageable, table, S.copy)
    assert ei.value.code == B.E_INVALID
