"""GPU parity of the stacked decode path (persistent launch and per-layer
launches) against the fp64 oracle.

Free-running: the GPU runs all layers from a token, recording each layer's
input h_l and top-K.  The gate is teacher forcing along the GPU's own
trajectory: at every layer the oracle runs the layer on the GPU's input h_l
(fp32, exact in fp64), the GPU's top-K must equal the oracle's exactly and
its h_{l+1} must be within max|gpu - oracle| <= 2e-3 * max|oracle|.  The
distance of the GPU trajectory from the oracle's own free-running one is
reported, not gated: it accumulates every layer's rounding (the activations
are fp16) and, where a logit margin is small, can take another valid
selection.
Oracle-fed: the oracle's h_l is given to the GPU for one layer, and top-K
and h_{l+1} are compared with the oracle's layer on the same input.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_expert_gemv_router_amd as q
import synth
from tests.gpu_util import assert_close, bf16_dev, say, slot_stride

pytestmark = pytest.mark.gpu



def build_stack(cfg, L):
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


def compare_free_running(cfg, L, token_set, traces, gpu_h):
    tk, hk = traces
    idx = tk.cpu().numpy()[:, 0, :]
    hs = hk.cpu().numpy()[:, 0, :].astype(np.float64)
    outs = [hs[l + 1] for l in range(L - 1)] + [np.asarray(gpu_h, dtype=np.float64)]
    K = cfg.top_k
    worst, min_gap = 0.0, np.inf
    for l in range(L):
        exp = oracle.run_layer(cfg, l, hs[l][None, :], want_intermediates=False)
        srt = -np.sort(-exp["logits"][0])
        min_gap = min(min_gap, srt[K - 1] - srt[K])
        assert np.array_equal(idx[l], exp["idx"][0]), (l, idx[l], exp["idx"][0], srt[K - 1] - srt[K])
        worst = max(worst, assert_close(outs[l], exp["y"][0], f"layer {l} output (GPU input)"))
    # drift from the oracle's own trajectory, for the record
    ref = oracle.run_stack(cfg, synth.bf16_to_f64(synth.tokens(cfg, token_set, 1)), layers=L)
    same = 0
    while same < L and np.array_equal(idx[same], ref["idx"][same, 0]):
        same += 1
    last = min(same, L - 1)
    drift = np.abs(hs[last] - ref["h"][last, 0]).max() / np.abs(ref["h"][last, 0]).max()
    say(f"  token set {token_set}: {L} layers, exact top-K on the GPU's inputs (min gap {min_gap:.2e}), "
        f"worst layer output rel err {worst:.2e}; same selections as the free-running oracle for "
        f"{same} layers, h drift at layer {last} {drift:.2e}")


@pytest.mark.parametrize("flags", [0, q.F_STACK_LAYERWISE])
def test_stack_small_shape(flags):
    cfg = synth.with_changes(synth.CONFIGS["stack60_decode"], name="stack_tiny", hidden=256, inter=128,
                             n_experts=8, top_k=2, layers=6)
    say(f"[stack] tiny 6 layers flags={flags}")
    shape, ex, rt = build_stack(cfg, cfg.layers)
    for ts in (0, 1, 2):
        h = torch.from_numpy(synth.bf16_to_f64(synth.tokens(cfg, ts, 1)).astype(np.float32)).cuda()
        ws = q.new_workspace(shape, 1, cfg.top_k)
        traces = q.moe_expert_stack_decode(shape, ex, rt, h, cfg.top_k, flags=flags, workspace=ws,
                                           trace=True)
        assert q.moeq_last_stack_path() == (2 if flags else 1)
        assert q.moe_read_device_status(ws) == 0
        compare_free_running(cfg, cfg.layers, ts, traces, h.cpu().numpy()[0])


@pytest.mark.parametrize("flags", [0, q.F_STACK_LAYERWISE])
def test_stack_all_logits_tied(flags):
    """A zero router ties all 128 logits: more candidates pass the top-K
    threshold than one wave ranks, so the persistent kernel takes its
    block-wide selection; ties go to the lower index (experts 0..K-1,
    weights 1/K)."""
    cfg = synth.with_changes(synth.CONFIGS["stack60_decode"], name="stack_ties", hidden=256, inter=128,
                             n_experts=128, top_k=2, layers=3)
    shape, ex, _ = build_stack(cfg, cfg.layers)
    zero = np.zeros((cfg.n_experts, cfg.hidden), dtype=np.uint16)
    rt = q.RouterTable([bf16_dev(zero) for _ in range(cfg.layers)])
    h = torch.from_numpy(synth.bf16_to_f64(synth.tokens(cfg, 4, 1)).astype(np.float32)).cuda()
    ws = q.new_workspace(shape, 1, cfg.top_k)
    tk, hk = q.moe_expert_stack_decode(shape, ex, rt, h, cfg.top_k, flags=flags, workspace=ws, trace=True)
    assert q.moeq_last_stack_path() == (2 if flags else 1)
    assert q.moe_read_device_status(ws) == 0
    idx = tk.cpu().numpy()[:, 0, :]
    hs = hk.cpu().numpy()[:, 0, :].astype(np.float64)
    outs = [hs[l + 1] for l in range(cfg.layers - 1)] + [h.cpu().numpy()[0].astype(np.float64)]
    for l in range(cfg.layers):
        assert np.array_equal(idx[l], np.arange(cfg.top_k)), (l, idx[l])
        exp = oracle.run_layer(cfg, l, hs[l][None, :], want_intermediates=False, wr=zero)
        assert np.array_equal(exp["idx"][0], np.arange(cfg.top_k))
        assert_close(outs[l], exp["y"][0], f"tied layer {l} output")


def test_stack_2bit_full_width():
    """The 2-bit persistent instantiation (hidden 4096, 512 experts, top-4 +
    1 shared) on three layers, gated per layer along its own trajectory."""
    cfg = synth.with_changes(synth.CONFIGS["decode_2bit"], name="stack_2bit", layers=3, rmsnorm=True)
    say("[stack] 2-bit, 3 layers at full width")
    shape, ex, rt = build_stack(cfg, cfg.layers)
    for ts in (0, 1):
        h = torch.from_numpy(synth.bf16_to_f64(synth.tokens(cfg, ts, 1)).astype(np.float32)).cuda()
        ws = q.new_workspace(shape, 1, cfg.top_k)
        traces = q.moe_expert_stack_decode(shape, ex, rt, h, cfg.top_k, workspace=ws, trace=True)
        assert q.moeq_last_stack_path() == 1
        assert q.moe_read_device_status(ws) == 0
        compare_free_running(cfg, cfg.layers, ts, traces, h.cpu().numpy()[0])


@pytest.fixture(scope="module")
def stack60():
    cfg = synth.CONFIGS["stack60_decode"]
    say(f"[stack60] filling {cfg.layers} layers x {cfg.n_slots} experts on device")
    built = build_stack(cfg, cfg.layers)
    yield cfg, built
    del built
    torch.cuda.empty_cache()


@pytest.mark.parametrize("token_set", [0, 1])
def test_stack60_free_running(stack60, token_set):
    cfg, (shape, ex, rt) = stack60
    say(f"[stack60] persistent, token set {token_set}")
    h = torch.from_numpy(synth.bf16_to_f64(synth.tokens(cfg, token_set, 1)).astype(np.float32)).cuda()
    ws = q.new_workspace(shape, 1, cfg.top_k)
    traces = q.moe_expert_stack_decode(shape, ex, rt, h, cfg.top_k, workspace=ws, trace=True)
    assert q.moeq_last_stack_path() == 1
    assert q.moe_read_device_status(ws) == 0
    compare_free_running(cfg, cfg.layers, token_set, traces, h.cpu().numpy()[0])


@pytest.mark.parametrize("flags,layers", [(0, tuple(range(60))), (q.F_STACK_LAYERWISE, (0, 17, 42, 59))])
def test_stack60_oracle_fed_layers(stack60, flags, layers):
    """Each listed layer runs once on the oracle's own input h_l (rounded to
    the GPU's fp32): top-K must be bit-exact and h_{l+1} within tolerance."""
    cfg, (shape, ex, rt) = stack60
    x64 = synth.bf16_to_f64(synth.tokens(cfg, 7, 1))
    ref = oracle.run_stack(cfg, x64, layers=cfg.layers)
    worst = 0.0
    for l in layers:
        h_in = ref["h"][l].astype(np.float32)           # what the GPU is given
        exp = oracle.run_layer(cfg, l, h_in.astype(np.float64), want_intermediates=False)
        h = torch.from_numpy(h_in).cuda()
        ws = q.new_workspace(shape, 1, cfg.top_k)
        tk, _ = q.moe_expert_stack_decode(shape, ex, rt, h, cfg.top_k, layer0=l, L=1, flags=flags,
                                          workspace=ws, trace=True)
        assert q.moeq_last_stack_path() == (2 if flags else 1)
        assert q.moe_read_device_status(ws) == 0
        assert np.array_equal(tk.cpu().numpy()[0], exp["idx"]), l
        worst = max(worst, assert_close(h.cpu().numpy(), exp["y"], f"layer {l} output"))
    say(f"  {len(layers)} layers flags={flags}: exact top-K on each, worst output rel err {worst:.2e}")


def test_stack60_persistent_is_reproducible(stack60):
    cfg, (shape, ex, rt) = stack60
    x = torch.from_numpy(synth.bf16_to_f64(synth.tokens(cfg, 3, 1)).astype(np.float32)).cuda()
    outs = []
    for _ in range(2):
        h = x.clone()
        q.moe_expert_stack_decode(shape, ex, rt, h, cfg.top_k)
        outs.append(h)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
