"""GPU checks of the persistent decode kernel's diagnostic clock traces
(moeq_stack_block_clock_trace, moeq_stack_clock_trace): an armed launch
gives the same top-K, layer inputs and output bit for bit as an unarmed one,
and every workgroup's per-layer stamps come in the kernel's phase order."""
import numpy as np
import pytest
import torch

import quantized_expert_gemv_router_amd as q
import synth
from tests.gpu_util import bf16_dev, say, slot_stride

pytestmark = pytest.mark.gpu

# block trace events in the order the kernel passes them within a layer:
# start, h polled, own logits published, logits polled, top-K selected by
# wave 0, top-K after its barrier, routed gate/up rows requested, shared
# activations published, routed gate/up dots, routed activations published,
# activations polled, h published (latest wave)
PHASES = [0, 1, 2, 3, 7, 4, 14, 15, 5, 6, 8, 9]
POLL_ROUNDS = [10, 11, 12, 13]


def _stack(E, K, L):
    cfg = synth.with_changes(synth.CONFIGS["stack60_decode"], name=f"trace_e{E}", hidden=256, inter=128,
                             n_experts=E, top_k=K, layers=L)
    shape = q.Shape.of(cfg)
    stride = slot_stride(cfg)
    arenas = []
    for l in range(L):
        a = torch.empty(cfg.n_slots * stride, dtype=torch.uint8, device="cuda")
        synth.device_fill_experts(cfg, l, a.data_ptr(), stride)
        arenas.append(a)
    rt = q.RouterTable([bf16_dev(synth.router(cfg, l)) for l in range(L)])
    torch.cuda.synchronize()
    return cfg, shape, q.ExpertTable(shape, arenas, stride), rt


def _run(cfg, shape, ex, rt, x):
    h = x.clone()
    ws = q.new_workspace(shape, 1, cfg.top_k)
    tk, hk = q.moe_expert_stack_decode(shape, ex, rt, h, cfg.top_k, workspace=ws, trace=True)
    torch.cuda.synchronize()
    assert q.moeq_last_stack_path() == 1
    assert q.moe_read_device_status(ws) == 0
    return tk, hk, h


@pytest.mark.parametrize("E,K", [(8, 2), (512, 3)])
def test_block_clock_trace_order_and_bit_identity(E, K):
    L = 6
    cfg, shape, ex, rt = _stack(E, K, L)
    x = torch.from_numpy(synth.bf16_to_f64(synth.tokens(cfg, 0, 1)).astype(np.float32)).cuda()
    plain = _run(cfg, shape, ex, rt, x)
    nb = torch.cuda.get_device_properties(0).multi_processor_count
    clk = torch.zeros((nb, L, 16), dtype=torch.int64, device="cuda")
    assert q.moeq_stack_block_clock_trace(clk) == 16
    traced = _run(cfg, shape, ex, rt, x)
    for a, b in zip(plain, traced):
        assert torch.equal(a, b)
    c = clk.cpu().numpy()
    t = c[:, :, PHASES]
    assert (t > 0).all(), "a stamp was not written"
    steps = np.diff(t, axis=2)
    bad = np.argwhere(steps < 0)
    assert bad.size == 0, [(int(w), int(l), PHASES[int(i)], PHASES[int(i) + 1]) for w, l, i in bad[:8]]
    # a workgroup starts a layer after its thread 0 has taken the previous layer's activations
    assert (c[:, 1:, 0] >= c[:, :-1, 8]).all()
    assert (c[:, :, POLL_ROUNDS] >= 0).all()
    span = (c[:, :, 9].max(0) - c[:, :, 0].min(0)) * 0.01
    say(f"  E={E} K={K}: {nb} workgroups x {L} layers in phase order; layer spans {np.round(span, 2)} us")


def test_phase_clock_trace_keeps_results():
    L = 6
    cfg, shape, ex, rt = _stack(8, 2, L)
    x = torch.from_numpy(synth.bf16_to_f64(synth.tokens(cfg, 1, 1)).astype(np.float32)).cuda()
    plain = _run(cfg, shape, ex, rt, x)
    clk = torch.zeros((L, 24), dtype=torch.int64, device="cuda")
    n = q.moeq_stack_clock_trace(clk)
    assert n == 24
    traced = _run(cfg, shape, ex, rt, x)
    for a, b in zip(plain, traced):
        assert torch.equal(a, b)
    c = clk.cpu().numpy()
    assert (c[:, 0] > 0).all() and (np.diff(c[:, 0]) > 0).all()   # layer starts, in order
