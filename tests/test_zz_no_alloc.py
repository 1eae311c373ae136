"""The allocation-free stack decode (moe_expert_stack_decode_noalloc, static
scratch) against the workspace entry point (moe_expert_stack_decode): both
run the same kernels, so top-K, the per-layer inputs and the output must be
bit-identical.  Two calls in a row on the shared scratch, the second with a
smaller input, for the persistent and the per-layer paths."""
import numpy as np
import pytest
import torch

import quantized_expert_gemv_router_amd as q
import synth
from tests.gpu_util import bf16_dev, say, slot_stride

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


def compare(cfg, L, flags, token_set):
    shape, ex, rt = build(cfg, L)
    K = cfg.top_k
    x = torch.from_numpy(synth.bf16_to_f64(synth.tokens(cfg, token_set, 1)).astype(np.float32)).cuda()
    h_ref = x.clone()
    ws = q.new_workspace(shape, 1, K)
    tk_ref, hk_ref = q.moe_expert_stack_decode(shape, ex, rt, h_ref, K, flags=flags, workspace=ws, trace=True)
    path_ref = q.moeq_last_stack_path()
    h = x.clone()
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    tk, hk = q.moe_expert_stack_decode_noalloc(shape, ex, rt, h, K, flags=flags, trace=True, status=status)
    torch.cuda.synchronize()
    assert q.moeq_last_stack_path() == path_ref
    assert q.moe_read_device_status(ws) == 0
    assert int(status.item()) == 0
    assert torch.equal(tk, tk_ref)
    assert torch.equal(hk, hk_ref)
    assert torch.equal(h, h_ref)
    say(f"  {cfg.name} L={L} flags={flags}: noalloc == workspace call (path {path_ref})")


@pytest.mark.parametrize("flags", [0, q.F_STACK_LAYERWISE])
def test_noalloc_matches_workspace_call_twice(flags):
    big = synth.with_changes(synth.CONFIGS["decode_2bit"], name="noalloc_2bit", layers=3, rmsnorm=True)
    small = synth.with_changes(synth.CONFIGS["stack60_decode"], name="noalloc_tiny", hidden=256, inter=128,
                               n_experts=8, top_k=2, layers=2)
    say(f"[noalloc] flags={flags}")
    compare(big, big.layers, flags, 0)
    compare(small, small.layers, flags, 1)
