"""GPU parity of one decode layer (router -> gate/up -> SwiGLU/down/combine)
against the fp64 oracle on the same seeded inputs.

Bar: top-K indices and order bit-exact; router logits to fp64 rounding;
softmax weights to 1e-6 relative; gate/up and the layer output within
max |gpu - oracle| <= 2e-3 * max |oracle|.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_expert_gemv_router_amd as q
import synth
from tests.gpu_util import assert_close, bf16_dev, experts_for, say

pytestmark = pytest.mark.gpu


def run_and_check(cfg, flags=0, shared_gate=None, x_np=None, x_dev=None, check_gate_up=True):
    say(f"[parity] {cfg.name} H={cfg.hidden} I={cfg.inter} E={cfg.n_experts} S={cfg.n_shared} "
        f"k={cfg.top_k} T={cfg.tokens} bits={cfg.bits} flags={flags}")
    shape, ex = experts_for(cfg)
    if x_dev is None:
        x_np = synth.tokens(cfg, 0) if x_np is None else x_np
        x_dev = bf16_dev(x_np)
        x64 = synth.bf16_to_f64(x_np)
    else:
        x64 = x_dev.double().cpu().numpy()
    wr_np = synth.router(cfg, 0)
    sg_dev = None if shared_gate is None else bf16_dev(shared_gate)
    out = q.moe_layer(shape, ex, 0, x_dev, bf16_dev(wr_np), cfg.top_k, flags, sg_dev)
    torch.cuda.synchronize()
    shape_o = oracle.shape_of(cfg)
    blobs = {}
    _, idx_o, _, _ = oracle.route(shape_o, wr_np, x64, cfg.top_k, flags, shared_gate)
    for e in set(np.unique(idx_o).tolist()) | set(range(cfg.n_experts, cfg.n_slots)):
        blobs[e] = synth.expert_blob(cfg, 0, e)
    ref = oracle.moe_layer(shape_o, blobs, wr_np, x64, cfg.top_k, flags, shared_gate)
    idx = out["idx"].cpu().numpy()
    assert np.array_equal(idx, ref["idx"]), (idx, ref["idx"])
    lg = out["logits"].cpu().numpy()
    np.testing.assert_allclose(lg, ref["logits"], rtol=0, atol=1e-12 * np.abs(ref["logits"]).max())
    np.testing.assert_allclose(out["w"].cpu().numpy(), ref["w"], rtol=1e-6, atol=1e-7)
    if cfg.n_shared:
        np.testing.assert_allclose(out["shared_w"].cpu().numpy(), ref["gamma"], rtol=1e-6)
    e_gu = assert_close(out["gate_up"].cpu().numpy(), ref["gu"], "gate_up") if check_gate_up else 0
    e_y = assert_close(out["y"].cpu().numpy(), ref["y"], "output")
    say(f"  ok: gate_up rel {e_gu:.2e}, output rel {e_y:.2e}")
    return out, ref


@pytest.mark.parametrize("name", ["tiny", "decode_4bit", "decode_2bit", "decode_3bit", "batch16_top10"])
def test_config_parity(name):
    run_and_check(synth.CONFIGS[name])


@pytest.mark.parametrize("H,I,E,k,T", [(256, 128, 8, 2, 1), (384, 256, 37, 5, 3), (4096, 1024, 512, 10, 16),
                                       (8192, 8192, 6, 2, 2)])
def test_three_bit_shapes(H, I, E, k, T):
    """3-bit experts (two bit planes) through the one-token and the batched
    kernels: small, ragged (not multiples of the tiles), the 16-token top-10
    batch, and the widest rows."""
    cfg = synth.with_changes(synth.CONFIGS["decode_3bit"], name=f"q3_{H}_{T}", hidden=H, inter=I, n_experts=E,
                             top_k=k, tokens=T)
    run_and_check(cfg)


def _arena_from_blobs(blobs, stride):
    host = np.zeros((len(blobs), stride), dtype=np.uint8)
    for e, b in enumerate(blobs):
        host[e, :b.size] = b
    return torch.from_numpy(host.reshape(-1)).cuda()


def test_two_bit_values_in_four_bit_container():
    """The same 2-bit values, scales and biases as a 2-bit layer and as a
    4-bit layer: the fp64 oracle gives bit-identical results for both (a
    pinned invariant); the GPU, whose two paths stage and dequantise
    differently, gives the same top-K and both outputs within the bar of it."""
    from tests import blobkit as bk
    H, I, E, K = 256, 128, 8, 2
    rng = np.random.default_rng(77)
    mats = [bk.random_mats(rng, H, I, 2, s_range=(0.004, 0.08), bias_mult=-1.5) for _ in range(E + 1)]
    wr = bk.f64_to_bf16(rng.standard_normal((E, H)) * 0.02)
    x_np = bk.f64_to_bf16(rng.standard_normal((3, H)))
    x64 = bk.bf16_to_f64(x_np)
    outs = {}
    for bits in (2, 4):
        blobs = [bk.build_blob(H, I, bits, m) for m in mats]
        stride = (blobs[0].size + 255) // 256 * 256
        shape = q.Shape(H, I, E, 1, bits, 64)
        ex = q.ExpertTable(shape, [_arena_from_blobs(blobs, stride)], stride)
        out = q.moe_layer(shape, ex, 0, bf16_dev(x_np), bf16_dev(wr), K)
        torch.cuda.synchronize()
        ref = oracle.moe_layer(oracle.Shape(H, I, E, 1, bits, 64), dict(enumerate(blobs)), wr, x64, K)
        outs[bits] = (out, ref)
    assert np.array_equal(outs[2][1]["y"], outs[4][1]["y"])
    for bits in (2, 4):
        out, ref = outs[bits]
        assert np.array_equal(out["idx"].cpu().numpy(), ref["idx"])
        assert_close(out["y"].cpu().numpy(), ref["y"], f"{bits}-bit container output")
    assert torch.equal(outs[2][0]["idx"], outs[4][0]["idx"])


@pytest.mark.parametrize("T", [1, 16])
def test_expert_permutation_invariance(T):
    """Permuting the routed experts (blobs and router rows together): the
    selection maps through the permutation and the layer output is
    bit-identical (each selected expert meets the same arithmetic in the same
    slot)."""
    cfg = synth.with_changes(synth.CONFIGS["tiny"], name="perm", n_experts=32, top_k=4, tokens=T)
    shape = q.Shape.of(cfg)
    stride = (cfg.expert_bytes + 255) // 256 * 256
    host = synth.layer_blobs(cfg, 0, stride)
    perm = np.random.default_rng(5).permutation(cfg.n_experts)   # new index n holds old expert perm[n]
    host_p = host.copy()
    host_p[:cfg.n_experts] = host[perm]
    wr = synth.router(cfg, 0)
    x = bf16_dev(synth.tokens(cfg, 9, T))
    res = []
    for h_, w_ in ((host, wr), (host_p, wr[perm])):
        ex = q.ExpertTable(shape, [torch.from_numpy(h_.reshape(-1)).cuda()], stride)
        res.append(q.moe_layer(shape, ex, 0, x, bf16_dev(np.ascontiguousarray(w_)), cfg.top_k))
    torch.cuda.synchronize()
    a, b = res
    assert np.array_equal(perm[b["idx"].cpu().numpy()], a["idx"].cpu().numpy())
    assert torch.equal(a["y"], b["y"])


@pytest.mark.parametrize("bits", [4, 2])
def test_ragged_shapes(bits):
    """Sizes that are not multiples of the kernels' tiles: 320 = 5*64 hidden,
    192 = 3*64 intermediate, 37 experts, 3 tokens."""
    base = synth.CONFIGS["decode_4bit" if bits == 4 else "decode_2bit"]
    cfg = synth.with_changes(base, name=f"ragged{bits}", hidden=320, inter=192, n_experts=37,
                             top_k=5, tokens=3)
    run_and_check(cfg)


@pytest.mark.parametrize("bits,H,I", [(4, 8192, 4096), (2, 8192, 8192)])
def test_largest_supported_rows(bits, H, I):
    base = synth.CONFIGS["decode_4bit" if bits == 4 else "decode_2bit"]
    cfg = synth.with_changes(base, name=f"max{bits}", hidden=H, inter=I, n_experts=6, top_k=2,
                             tokens=2)
    run_and_check(cfg)


def test_wide_rows_many_tokens():
    """hidden 8192 with 10 tokens: wider than the MFMA router takes, so the
    vector logits kernel runs without its selection tail and the selection
    launch reads logits it already scaled."""
    cfg = synth.with_changes(synth.CONFIGS["decode_4bit"], name="max4t10", hidden=8192, inter=4096,
                             n_experts=6, top_k=2, tokens=10)
    run_and_check(cfg)


@pytest.mark.parametrize("k,E", [(1, 8), (8, 8), (16, 64)])
def test_topk_edges(k, E):
    cfg = synth.with_changes(synth.CONFIGS["tiny"], name=f"k{k}E{E}", n_experts=E, top_k=k, tokens=2)
    run_and_check(cfg)


@pytest.mark.parametrize("T", [2, 12])
def test_many_experts_lds_selection(T):
    """1024 experts, top-16: more logits than the register selection holds
    (8 per lane), so top-K runs from LDS -- in the last router workgroup
    (2 tokens) or in the separate selection launch (12 tokens)."""
    cfg = synth.with_changes(synth.CONFIGS["tiny"], name=f"e1024t{T}", n_experts=1024, top_k=16, tokens=T)
    run_and_check(cfg)


@pytest.mark.parametrize("T", [2, 12])
def test_maximum_experts_and_topk(T):
    """The largest shape the boundary accepts: 4096 routed experts (plus the
    shared one) and top-16, through both LDS selection paths."""
    cfg = synth.with_changes(synth.CONFIGS["tiny"], name=f"emax_t{T}", n_experts=4096, top_k=16, tokens=T)
    run_and_check(cfg)


def test_without_shared_expert():
    cfg = synth.with_changes(synth.CONFIGS["tiny"], name="noshared", n_shared=0, tokens=3)
    run_and_check(cfg)


def test_shared_gate_and_full_softmax():
    cfg = synth.with_changes(synth.CONFIGS["decode_4bit"], name="gated", tokens=2)
    run_and_check(cfg, flags=q.F_NO_RENORM, shared_gate=synth.shared_gate_vector(cfg, 0))


def test_rmsnorm_fp32_input():
    """fp32 input with a large scale and the RMS-norm flag (the stacked-layer form)."""
    cfg = synth.with_changes(synth.CONFIGS["decode_4bit"], name="rms", tokens=4)
    g = torch.Generator().manual_seed(3)
    x = (torch.randn(4, cfg.hidden, generator=g, dtype=torch.float32) * 37.0).cuda()
    run_and_check(cfg, flags=q.F_RMSNORM, x_dev=x)


def test_max_decode_batch_many_chunks():
    """64 tokens (the decode maximum) over 8 experts, top-2: every expert holds
    about 16 (token, slot) pairs, so the batched kernels run several token
    chunks per expert, and the router stages its tokens in several passes."""
    cfg = synth.with_changes(synth.CONFIGS["tiny"], name="t64", tokens=64)
    run_and_check(cfg)


def test_many_tokens_fp32_rmsnorm_gated():
    """20 fp32 tokens with RMS norm, the shared-expert gate and full softmax:
    more tokens than the router stages in one pass at this width (8 fp32
    tokens of 4096), and selection in its own launch."""
    cfg = synth.with_changes(synth.CONFIGS["decode_4bit"], name="rms20", tokens=20)
    g = torch.Generator().manual_seed(5)
    x = (torch.randn(20, cfg.hidden, generator=g, dtype=torch.float32) * 11.0).cuda()
    run_and_check(cfg, flags=q.F_RMSNORM | q.F_NO_RENORM, shared_gate=synth.shared_gate_vector(cfg, 0), x_dev=x)


def test_empty_batch_is_noop():
    cfg = synth.CONFIGS["tiny"]
    shape, ex = experts_for(cfg)
    x = torch.zeros((0, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    wr = bf16_dev(synth.router(cfg, 0))
    ws = q.new_workspace(shape, 1, cfg.top_k)
    idx, w, sw, _ = q.moe_router_topk(shape, x, wr, cfg.top_k, workspace=ws)
    gu = q.moe_q4_expert_gemv(shape, ex, 0, x, idx, cfg.top_k, workspace=ws)
    y = q.moe_swiglu_down_combine(shape, ex, 0, gu, idx, w, sw, x, cfg.top_k, workspace=ws)
    torch.cuda.synchronize()
    assert y.shape == (0, cfg.hidden)


def test_run_to_run_bit_identical():
    cfg = synth.CONFIGS["batch16_top10"]
    shape, ex = experts_for(cfg)
    x = bf16_dev(synth.tokens(cfg, 0))
    wr = bf16_dev(synth.router(cfg, 0))
    a = q.moe_layer(shape, ex, 0, x, wr, cfg.top_k)
    b = q.moe_layer(shape, ex, 0, x, wr, cfg.top_k)
    torch.cuda.synchronize()
    for key in ("idx", "w", "gate_up", "y"):
        assert torch.equal(a[key], b[key]), key


def test_batch_invariance():
    """Token t's output in the 16-token batch equals its output alone, bit for bit."""
    cfg = synth.CONFIGS["batch16_top10"]
    shape, ex = experts_for(cfg)
    x = bf16_dev(synth.tokens(cfg, 0))
    wr = bf16_dev(synth.router(cfg, 0))
    full = q.moe_layer(shape, ex, 0, x, wr, cfg.top_k)
    for t in (0, 7, 15):
        one = q.moe_layer(shape, ex, 0, x[t:t + 1].contiguous(), wr, cfg.top_k)
        torch.cuda.synchronize()
        assert torch.equal(one["idx"][0], full["idx"][t])
        assert torch.equal(one["y"][0], full["y"][t]), t


def test_given_ids_with_duplicates_and_bad_id():
    """Caller-supplied routing: a repeated expert is computed per slot; an id
    outside [0, E) sets the status word and leaves the other slots intact."""
    cfg = synth.with_changes(synth.CONFIGS["decode_4bit"], name="given", tokens=2)
    shape, ex = experts_for(cfg)
    x_np = synth.tokens(cfg, 0, 2)
    x = bf16_dev(x_np)
    idx = torch.tensor([[5, 5, 100], [7, 600, 5]], dtype=torch.int32, device="cuda")
    ws = q.new_workspace(shape, 2, 3)
    gu = torch.zeros((2, 4, 2, cfg.inter), dtype=torch.float32, device="cuda")
    q.moe_q4_expert_gemv(shape, ex, 0, x, idx, 3, workspace=ws, gate_up=gu)
    status = q.moe_read_device_status(ws)
    assert status == 1
    gu = gu.cpu().numpy()
    x64 = synth.bf16_to_f64(x_np)
    sh = oracle.shape_of(cfg)
    for t, slot, e in [(0, 0, 5), (0, 1, 5), (0, 2, 100), (1, 0, 7), (1, 2, 5), (0, 3, 512), (1, 3, 512)]:
        g, u, _, _ = oracle.expert_ffn(sh, synth.expert_blob(cfg, 0, e), x64[t])
        assert_close(gu[t, slot, 0], g, f"gate t{t} s{slot}")
        assert_close(gu[t, slot, 1], u, f"up t{t} s{slot}")
    assert np.all(gu[1, 1] == 0)
    assert q.moe_read_device_status(ws) == 0


def test_layer_calls_replay_in_a_hip_graph():
    """The three calls of a one-token layer captured in a HIP graph: every
    replay, with eager launches and synchronisations between the replays,
    equals the eager result bit for bit (top-K, weights, gate/up, output)."""
    cfg = synth.CONFIGS["decode_4bit"]
    say(f"[graph] {cfg.name}: capture the three calls, replay six times")
    shape, ex = experts_for(cfg)
    wr = bf16_dev(synth.router(cfg, 0))
    xs = [bf16_dev(synth.tokens(cfg, t)) for t in range(3)]
    ws = q.new_workspace(shape, 1, cfg.top_k)
    eager = [q.moe_layer(shape, ex, 0, x, wr, cfg.top_k, workspace=ws) for x in xs]
    torch.cuda.synchronize()
    x_in = xs[0].clone()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        out = q.moe_layer(shape, ex, 0, x_in, wr, cfg.top_k, workspace=ws, stream=s)
    torch.cuda.synchronize()
    for rep in range(6):
        t = rep % 3
        x_in.copy_(xs[t])
        g.replay()
        torch.cuda.synchronize()
        for key in ("idx", "w", "gate_up", "y"):
            assert torch.equal(out[key], eager[t][key]), (rep, key)
        other = q.moe_layer(shape, ex, 0, xs[(t + 1) % 3], wr, cfg.top_k, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(other["y"], eager[(t + 1) % 3]["y"]), rep
