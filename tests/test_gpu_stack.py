"""GPU parity of the stacked decode path (persistent launch and per-layer
launches) against the fp64 oracle.

Free-running: the GPU runs all layers from a token, recording each layer's
input h_l and top-K.  The gate is teacher forcing along the GPU's own
trajectory: at every layer the oracle runs the layer on the GPU's input h_l
(fp32, exact in fp64), the GPU's top-K must equal the oracle's and its
h_{l+1} must be within max|gpu - oracle| <= 2e-3 * max|oracle|.  "Equal"
allows one thing only: the persistent launch hands logits over rounded to a
36-bit significand, so two distinct logits within 2^-35 of each other
(relative to the largest) may swap ranks (topk_matches); exact ties and
every wider gap must match exactly.  No seeded workload here has a gap
that small.  The
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
from tests.gpu_util import assert_close, bf16_dev, say, slot_stride, topk_matches

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
        gap = srt[K - 1] - srt[K] if K < len(srt) else np.inf   # every expert selected: no margin
        min_gap = min(min_gap, gap)
        assert topk_matches(idx[l], exp["idx"][0], exp["logits"][0]), (l, idx[l], exp["idx"][0], gap)
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


def test_stack_small_shape_delay_injection():
    """Small shape (8 experts: most workgroups own no router row): the
    delay-injection build equals the plain launch bit for bit."""
    cfg = synth.with_changes(synth.CONFIGS["stack60_decode"], name="stack_tiny_jit", hidden=256, inter=128,
                             n_experts=8, top_k=2, layers=6)
    shape, ex, rt = build_stack(cfg, cfg.layers)
    for ts in (0, 1, 2):
        x = torch.from_numpy(synth.bf16_to_f64(synth.tokens(cfg, ts, 1)).astype(np.float32)).cuda()
        res = []
        for flags in (0, q.F_STACK_JITTER):
            h = x.clone()
            ws = q.new_workspace(shape, 1, cfg.top_k)
            tk, hk = q.moe_expert_stack_decode(shape, ex, rt, h, cfg.top_k, flags=flags, workspace=ws, trace=True)
            assert q.moeq_last_stack_path() == 1
            assert q.moe_read_device_status(ws) == 0
            res.append((tk, hk, h))
        torch.cuda.synchronize()
        for a, b in zip(*res):
            assert torch.equal(a, b)


def _tiny_stack_cfg():
    return synth.with_changes(synth.CONFIGS["stack60_decode"], name="stack_tiny", hidden=256, inter=128,
                              n_experts=8, top_k=2, layers=6)


def _token(cfg, ts):
    return torch.from_numpy(synth.bf16_to_f64(synth.tokens(cfg, ts, 1)).astype(np.float32)).cuda()


def test_stack_launches_share_one_workspace():
    """Persistent launches of different lengths and first layers, one after
    another on one workspace, equal the same launches on fresh workspaces
    bit for bit: words an earlier launch left in the workspace (other
    launch numbers in their tags) never satisfy a later launch's polls."""
    cfg = _tiny_stack_cfg()
    say("[stack] tiny: eight launches of 1-6 layers on one workspace")
    shape, ex, rt = build_stack(cfg, cfg.layers)
    ws = q.new_workspace(shape, 1, cfg.top_k)
    for i, (l0, L) in enumerate([(0, 2), (2, 1), (3, 1), (4, 2), (0, 6), (5, 1), (1, 3), (0, 1)]):
        x = _token(cfg, 10 + i)
        h1, h2 = x.clone(), x.clone()
        tk1, hk1 = q.moe_expert_stack_decode(shape, ex, rt, h1, cfg.top_k, layer0=l0, L=L, workspace=ws, trace=True)
        assert q.moeq_last_stack_path() == 1
        assert q.moe_read_device_status(ws) == 0
        fresh = q.new_workspace(shape, 1, cfg.top_k)
        tk2, hk2 = q.moe_expert_stack_decode(shape, ex, rt, h2, cfg.top_k, layer0=l0, L=L, workspace=fresh,
                                             trace=True)
        assert q.moe_read_device_status(fresh) == 0
        assert torch.equal(tk1, tk2) and torch.equal(hk1, hk2) and torch.equal(h1, h2), (l0, L)


@pytest.mark.parametrize("name,layer0,L", [("tiny", 1, 4), ("decode_4bit", 0, 1)])
def test_stack_launch_replays_in_a_hip_graph(name, layer0, L):
    """A persistent launch captured in a HIP graph: every replay, with eager
    launches on the same workspace and synchronisations between the replays,
    equals the eager result bit for bit."""
    if name == "tiny":
        cfg, flags = _tiny_stack_cfg(), 0
    else:   # one layer of the one-token configuration, its input taken as is
        cfg, flags = synth.CONFIGS[name], q.F_STACK_NO_NORM
    say(f"[stack] {name}: capture layers [{layer0}, {layer0 + L}), replay six times")
    shape, ex, rt = build_stack(cfg, layer0 + L)
    ws = q.new_workspace(shape, 1, cfg.top_k)
    xs = [_token(cfg, t) for t in range(3)]
    eager = []
    for x in xs:
        h = x.clone()
        q.moe_expert_stack_decode(shape, ex, rt, h, cfg.top_k, layer0=layer0, L=L, flags=flags, workspace=ws)
        assert q.moeq_last_stack_path() == 1
        eager.append(h)
    torch.cuda.synchronize()
    assert q.moe_read_device_status(ws) == 0
    h_in = xs[0].clone()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        q.moe_expert_stack_decode(shape, ex, rt, h_in, cfg.top_k, layer0=layer0, L=L, flags=flags, workspace=ws,
                                  stream=s)
    torch.cuda.synchronize()
    for rep in range(6):
        t = rep % 3
        h_in.copy_(xs[t])
        g.replay()
        torch.cuda.synchronize()
        assert q.moe_read_device_status(ws) == 0, rep
        assert torch.equal(h_in, eager[t]), rep
        other = xs[(t + 1) % 3].clone()
        q.moe_expert_stack_decode(shape, ex, rt, other, cfg.top_k, layer0=layer0, L=L, flags=flags, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(other, eager[(t + 1) % 3]), rep


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


@pytest.mark.parametrize("flags", [0, q.F_STACK_LAYERWISE])
def test_stack_near_tied_logits(flags):
    """Four experts whose logits differ only in their low bits: experts 3 and
    5 share one router row, expert 9 has that row one bf16 ulp larger in
    magnitude at the input's smallest nonzero component (a logit higher by
    ~1e-8 relative) and expert 17 one ulp smaller.  Their logits agree to far
    more bits than the persistent kernel's selection network compares (its
    keys keep 17 significand bits), so it must defer to the full-key rounds;
    the selection must still be the oracle's: expert 9, then the lower index
    of the equal pair."""
    from tests import blobkit as bk
    cfg = synth.with_changes(synth.CONFIGS["stack60_decode"], name="stack_near_ties", hidden=256, inter=128,
                             n_experts=128, top_k=2, layers=1)
    shape, ex, _ = build_stack(cfg, 1)
    x = synth.bf16_to_f64(synth.tokens(cfg, 6, 1))
    rng = np.random.default_rng(11)
    wr = bk.f64_to_bf16(rng.standard_normal((cfg.n_experts, cfg.hidden)) * 0.02)
    row = bk.f64_to_bf16(np.sign(x[0]) * 0.05)
    nz = np.flatnonzero(x[0] != 0)
    j = nz[np.argmin(np.abs(x[0][nz]))]
    up, down = row.copy(), row.copy()
    up[j] += 1     # bf16 is sign-magnitude: one ulp more magnitude, same sign as x_j
    down[j] -= 1
    for e, r in ((3, row), (5, row), (9, up), (17, down)):
        wr[e] = r
    rt = q.RouterTable([bf16_dev(wr)])
    h = torch.from_numpy(x.astype(np.float32)).cuda()
    ws = q.new_workspace(shape, 1, cfg.top_k)
    tk, hk = q.moe_expert_stack_decode(shape, ex, rt, h, cfg.top_k, flags=flags, workspace=ws, trace=True)
    assert q.moeq_last_stack_path() == (2 if flags else 1)
    assert q.moe_read_device_status(ws) == 0
    exp = oracle.run_layer(cfg, 0, x, want_intermediates=False, wr=wr)
    lg = exp["logits"][0][[3, 5, 9, 17]]
    assert lg[2] > lg[0] == lg[1] > lg[3]
    assert (lg.max() - lg.min()) / abs(lg.max()) < 2.0 ** -20, lg
    assert np.array_equal(exp["idx"][0], [9, 3]), exp["idx"][0]
    assert np.array_equal(tk.cpu().numpy()[0, 0], exp["idx"][0]), (tk.cpu().numpy()[0, 0], exp["idx"][0])
    assert_close(h.cpu().numpy()[0].astype(np.float64), exp["y"][0], "near-tied layer output")


@pytest.mark.parametrize("flags", [0, q.F_STACK_LAYERWISE])
def test_stack_top4_boundary_near_tie(flags):
    """Top-4 whose fourth and fifth logits differ only in their low bits:
    experts 40, 50, 60 take clearly separated rows, expert 20 a fourth row
    and expert 30 the same row one bf16 ulp larger in magnitude at the
    input's smallest nonzero component.  Both sit in the first logit slot,
    so their truncated keys are identical: the four best prefixes decrease
    strictly, and only the count of elements at or above the fourth prefix
    (five, not four) sends the selection network to the full-key rounds.
    The selection must be the oracle's: 40, 50, 60, then 30 (not 20)."""
    from tests import blobkit as bk
    cfg = synth.with_changes(synth.CONFIGS["decode_2bit"], name="stack_top4_tie", hidden=256, inter=128,
                             n_experts=128, top_k=4, layers=1, rmsnorm=True)
    shape, ex, _ = build_stack(cfg, 1)
    x = synth.bf16_to_f64(synth.tokens(cfg, 7, 1))
    rng = np.random.default_rng(12)
    wr = bk.f64_to_bf16(rng.standard_normal((cfg.n_experts, cfg.hidden)) * 0.02)
    nz = np.flatnonzero(x[0] != 0)
    j = nz[np.argmin(np.abs(x[0][nz]))]
    for e, a in ((40, 0.05), (50, 0.045), (60, 0.04), (20, 0.035)):
        wr[e] = bk.f64_to_bf16(np.sign(x[0]) * a)
    wr[30] = wr[20]
    wr[30, j] += 1   # bf16 is sign-magnitude: one ulp more magnitude, same sign as x_j
    rt = q.RouterTable([bf16_dev(wr)])
    h = torch.from_numpy(x.astype(np.float32)).cuda()
    ws = q.new_workspace(shape, 1, cfg.top_k)
    tk, hk = q.moe_expert_stack_decode(shape, ex, rt, h, cfg.top_k, flags=flags, workspace=ws, trace=True)
    assert q.moeq_last_stack_path() == (2 if flags else 1)
    assert q.moe_read_device_status(ws) == 0
    exp = oracle.run_layer(cfg, 0, x, want_intermediates=False, wr=wr)
    lg = exp["logits"][0]
    assert lg[30] > lg[20] and (lg[30] - lg[20]) / abs(lg[30]) < 2.0 ** -20, (lg[30], lg[20])
    assert np.array_equal(exp["idx"][0], [40, 50, 60, 30]), exp["idx"][0]
    assert np.array_equal(tk.cpu().numpy()[0, 0], exp["idx"][0]), (tk.cpu().numpy()[0, 0], exp["idx"][0])
    assert_close(h.cpu().numpy()[0].astype(np.float64), exp["y"][0], "top-4 near-tie layer output")


@pytest.mark.parametrize("bits,K", [(4, 1), (4, 2), (4, 3), (2, 4)])
def test_stack_selection_sweep(bits, K):
    """Seeded sweep of the persistent kernel's top-K over 512 experts: per
    case a fresh token and router in which K + 2 experts get strong rows
    (a multiple of sign(x)), each either a strength of its own, an exact
    copy of an earlier strong row (an exact tie) or such a copy one bf16
    ulp up or down at a random nonzero component (a near-tie far below the
    selection network's 17-bit keys).  The ties fall at random ranks, at
    and across the top-K boundary, so the network, its certificate and the
    full-key rounds all decide some cases; every selection must be the
    oracle's, and the layer output within the bar."""
    from tests import blobkit as bk
    cfg = synth.with_changes(synth.CONFIGS[f"decode_{bits}bit"], name=f"stack_sweep{bits}_{K}", hidden=256,
                             inter=128, n_experts=512, top_k=K, layers=1, rmsnorm=True)
    shape, ex, _ = build_stack(cfg, 1)
    rng = np.random.default_rng(1000 * bits + K)
    n_ties = 0
    for case in range(24):
        x = synth.bf16_to_f64(synth.tokens(cfg, 100 + case, 1))
        wr = bk.f64_to_bf16(rng.standard_normal((cfg.n_experts, cfg.hidden)) * 0.02)
        nz = np.flatnonzero(x[0] != 0)
        strong = rng.choice(cfg.n_experts, K + 2, replace=False)
        for i, e in enumerate(strong):
            kind = rng.integers(4) if i > 0 else 0
            if kind == 0:
                wr[e] = bk.f64_to_bf16(np.sign(x[0]) * rng.choice([0.03, 0.035, 0.04, 0.045, 0.05]))
            else:
                wr[e] = wr[strong[rng.integers(i)]]
                j = rng.choice(nz)
                if kind == 2:   # bf16 is sign-magnitude: one ulp of magnitude up
                    wr[e, j] += 1
                elif kind == 3:   # or down
                    wr[e, j] -= 1
        rt = q.RouterTable([bf16_dev(wr)])
        h = torch.from_numpy(x.astype(np.float32)).cuda()
        ws = q.new_workspace(shape, 1, K)
        tk, _ = q.moe_expert_stack_decode(shape, ex, rt, h, K, workspace=ws, trace=True)
        assert q.moeq_last_stack_path() == 1
        assert q.moe_read_device_status(ws) == 0
        exp = oracle.run_layer(cfg, 0, x, want_intermediates=False, wr=wr)
        srt = -np.sort(-exp["logits"][0])
        n_ties += int(np.min(np.abs(np.diff(srt[:K + 1])) / np.abs(srt[0])) < 2.0 ** -17)
        assert np.array_equal(tk.cpu().numpy()[0, 0], exp["idx"][0]), (case, tk.cpu().numpy()[0, 0], exp["idx"][0])
        assert_close(h.cpu().numpy()[0].astype(np.float64), exp["y"][0], f"sweep case {case}")
    say(f"  {bits}-bit top-{K}: 24 cases, {n_ties} with a tie or near-tie among the K + 1 best")
    assert n_ties >= 6


@pytest.mark.parametrize("name", ["tiny", "decode_4bit", "decode_2bit", "decode_3bit"])
def test_single_layer_no_norm_matches_oracle(name):
    """One layer through the stack entry with MOEQ_F_STACK_NO_NORM (the layer
    input taken as is, as the one-layer calls without the norm flag): the
    persistent launch and the per-layer launches both give the oracle's
    exact top-K and an output within the bar, for the configured one-token
    layers (bf16 token, no norm, gamma = 1)."""
    cfg = synth.CONFIGS[name]
    shape, ex, rt = build_stack(cfg, 2)
    for ts in (0, 1):
        x64 = synth.bf16_to_f64(synth.tokens(cfg, ts, 1))
        for layer in (0, 1):
            exp = oracle.run_layer(cfg, layer, x64, want_intermediates=False)
            for flags in (q.F_STACK_NO_NORM, q.F_STACK_NO_NORM | q.F_STACK_LAYERWISE):
                h = torch.from_numpy(x64.astype(np.float32)).cuda()
                ws = q.new_workspace(shape, 1, cfg.top_k)
                tk, _ = q.moe_expert_stack_decode(shape, ex, rt, h, cfg.top_k, layer0=layer, L=1, flags=flags,
                                                  workspace=ws, trace=True)
                assert q.moeq_last_stack_path() == (2 if flags & q.F_STACK_LAYERWISE else 1)
                assert q.moe_read_device_status(ws) == 0
                assert topk_matches(tk.cpu().numpy()[0, 0], exp["idx"][0], exp["logits"][0]), (name, ts, layer, flags)
                assert_close(h.cpu().numpy(), exp["y"], f"{name} layer {layer} flags {flags}")


def _width_cfg(base, bits):
    src = synth.CONFIGS[{4: "decode_4bit", 3: "decode_3bit", 2: "decode_2bit"}[bits]]
    return synth.with_changes(base, bits=bits, s_lo=src.s_lo, s_hi=src.s_hi, bias_mult=src.bias_mult)


def test_stack_mixed_widths_full_width():
    """A stack whose layers hold 4-, 2- and 3-bit experts (hidden 4096, 512
    experts, top-3 + 1 shared): moe_expert_stack_decode_mixed runs each run
    of equal width as one stack call (each a persistent launch: every width
    has an instantiation at this shape); every layer is checked against the
    oracle of its own width on the GPU's input (teacher forcing)."""
    base = synth.with_changes(synth.CONFIGS["stack60_decode"], name="mixed", layers=5)
    bits = [4, 2, 2, 3, 4]
    shape = q.Shape.of(base)
    arenas = []
    for l, b in enumerate(bits):
        cl = _width_cfg(base, b)
        stride = slot_stride(cl)
        a = torch.empty(cl.n_slots * stride, dtype=torch.uint8, device="cuda")
        synth.device_fill_experts(cl, l, a.data_ptr(), stride)
        arenas.append((a, stride))
    ptrs = torch.tensor([a.data_ptr() + e * st for a, st in arenas for e in range(base.n_slots)],
                        dtype=torch.int64, device="cuda")
    ex = q.ExpertTable.from_pointers(ptrs, len(bits))
    rt = q.RouterTable([bf16_dev(synth.router(base, l)) for l in range(len(bits))])
    torch.cuda.synchronize()
    for ts in (0, 1):
        h = torch.from_numpy(synth.bf16_to_f64(synth.tokens(base, ts, 1)).astype(np.float32)).cuda()
        ws = q.new_workspace(shape, 1, base.top_k)
        tk, hk = q.moe_expert_stack_decode_mixed(shape, bits, ex, rt, h, base.top_k, workspace=ws, trace=True)
        assert q.moeq_last_stack_path() == 1
        assert q.moe_read_device_status(ws) == 0
        hs = hk.cpu().numpy()[:, 0, :].astype(np.float64)
        outs = [hs[l + 1] for l in range(len(bits) - 1)] + [h.cpu().numpy()[0].astype(np.float64)]
        for l, b in enumerate(bits):
            exp = oracle.run_layer(_width_cfg(base, b), l, hs[l][None, :], want_intermediates=False)
            assert topk_matches(tk.cpu().numpy()[l, 0], exp["idx"][0], exp["logits"][0]), (ts, l, b)
            assert_close(outs[l], exp["y"][0], f"mixed stack layer {l} ({b}-bit)")


@pytest.mark.parametrize("flags", [0, q.F_STACK_LAYERWISE])
@pytest.mark.parametrize("bits,E,K", [(4, 100, 3), (4, 449, 1), (4, 3, 3), (2, 77, 4), (3, 300, 2), (2, 512, 1)])
def test_stack_ragged_expert_counts(bits, E, K, flags):
    """Expert counts that are not a multiple of the 64-lane wave (the
    selection's last logit slot partly empty), one selected expert, every
    expert selected (K = E), and top-4 (past the selection network, rounds
    of wave maxima) at a ragged count: three layers, gated per layer along
    the GPU's own trajectory."""
    cfg = synth.with_changes(synth.CONFIGS[f"decode_{bits}bit"], name=f"stack_r{bits}_{E}_{K}", hidden=256,
                             inter=128, n_experts=E, top_k=K, layers=3, rmsnorm=True)
    say(f"[stack] {bits}-bit E={E} K={K} flags={flags}")
    shape, ex, rt = build_stack(cfg, cfg.layers)
    for ts in (0, 1):
        h = torch.from_numpy(synth.bf16_to_f64(synth.tokens(cfg, ts, 1)).astype(np.float32)).cuda()
        ws = q.new_workspace(shape, 1, cfg.top_k)
        traces = q.moe_expert_stack_decode(shape, ex, rt, h, cfg.top_k, flags=flags, workspace=ws, trace=True)
        assert q.moeq_last_stack_path() == (2 if flags else 1)
        assert q.moe_read_device_status(ws) == 0
        compare_free_running(cfg, cfg.layers, ts, traces, h.cpu().numpy()[0])


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


def test_stack_3bit_full_width():
    """The 3-bit persistent instantiation (two bit planes; hidden 4096, 512
    experts, top-4 + 1 shared) on three layers, gated per layer along its
    own trajectory."""
    cfg = synth.with_changes(synth.CONFIGS["decode_3bit"], name="stack_3bit", layers=3, rmsnorm=True)
    say("[stack] 3-bit, 3 layers at full width")
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
        assert topk_matches(tk.cpu().numpy()[0, 0], exp["idx"][0], exp["logits"][0]), l
        worst = max(worst, assert_close(h.cpu().numpy(), exp["y"], f"layer {l} output"))
    say(f"  {len(layers)} layers flags={flags}: exact top-K on each, worst output rel err {worst:.2e}")


def test_stack60_delay_injection_is_bit_identical(stack60):
    """The delay-injection build of the persistent kernel (every wave sleeps a
    pseudo-random 0..~13 us before each hand-off publish) gives top-K, layer
    inputs and output bit-identical to the plain launch over all 60 layers:
    the tagged hand-offs order the layers by themselves."""
    cfg, (shape, ex, rt) = stack60
    for ts in (5, 6):
        x = torch.from_numpy(synth.bf16_to_f64(synth.tokens(cfg, ts, 1)).astype(np.float32)).cuda()
        res = []
        for flags in (0, q.F_STACK_JITTER):
            h = x.clone()
            ws = q.new_workspace(shape, 1, cfg.top_k)
            tk, hk = q.moe_expert_stack_decode(shape, ex, rt, h, cfg.top_k, flags=flags, workspace=ws, trace=True)
            assert q.moeq_last_stack_path() == 1
            assert q.moe_read_device_status(ws) == 0
            res.append((tk, hk, h))
        torch.cuda.synchronize()
        for a, b in zip(*res):
            assert torch.equal(a, b)


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
