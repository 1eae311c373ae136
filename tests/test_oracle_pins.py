"""Pins for the fp64 oracle: closed forms, brute force and special cases.

Each test checks the oracle against something other than itself: a value
the pages print, a closed form of the definition, a brute-force search, or a
special case that reduces to a library routine applied to matrices decoded
by a different (vectorised) decoder in tests/blobkit.py.  A plausible slip
in the oracle (a dropped bias term, a wrong shift, a transposed section, a
wrong tie rule, an un-normalised softmax) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
import synth
from tests import blobkit as bk

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def shape(H, I, E=4, S=1, bits=4, G=64):
    return oracle.Shape(H, I, E, S, bits, G)


# ------------------------------------------------------------------ layout

def test_expert_bytes_match_page_figure():
    """Flash-MoE ('SSD Expert Streaming'): about 6.75 MB per 4-bit expert.
    With H=4096, I=1024, group 64 and a bf16 scale + bf16 bias per group the
    layout is exactly 6.75 * 2^20 bytes."""
    fig = json.load(open(os.path.join(GOLD, "page_figures.json")))
    H = fig["hidden"]["value"]
    b4 = oracle.expert_bytes(shape(H, 1024, bits=4))
    assert b4 == 7_077_888 == int(fig["expert_size_mb"]["value"] * 2 ** 20)
    assert oracle.expert_bytes(shape(H, 1024, bits=2)) == 3_932_160
    # 3-bit: 3 bits per value (two planes) + the same scale/bias words
    assert oracle.expert_bytes(shape(H, 1024, bits=3)) == 3 * (H * 1024 * 3 // 8 + H * 1024 // 64 * 4) == 5_505_024
    assert oracle.expert_bytes(shape(256, 128, bits=4)) == 55_296
    for name, cfg in synth.CONFIGS.items():
        assert oracle.expert_bytes(oracle.shape_of(cfg)) == cfg.expert_bytes, name


# --------------------------------------------------------- dequant + GEMV

@pytest.mark.parametrize("bits", [4, 3, 2])
@pytest.mark.parametrize("sec", [0, 1, 2])
def test_zero_values_give_bias_times_group_sum(bits, sec):
    """All-zero packed values: y_r = sum_g b_{r,g} * X_g, X_g = sum of x over group g."""
    rng = np.random.default_rng(1)
    H, I = 192, 128
    mats = bk.random_mats(rng, H, I, bits)
    mats = {k: (np.zeros_like(q), s, b) for k, (q, s, b) in mats.items()}
    blob = bk.build_blob(H, I, bits, mats)
    sh = shape(H, I, bits=bits)
    name = ("gate", "up", "down")[sec]
    cols = I if sec == 2 else H
    x = rng.standard_normal(cols)
    y = oracle.section_matvec(sh, blob, sec, x)
    X = x.reshape(-1, 64).sum(axis=1)
    expect = bk.bf16_to_f64(mats[name][2]) @ X
    np.testing.assert_allclose(y, expect, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_one_hot_input_recovers_dequantised_column(bits):
    """x = e_j: y_r = scale_{r, j//64} * q_{r,j} + bias_{r, j//64}."""
    rng = np.random.default_rng(2)
    H, I = 256, 128
    mats = bk.random_mats(rng, H, I, bits)
    blob = bk.build_blob(H, I, bits, mats)
    sh = shape(H, I, bits=bits)
    for sec, name in enumerate(("gate", "up", "down")):
        q, s, b = mats[name]
        cols = q.shape[1]
        for j in (0, 1, 7, 8, 15, 16, 63, 64, 101, cols - 1):
            x = np.zeros(cols)
            x[j] = 1.0
            y = oracle.section_matvec(sh, blob, sec, x)
            expect = bk.bf16_to_f64(s[:, j // 64]) * q[:, j] + bk.bf16_to_f64(b[:, j // 64])
            np.testing.assert_array_equal(y, expect)


def test_hand_worked_row():
    """One 64-wide row with values 0..15 repeated four times, scale 0.5,
    bias -4, x = 1: sum_j (0.5 q_j - 4) = 0.5 * 4 * 120 - 256 = -16."""
    H, I = 64, 64
    q = np.tile(np.arange(16), 4)[None, :].repeat(I, axis=0)
    s = bk.f64_to_bf16(np.full((I, 1), 0.5))
    b = bk.f64_to_bf16(np.full((I, 1), -4.0))
    qd = np.zeros((H, I), dtype=np.int64)
    sd = bk.f64_to_bf16(np.zeros((H, 1)))
    blob = bk.build_blob(H, I, 4, {"gate": (q, s, b), "up": (q, s, b), "down": (qd, sd, sd)})
    y = oracle.section_matvec(shape(H, I), blob, 0, np.ones(H))
    assert np.all(y == -16.0)


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_constant_values(bits):
    """Every packed value = c: y_r = sum_g (c * s_{r,g} + b_{r,g}) * X_g."""
    rng = np.random.default_rng(3)
    H, I = 128, 64
    c = (1 << bits) - 2
    mats = bk.random_mats(rng, H, I, bits)
    mats = {k: (np.full_like(q, c), s, b) for k, (q, s, b) in mats.items()}
    blob = bk.build_blob(H, I, bits, mats)
    x = rng.standard_normal(H)
    y = oracle.section_matvec(shape(H, I, bits=bits), blob, 1, x)
    _, s, b = mats["up"]
    X = x.reshape(-1, 64).sum(axis=1)
    expect = (c * bk.bf16_to_f64(s) + bk.bf16_to_f64(b)) @ X
    np.testing.assert_allclose(y, expect, rtol=1e-12)


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_three_algebraic_forms_agree(bits):
    """Explicit dequantise-then-dot (oracle) == the FMA form on the Flash-MoE
    page, sum_j fma(q_j, s*x_j, b*x_j) ('Noyau de déquantification optimisé
    FMA') == the per-group form s*sum(q x) + b*sum(x), to fp64 rounding."""
    cfg = synth.CONFIGS["tiny"] if bits == 4 else synth.with_changes(
        synth.CONFIGS[f"decode_{bits}bit"], hidden=256, inter=128, n_experts=8)
    blob = synth.expert_blob(cfg, 0, 1)
    x = bk.bf16_to_f64(synth.tokens(cfg, 0, 1)[0])
    y = oracle.section_matvec(oracle.shape_of(cfg), blob, 0, x)
    q, s, b = bk.decode_blob(blob, cfg.hidden, cfg.inter, bits)["gate_raw"]
    S = np.repeat(s, 64, axis=1)
    B = np.repeat(b, 64, axis=1)
    fma_form = (q * (S * x) + B * x).sum(axis=1)
    qx = (q * x).reshape(q.shape[0], -1, 64).sum(axis=2)
    X = x.reshape(-1, 64).sum(axis=1)
    group_form = (s * qx + b * X).sum(axis=1)
    scale = np.abs(y).max()
    np.testing.assert_allclose(y, fma_form, rtol=0, atol=1e-12 * scale)
    np.testing.assert_allclose(y, group_form, rtol=0, atol=1e-12 * scale)


@pytest.mark.parametrize("name", ["tiny", "decode_2bit", "decode_3bit"])
def test_section_matvec_equals_dense_decode_and_matmul(name):
    """The oracle's row loop equals a dense decode (vectorised, test-side)
    followed by numpy's matmul, on the generator's own blobs."""
    cfg = synth.CONFIGS[name]
    if cfg.hidden > 256:
        cfg = synth.with_changes(cfg, hidden=512, inter=256, n_experts=8)
    blob = synth.expert_blob(cfg, 0, 3)
    dense = bk.decode_blob(blob, cfg.hidden, cfg.inter, cfg.bits)
    sh = oracle.shape_of(cfg)
    rng = np.random.default_rng(4)
    for sec, nm in enumerate(("gate", "up", "down")):
        x = rng.standard_normal(dense[nm].shape[1])
        np.testing.assert_allclose(oracle.section_matvec(sh, blob, sec, x), dense[nm] @ x,
                                   rtol=1e-11, atol=1e-12)
        r = 5
        np.testing.assert_array_equal(oracle.dequant_row(sh, blob, sec, r), dense[nm][r])


def test_two_bit_expert_in_four_bit_container_is_identical():
    """The same 2-bit values, scales and biases packed as 4-bit give a
    bit-identical expert output."""
    rng = np.random.default_rng(5)
    H, I = 256, 128
    mats = bk.random_mats(rng, H, I, 2, s_range=(0.004, 0.08), bias_mult=-1.5)
    b2 = bk.build_blob(H, I, 2, mats)
    b4 = bk.build_blob(H, I, 4, mats)
    x = rng.standard_normal(H)
    o2 = oracle.expert_ffn(shape(H, I, bits=2), b2, x)
    o4 = oracle.expert_ffn(shape(H, I, bits=4), b4, x)
    for a, b in zip(o2, o4):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("lo_bits,hi_bits,qmax", [(3, 4, 7), (2, 3, 3)])
def test_narrower_values_in_wider_container_are_identical(lo_bits, hi_bits, qmax):
    """The same values (0..qmax), scales and biases packed as 3-bit and as
    4-bit, or as 2-bit and as 3-bit, give a bit-identical expert output: the
    3-bit planes decode to the values a plain packing holds."""
    rng = np.random.default_rng(6)
    H, I = 256, 128
    mats = bk.random_mats(rng, H, I, lo_bits, qmax=qmax, s_range=(0.002, 0.04), bias_mult=-3.5)
    a = bk.build_blob(H, I, lo_bits, mats)
    b = bk.build_blob(H, I, hi_bits, mats)
    x = rng.standard_normal(H)
    oa = oracle.expert_ffn(shape(H, I, bits=lo_bits), a, x)
    ob = oracle.expert_ffn(shape(H, I, bits=hi_bits), b, x)
    for u, v in zip(oa, ob):
        np.testing.assert_array_equal(u, v)


def test_three_bit_plane_positions_hand_worked():
    """One 3-bit row of 64 values written bit by bit from the layout rule
    (low plane: value j's two low bits at bit 2(j mod 16) of word j/16; high
    plane: value j's high bit at bit 2(j mod 16) + (j/16 mod 2) of word j/32)
    decodes to the values: a transposed plane or a wrong bit offset fails."""
    H, I = 64, 64
    vals = (np.arange(64) * 5 + 3) % 8
    lo = np.zeros(4, dtype=np.uint32)
    hi = np.zeros(2, dtype=np.uint32)
    for j, v in enumerate(vals):
        lo[j // 16] |= np.uint32((int(v) & 3) << (2 * (j % 16)))
        hi[j // 32] |= np.uint32((int(v) >> 2) << (2 * (j % 16) + (j // 16) % 2))
    row = np.concatenate([lo, hi])
    q = np.tile(vals, (I, 1))
    mats = {n: (q if n != "down" else np.tile(vals, (H, 1)), bk.f64_to_bf16(np.full((r, 1), 0.5)),
                bk.f64_to_bf16(np.full((r, 1), -1.0))) for n, r in (("gate", I), ("up", I), ("down", H))}
    blob = bk.build_blob(H, I, 3, mats)
    assert np.array_equal(blob[:24].view(np.uint32), row)
    w = oracle.dequant_row(shape(H, I, bits=3), blob, 0, 0)
    np.testing.assert_array_equal(w, 0.5 * vals - 1.0)


# ------------------------------------------------------------------ routing

def _brute_topk(l, k):
    return [e for e in sorted(range(len(l)), key=lambda e: (-l[e], e))][:k]


def test_topk_matches_brute_force_with_ties():
    rng = np.random.default_rng(6)
    for trial in range(3000):
        E = int(rng.integers(1, 40))
        K = int(rng.integers(0, E + 1))
        l = np.round(rng.standard_normal(E) * 3) / 2   # coarse grid: many exact ties
        assert list(oracle.topk(l, K)) == _brute_topk(list(l), K)


def test_topk_exhaustive_tiny():
    """Every ordering of 5 distinct values (and of a tied multiset), every K."""
    import itertools
    for perm in itertools.permutations([0.5, -1.0, 2.0, 2.0, 7.0]):
        for K in range(6):
            assert list(oracle.topk(np.array(perm), K)) == _brute_topk(list(perm), K)


def test_duplicated_router_rows_tie_to_lower_index():
    cfg = synth.CONFIGS["tiny"]
    wr = synth.router(cfg, 0).copy()
    wr[5] = wr[2]
    wr[6] = wr[2]
    x = bk.bf16_to_f64(synth.tokens(cfg, 0, 1))
    lg, idx, w, gamma = oracle.route(oracle.shape_of(cfg), wr, x, 3)
    assert lg[0, 2] == lg[0, 5] == lg[0, 6]
    # whatever the rank of the tied group, the three tied experts appear in index order
    order = _brute_topk(list(lg[0]), 8)
    pos = [order.index(e) for e in (2, 5, 6)]
    assert pos == sorted(pos) and pos[1] == pos[0] + 1 and pos[2] == pos[1] + 1
    assert list(idx[0]) == order[:3]
    assert gamma[0] == 1.0


def test_router_logits_one_hot_and_matmul():
    cfg = synth.CONFIGS["tiny"]
    sh = oracle.shape_of(cfg)
    wr = synth.router(cfg, 0)
    W = bk.bf16_to_f64(wr)
    for j in (0, 17, 255):
        x = np.zeros(cfg.hidden)
        x[j] = 1.0
        np.testing.assert_array_equal(oracle.router_logits(sh, wr, x), W[:, j])
    x = np.random.default_rng(7).standard_normal(cfg.hidden)
    np.testing.assert_allclose(oracle.router_logits(sh, wr, x), W @ x, rtol=1e-13, atol=1e-15)


def test_softmax_closed_forms():
    rng = np.random.default_rng(8)
    l = rng.standard_normal(32)
    idx = oracle.topk(l, 5)
    w = oracle.softmax_selected(l, idx)
    assert abs(w.sum() - 1.0) < 1e-15
    np.testing.assert_allclose(w, softmax(l[idx]), rtol=1e-14)
    assert np.all(np.diff(w) <= 0)                      # descending logits -> descending weights
    np.testing.assert_allclose(oracle.softmax_selected(l + 123.0, idx), w, rtol=1e-13)
    assert oracle.softmax_selected(l, oracle.topk(l, 1))[0] == 1.0
    eq = np.zeros(16)
    np.testing.assert_allclose(oracle.softmax_selected(eq, np.arange(4, dtype=np.int32)), 0.25, rtol=0)
    full = oracle.softmax_selected(l, idx, renorm=False)
    np.testing.assert_allclose(full, softmax(l)[idx], rtol=1e-14)


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    for z in (0.1, 1.0, 3.7, 20.0):
        assert abs((oracle.silu(z) - oracle.silu(-z)) - z) < 1e-14 * max(1, z)
        np.testing.assert_allclose(oracle.silu(z), z * expit(z), rtol=1e-15)
    assert oracle.silu(100.0) == 100.0
    assert 0 > oracle.silu(-100.0) > -1e-40


def test_rmsnorm_closed_forms():
    for c in (0.001, 1.0, -3.0, 250.0):
        out = oracle.rmsnorm(np.full(64, c))
        np.testing.assert_allclose(out, c / math.sqrt(c * c + 1e-6), rtol=1e-15)
    h = np.random.default_rng(9).standard_normal(4096) * 17
    x = oracle.rmsnorm(h)
    ms = np.mean(h * h)
    np.testing.assert_allclose(np.sqrt(np.mean(x * x)), math.sqrt(ms / (ms + 1e-6)), rtol=1e-13)


# ------------------------------------------------------------------ combine

def _tiny_layer_inputs(E=6, S=1, H=128, I=64, seed=10, bits=4):
    rng = np.random.default_rng(seed)
    blobs = {e: bk.build_blob(H, I, bits, bk.random_mats(rng, H, I, bits)) for e in range(E + S)}
    wr = bk.f64_to_bf16(rng.standard_normal((E, H)) * 0.05)
    return rng, blobs, wr


def test_zero_weights_give_residual_exactly():
    H, I, E = 128, 64, 6
    zero = {n: (np.zeros((r, c), dtype=np.int64), bk.f64_to_bf16(np.zeros((r, c // 64))),
                bk.f64_to_bf16(np.zeros((r, c // 64))))
            for n, (r, c) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I)))}
    blob = bk.build_blob(H, I, 4, zero)
    rng = np.random.default_rng(11)
    wr = bk.f64_to_bf16(rng.standard_normal((E, H)))
    h = rng.standard_normal((3, H))
    out = oracle.moe_layer(shape(H, I, E, 1), {e: blob for e in range(E + 1)}, wr, h, 2)
    np.testing.assert_array_equal(out["y"], h)


def _dense_expert(blob, H, I, x):
    D = bk.decode_blob(blob, H, I, 4)
    g = D["gate"] @ x
    u = D["up"] @ x
    return D["down"] @ (g * expit(g) * u)


def test_all_experts_active_is_dense_soft_moe():
    """K = E: the layer is a dense soft mixture: y = h + sum_e softmax(l)_e d_e + d_shared,
    computed here with dense matrices and numpy matmuls."""
    H, I, E = 128, 64, 6
    rng, blobs, wr = _tiny_layer_inputs(E=E, H=H, I=I)
    h = rng.standard_normal((2, H))
    out = oracle.moe_layer(shape(H, I, E, 1), blobs, wr, h, E)
    for t in range(2):
        p = softmax(bk.bf16_to_f64(wr) @ h[t])
        y = h[t] + sum(p[e] * _dense_expert(blobs[e], H, I, h[t]) for e in range(E))
        y = y + _dense_expert(blobs[E], H, I, h[t])
        np.testing.assert_allclose(out["y"][t], y, rtol=1e-10, atol=1e-10 * np.abs(y).max())


def test_shared_only_is_dense_swiglu_mlp():
    """K = 0 with one shared expert: y = h + Wd (silu(Wg h) * (Wu h))."""
    H, I, E = 128, 64, 6
    rng, blobs, wr = _tiny_layer_inputs(E=E, H=H, I=I, seed=12)
    h = rng.standard_normal((1, H))
    out = oracle.moe_layer(shape(H, I, E, 1), blobs, wr, h, 0)
    y = h[0] + _dense_expert(blobs[E], H, I, h[0])
    np.testing.assert_allclose(out["y"][0], y, rtol=1e-10, atol=1e-10 * np.abs(y).max())


def test_zero_shared_gate_vector_halves_shared_contribution():
    """gamma = sigmoid(0) = 1/2 for an all-zero gate vector."""
    H, I, E = 128, 64, 6
    rng, blobs, wr = _tiny_layer_inputs(E=E, H=H, I=I, seed=13)
    h = rng.standard_normal((1, H))
    ungated = oracle.moe_layer(shape(H, I, E, 1), blobs, wr, h, 0)
    gated = oracle.moe_layer(shape(H, I, E, 1), blobs, wr, h, 0,
                             shared_gate=np.zeros(H, dtype=np.uint16))
    assert gated["gamma"][0] == 0.5
    np.testing.assert_allclose(gated["y"] - h, 0.5 * (ungated["y"] - h), rtol=1e-14, atol=1e-15)


def _one_hot_gate(H, j, c):
    """bf16 gate vector c * e_j (c exactly representable in bf16)."""
    g = np.zeros(H)
    g[j] = c
    gb = bk.f64_to_bf16(g)
    assert bk.bf16_to_f64(gb)[j] == c
    return gb


@pytest.mark.parametrize("rms", [False, True])
@pytest.mark.parametrize("j,c", [(0, 0.75), (5, -1.5), (77, 2.0), (127, -0.375)])
def test_one_hot_shared_gate_closed_form(rms, j, c):
    """A one-hot gate c * e_j gives gamma = sigmoid(c * xhat_j): xhat = h without
    the norm flag, h_j / sqrt(mean(h^2) + 1e-6) with it.  The shared term of the
    output is then gamma times the dense SwiGLU expert applied to xhat
    (K = 0, so nothing else is added to the residual).  A sign slip in the
    exponent, a dot taken over h instead of xhat, or the gate applied to the
    wrong term fails here."""
    H, I, E = 128, 64, 6
    rng, blobs, wr = _tiny_layer_inputs(E=E, H=H, I=I, seed=16)
    h = rng.standard_normal((2, H)) * 3.0
    flags = oracle.RMSNORM if rms else 0
    out = oracle.moe_layer(shape(H, I, E, 1), blobs, wr, h, 0, flags=flags,
                           shared_gate=_one_hot_gate(H, j, c))
    for t in range(2):
        xhat = h[t] / math.sqrt(np.mean(h[t] ** 2) + 1e-6) if rms else h[t]
        gamma = 1.0 / (1.0 + math.exp(-c * xhat[j]))
        assert math.isclose(out["gamma"][t], gamma, rel_tol=1e-14)
        y = h[t] + gamma * _dense_expert(blobs[E], H, I, xhat)
        np.testing.assert_allclose(out["y"][t], y, rtol=1e-10, atol=1e-10 * np.abs(y).max())


def test_shared_gate_sign_and_scale_symmetries():
    """sigmoid(-z) = 1 - sigmoid(z): negating the gate vector maps gamma to
    1 - gamma; with the norm flag, scaling h (well above the epsilon) leaves
    gamma unchanged, and without it the logit of gamma is the dot product
    gate . h, scaled with h."""
    H, I, E = 128, 64, 6
    rng, blobs, wr = _tiny_layer_inputs(E=E, H=H, I=I, seed=17)
    h = rng.standard_normal((3, H)) * 2.0
    gv = bk.f64_to_bf16(rng.standard_normal(H) * 0.1)
    neg = bk.f64_to_bf16(-bk.bf16_to_f64(gv))
    sh = shape(H, I, E, 1)
    for flags in (0, oracle.RMSNORM):
        _, _, _, g_pos = oracle.route(sh, wr, h, 2, flags, shared_gate=gv)
        _, _, _, g_neg = oracle.route(sh, wr, h, 2, flags, shared_gate=neg)
        np.testing.assert_allclose(g_pos + g_neg, 1.0, rtol=0, atol=1e-15)
        assert np.all(np.abs(g_pos - 0.5) > 1e-6)
    big = h * 1e4          # mean(h^2) ~ 4e8: the 1e-6 under the root is below fp64 resolution
    _, _, _, g1 = oracle.route(sh, wr, big, 2, oracle.RMSNORM, shared_gate=gv)
    _, _, _, g8 = oracle.route(sh, wr, 8.0 * big, 2, oracle.RMSNORM, shared_gate=gv)
    np.testing.assert_allclose(g8, g1, rtol=1e-13)
    _, _, _, r1 = oracle.route(sh, wr, h, 2, 0, shared_gate=gv)
    _, _, _, r8 = oracle.route(sh, wr, 8.0 * h, 2, 0, shared_gate=gv)
    z1 = np.log(r1 / (1.0 - r1))
    z8 = np.log(r8 / (1.0 - r8))
    np.testing.assert_allclose(z8, 8.0 * z1, rtol=1e-9)
    np.testing.assert_allclose(z1, h @ bk.bf16_to_f64(gv), rtol=1e-9)


def test_layer_intermediates_are_consistent():
    """gu, a and d exported per slot are the expert's own g, u, silu(g)*u and Wd a."""
    cfg = synth.CONFIGS["tiny"]
    x = bk.bf16_to_f64(synth.tokens(cfg, 0))
    out = oracle.run_layer(cfg, 0, x)
    idx = out["idx"][0]
    blob = synth.expert_blob(cfg, 0, int(idx[1]))
    g, u, a, d = oracle.expert_ffn(oracle.shape_of(cfg), blob, x[0])
    np.testing.assert_array_equal(out["gu"][0, 1, 0], g)
    np.testing.assert_array_equal(out["gu"][0, 1, 1], u)
    np.testing.assert_array_equal(out["a"][0, 1], a)
    np.testing.assert_array_equal(out["d"][0, 1], d)
    y = x[0] + sum(out["w"][0, k] * out["d"][0, k] for k in range(cfg.top_k)) + out["d"][0, cfg.top_k]
    np.testing.assert_allclose(out["y"][0], y, rtol=1e-15, atol=1e-13)


def test_expert_permutation_invariance():
    """Permuting the routed experts (blobs and router rows together) leaves the
    layer output unchanged and maps the selection through the permutation."""
    H, I, E = 128, 64, 6
    rng, blobs, wr = _tiny_layer_inputs(E=E, H=H, I=I, seed=14)
    h = rng.standard_normal((3, H))
    perm = rng.permutation(E)              # new index n holds old expert perm[n]
    blobs_p = {n: blobs[int(perm[n])] for n in range(E)}
    blobs_p[E] = blobs[E]
    a = oracle.moe_layer(shape(H, I, E, 1), blobs, wr, h, 3)
    b = oracle.moe_layer(shape(H, I, E, 1), blobs_p, wr[perm], h, 3)
    np.testing.assert_array_equal(perm[b["idx"]], a["idx"])
    np.testing.assert_allclose(b["y"], a["y"], rtol=1e-14, atol=1e-13)


def test_rmsnorm_flag_normalises_input_but_keeps_residual():
    """With the norm flag the experts and router see h / rms(h) while the
    residual stays h: scaling h by c scales the residual only (h is large
    enough here that eps = 1e-6 under the root is below fp64 resolution)."""
    H, I, E = 128, 64, 6
    rng, blobs, wr = _tiny_layer_inputs(E=E, H=H, I=I, seed=15)
    h = rng.standard_normal((1, H)) * 1e5
    a = oracle.moe_layer(shape(H, I, E, 1), blobs, wr, h, 2, flags=oracle.RMSNORM)
    b = oracle.moe_layer(shape(H, I, E, 1), blobs, wr, 8.0 * h, 2, flags=oracle.RMSNORM)
    np.testing.assert_array_equal(a["idx"], b["idx"])
    np.testing.assert_allclose(b["y"] - 8.0 * h, a["y"] - h, rtol=1e-9, atol=1e-9)
