"""The seeded generator: known answers of SplitMix64 and the value
distributions each workload states (4-bit nibbles U{0..15}, bf16 scales
U(0.001, 0.02), bias = -8 * scale; 2-bit values U{0..3}, scales
U(0.004, 0.08), bias = bf16(-1.5 * scale); router N(0, 0.02^2); x N(0, 1))."""
import json
import os

import numpy as np

import synth
from tests import blobkit as bk

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_known_answers():
    gold = json.load(open(os.path.join(GOLD, "splitmix64_seed0.json")))
    for i, hx in enumerate(gold["outputs_hex"]):
        assert synth.lib().synth_hash(0, i) == int(hx, 16)


def test_layout_offsets():
    cfg = synth.CONFIGS["decode_4bit"]
    off = synth.expert_offsets(cfg)
    assert off == [0, 2 << 20, 4 << 20, 6 << 20, 6_553_600, 6_815_744, 7_077_888, ]


def test_four_bit_distributions():
    cfg = synth.CONFIGS["decode_4bit"]
    blob = synth.expert_blob(cfg, 0, 7)
    D = bk.decode_blob(blob, cfg.hidden, cfg.inter, 4)
    q, s, b = D["gate_raw"]
    hist = np.bincount(q.ravel(), minlength=16) / q.size
    assert np.all(np.abs(hist - 1 / 16) < 0.002)
    # bf16 rounding may step just past the interval ends
    assert s.min() >= 0.001 * (1 - 2 ** -8) and s.max() <= 0.02 * (1 + 2 ** -8)
    assert abs(s.mean() - 0.0105) < 0.0003
    np.testing.assert_array_equal(b, -8.0 * s)


def test_two_bit_distributions():
    cfg = synth.CONFIGS["decode_2bit"]
    blob = synth.expert_blob(cfg, 0, 3)
    D = bk.decode_blob(blob, cfg.hidden, cfg.inter, 2)
    q, s, b = D["down_raw"]
    hist = np.bincount(q.ravel(), minlength=4) / q.size
    assert np.all(np.abs(hist - 0.25) < 0.003)
    assert s.min() >= 0.004 * (1 - 2 ** -8) and s.max() <= 0.08 * (1 + 2 ** -8)
    np.testing.assert_array_equal(b, bk.bf16_to_f64(bk.f64_to_bf16(-1.5 * s)))


def test_gaussians():
    cfg = synth.CONFIGS["decode_4bit"]
    wr = bk.bf16_to_f64(synth.router(cfg, 0))
    assert wr.shape == (512, 4096)
    assert abs(wr.mean()) < 1e-4 and abs(wr.std() - 0.02) < 1e-4
    x = bk.bf16_to_f64(synth.tokens(synth.CONFIGS["batch16_top10"], 0))
    assert x.shape == (16, 4096)
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1.0) < 0.02
    assert not np.array_equal(x[0], x[1])


def test_streams_are_deterministic_and_distinct():
    cfg = synth.CONFIGS["tiny"]
    a = synth.expert_blob(cfg, 0, 1)
    assert np.array_equal(a, synth.expert_blob(cfg, 0, 1))
    assert not np.array_equal(a, synth.expert_blob(cfg, 0, 2))
    assert not np.array_equal(a, synth.expert_blob(cfg, 1, 1))
    blobs = synth.layer_blobs(cfg, 0, stride=cfg.expert_bytes + 256)
    assert np.array_equal(blobs[1, :cfg.expert_bytes], a)
    assert np.all(blobs[:, cfg.expert_bytes:] == 0)
