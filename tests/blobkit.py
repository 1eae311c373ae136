"""Test-side packing and dense decoding of expert blobs (numpy, vectorised).

Written from the layout specification alone, independently of the oracle's
row-by-row decoder and of the HIP kernels, so that the pins can build blobs
with chosen values and decode whole matrices with a different algorithm:
  [gate.q | up.q | down.q | gate.sb | up.sb | down.sb]
  value j of a row in word j // (32/bits) at bit bits * (j % (32/bits))
  3-bit rows: a low-bits plane (the row's values & 3 packed as a 2-bit
  row), then a high-bit plane of cols/32 words in which word w holds the
  high bits of values 32w..32w+15 at the even bits and of 32w+16..32w+31
  at the odd bits
  sb: u32 per (row, group of 64 inputs) = bf16 scale | bf16 bias << 16
"""
from __future__ import annotations

import numpy as np


def f64_to_bf16(x) -> np.ndarray:
    """Round to nearest even bf16 (via fp32), returned as uint16 bit patterns."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_to_f64(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _pack_hi_plane(hi: np.ndarray) -> np.ndarray:
    """High bits [rows, cols] -> words [rows, cols/32]: in each block of 32
    values, the first 16 at even bits, the next 16 at odd bits."""
    rows, cols = hi.shape
    blk = hi.reshape(rows, cols // 32, 2, 16).astype(np.uint32)
    shifts = (2 * np.arange(16, dtype=np.uint32))[None, None, None, :] + np.arange(2, dtype=np.uint32)[None, None, :, None]
    return (blk << shifts).sum(axis=(2, 3), dtype=np.uint64).astype(np.uint32)


def _unpack_hi_plane(words: np.ndarray, cols: int) -> np.ndarray:
    rows = words.shape[0]
    shifts = (2 * np.arange(16, dtype=np.uint32))[None, None, None, :] + np.arange(2, dtype=np.uint32)[None, None, :, None]
    bits = (words[:, :, None, None] >> shifts) & np.uint32(1)
    return bits.reshape(rows, cols).astype(np.int64)


def pack_q(q: np.ndarray, bits: int) -> np.ndarray:
    rows, cols = q.shape
    if bits == 3:
        lo = pack_q(q & 3, 2)
        hi = _pack_hi_plane(q >> 2)
        return np.concatenate([lo, hi], axis=1)
    pw = 32 // bits
    words = np.zeros((rows, cols // pw), dtype=np.uint32)
    for m in range(pw):
        words |= q[:, m::pw].astype(np.uint32) << np.uint32(bits * m)
    return words


def unpack_q(words: np.ndarray, cols: int, bits: int) -> np.ndarray:
    rows = words.shape[0]
    if bits == 3:
        return unpack_q(words[:, :cols // 16], cols, 2) + 4 * _unpack_hi_plane(words[:, cols // 16:], cols)
    pw = 32 // bits
    q = np.empty((rows, cols), dtype=np.int64)
    mask = (1 << bits) - 1
    for m in range(pw):
        q[:, m::pw] = (words >> np.uint32(bits * m)) & mask
    return q


def pack_sb(scale_bf16: np.ndarray, bias_bf16: np.ndarray) -> np.ndarray:
    return scale_bf16.astype(np.uint32) | (bias_bf16.astype(np.uint32) << np.uint32(16))


def build_blob(H: int, I: int, bits: int, mats: dict, G: int = 64) -> np.ndarray:
    """mats: {'gate'|'up'|'down': (q int array [rows, cols], scale bf16 [rows, cols/G],
    bias bf16 [rows, cols/G])}."""
    parts_q, parts_sb = [], []
    for name, (rows, cols) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        q, s, b = mats[name]
        assert q.shape == (rows, cols) and s.shape == (rows, cols // G)
        parts_q.append(pack_q(q, bits).ravel())
        parts_sb.append(pack_sb(s, b).ravel())
    return np.concatenate(parts_q + parts_sb).view(np.uint8).copy()


def random_mats(rng, H, I, bits, G=64, s_range=(0.001, 0.02), bias_mult=-8.0, qmax=None):
    qmax = (1 << bits) - 1 if qmax is None else qmax
    mats = {}
    for name, (rows, cols) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        q = rng.integers(0, qmax + 1, size=(rows, cols))
        s = f64_to_bf16(rng.uniform(*s_range, size=(rows, cols // G)))
        b = f64_to_bf16(bias_mult * bf16_to_f64(s))
        mats[name] = (q, s, b)
    return mats


def decode_blob(blob: np.ndarray, H: int, I: int, bits: int, G: int = 64) -> dict:
    """Dense fp64 matrices {'gate': [I,H], 'up': [I,H], 'down': [H,I]} plus the raw
    (q, scale, bias) per section."""
    words = np.ascontiguousarray(blob).view(np.uint32)
    qw = H * I * bits // 32
    sbw = H * I // G
    out = {}
    for k, (name, (rows, cols)) in enumerate((("gate", (I, H)), ("up", (I, H)), ("down", (H, I)))):
        w = words[k * qw:(k + 1) * qw].reshape(rows, cols * bits // 32)
        sb = words[3 * qw + k * sbw:3 * qw + (k + 1) * sbw].reshape(rows, cols // G)
        q = unpack_q(w, cols, bits)
        s = bf16_to_f64((sb & 0xFFFF).astype(np.uint16))
        b = bf16_to_f64((sb >> 16).astype(np.uint16))
        dense = q * np.repeat(s, G, axis=1) + np.repeat(b, G, axis=1)
        out[name] = dense
        out[name + "_raw"] = (q, s, b)
    return out
