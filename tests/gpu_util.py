"""Helpers for the GPU tests: seeded inputs moved to device memory, and the
parity bar (exact top-K; max |gpu - oracle| <= 2e-3 * max |oracle|)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import quantized_expert_gemv_router_amd as q
import synth

TOL = 2e-3


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def slot_stride(cfg) -> int:
    return (cfg.expert_bytes + 255) // 256 * 256


def bf16_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def layer_arena(cfg, layer: int) -> torch.Tensor:
    host = synth.layer_blobs(cfg, layer, slot_stride(cfg))
    return torch.from_numpy(host.reshape(-1)).cuda()


def experts_for(cfg, layers=(0,)):
    shape = q.Shape.of(cfg)
    arenas = [layer_arena(cfg, l) for l in layers]
    return shape, q.ExpertTable(shape, arenas, slot_stride(cfg))


def rel_err(gpu, ref) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = np.abs(ref).max()
    return float(np.abs(gpu - ref).max() / denom) if denom > 0 else float(np.abs(gpu).max())


def assert_close(gpu, ref, what: str, tol: float = TOL):
    e = rel_err(gpu, ref)
    assert np.all(np.isfinite(np.asarray(gpu))), f"{what}: non-finite values"
    assert e <= tol, f"{what}: max|gpu-oracle|/max|oracle| = {e:.3e} > {tol:g}"
    return e


# The persistent decode hands each router logit to the other workgroups as
# its fp64 value rounded to a 36-bit significand (2^-37 relative), and every
# workgroup selects from those rounded values.
HANDOFF_REL = 2.0 ** -35


def topk_matches(idx, ref_idx, ref_logits, rel: float = HANDOFF_REL) -> bool:
    """The GPU's top-K against the oracle's (fp64, ties to the lower index):
    equal, except that a rank may hold another expert whose oracle logit
    differs from the oracle's pick by a nonzero amount at most
    rel * max|logit| -- two logits that close can round to one value in the
    hand-off and then go to the lower index.  Exact ties keep the
    lower-index rule on both sides, so they must match exactly."""
    idx, ref_idx = np.asarray(idx), np.asarray(ref_idx)
    if np.array_equal(idx, ref_idx):
        return True
    if len(set(idx.tolist())) != idx.size:
        return False
    tol = rel * np.abs(ref_logits).max()
    for g, o in zip(idx.tolist(), ref_idx.tolist()):
        if g == o:
            continue
        if not 0 <= g < ref_logits.size:
            return False
        d = abs(ref_logits[g] - ref_logits[o])
        if not 0.0 < d <= tol:
            return False
    return True
