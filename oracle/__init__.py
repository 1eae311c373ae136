"""fp64 CPU oracle for the quantized MoE expert path (ctypes wrapper).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and the CPU
baseline leg of bench.py may import this package.  It shares no code with
the HIP library; its inputs come from the seeded generator in `synth`.
The arithmetic lives in moeq_oracle.c, whose header states what each
function follows on the pages.

Parity pins: every function here is pinned by a CPU test in
tests/test_oracle_pins.py (closed forms, brute force, special cases that
reduce to a library routine); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

import synth

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libmoeq_oracle.so")

NO_RENORM = 1
RMSNORM = 2


class Shape(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("group", ctypes.c_int32)]


def shape_of(cfg) -> Shape:
    return Shape(cfg.hidden, cfg.inter, cfg.n_experts, cfg.n_shared, cfg.bits, cfg.group)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: -O2, no fast-math, no fp contraction."""
    src = os.path.join(_HERE, "moeq_oracle.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c99", "-O2", "-fPIC", "-shared",
                               "-ffp-contract=off", "-fopenmp", "-o", tmp, src, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None
_P = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        S = ctypes.POINTER(Shape)
        L.oracle_expert_bytes.restype = ctypes.c_int64
        L.oracle_expert_bytes.argtypes = [S]
        L.oracle_dequant_row.argtypes = [S, _P, ctypes.c_int, ctypes.c_int, _P]
        L.oracle_section_matvec.argtypes = [S, _P, ctypes.c_int, _P, _P]
        L.oracle_silu.restype = ctypes.c_double
        L.oracle_silu.argtypes = [ctypes.c_double]
        L.oracle_expert_ffn.argtypes = [S, _P, _P, _P, _P, _P, _P]
        L.oracle_rmsnorm.argtypes = [_P, ctypes.c_int, ctypes.c_double, _P]
        L.oracle_router_logits.argtypes = [S, _P, _P, _P]
        L.oracle_topk.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P]
        L.oracle_softmax_selected.argtypes = [_P, ctypes.c_int, _P, ctypes.c_int,
                                              ctypes.c_int, _P]
        L.oracle_route.argtypes = [S, _P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   _P, _P, _P, _P]
        L.oracle_moe_layer.restype = ctypes.c_int
        L.oracle_moe_layer.argtypes = [S, _P, _P, _P, _P, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- primitives

def expert_bytes(shape: Shape) -> int:
    return lib().oracle_expert_bytes(ctypes.byref(shape))


def dequant_row(shape: Shape, blob: np.ndarray, sec: int, row: int) -> np.ndarray:
    cols = shape.inter if sec == 2 else shape.hidden
    out = np.empty(cols, dtype=np.float64)
    blob = _c(blob, np.uint8)
    lib().oracle_dequant_row(ctypes.byref(shape), _p(blob), sec, row, _p(out))
    return out


def section_matvec(shape: Shape, blob: np.ndarray, sec: int, x: np.ndarray) -> np.ndarray:
    rows = shape.hidden if sec == 2 else shape.inter
    out = np.empty(rows, dtype=np.float64)
    blob = _c(blob, np.uint8)
    x = _c(x, np.float64)
    lib().oracle_section_matvec(ctypes.byref(shape), _p(blob), sec, _p(x), _p(out))
    return out


def silu(z: float) -> float:
    return lib().oracle_silu(z)


def expert_ffn(shape: Shape, blob: np.ndarray, xhat: np.ndarray):
    I, H = shape.inter, shape.hidden
    g, u, a = (np.empty(I) for _ in range(3))
    d = np.empty(H)
    blob = _c(blob, np.uint8)
    xhat = _c(xhat, np.float64)
    lib().oracle_expert_ffn(ctypes.byref(shape), _p(blob), _p(xhat), _p(g), _p(u), _p(a), _p(d))
    return g, u, a, d


def rmsnorm(h: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    h = _c(h, np.float64)
    out = np.empty_like(h)
    lib().oracle_rmsnorm(_p(h), h.size, eps, _p(out))
    return out


def router_logits(shape: Shape, wr: np.ndarray, xhat: np.ndarray) -> np.ndarray:
    out = np.empty(shape.n_experts)
    wr = _c(wr, np.uint16)
    xhat = _c(xhat, np.float64)
    lib().oracle_router_logits(ctypes.byref(shape), _p(wr), _p(xhat), _p(out))
    return out


def topk(logits: np.ndarray, k: int) -> np.ndarray:
    logits = _c(logits, np.float64)
    idx = np.empty(k, dtype=np.int32)
    lib().oracle_topk(_p(logits), logits.size, k, _p(idx))
    return idx


def softmax_selected(logits: np.ndarray, idx: np.ndarray, renorm: bool = True) -> np.ndarray:
    logits = _c(logits, np.float64)
    idx = _c(idx, np.int32)
    w = np.empty(idx.size)
    lib().oracle_softmax_selected(_p(logits), logits.size, _p(idx), idx.size, int(renorm), _p(w))
    return w


def route(shape: Shape, wr, h, k: int, flags: int = 0, shared_gate=None):
    """Routing of T tokens: (logits [T,E], idx [T,k], w [T,k], gamma [T])."""
    h = _c(np.atleast_2d(h), np.float64)
    T = h.shape[0]
    logits = np.empty((T, shape.n_experts))
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k))
    gamma = np.empty(T)
    wr = _c(wr, np.uint16)
    sg = None if shared_gate is None else _c(shared_gate, np.uint16)
    lib().oracle_route(ctypes.byref(shape), _p(wr), _p(sg), _p(h), T, k, flags,
                       _p(logits), _p(idx), _p(w), _p(gamma))
    return logits, idx, w, gamma


def moe_layer(shape: Shape, blobs: dict, wr, h, k: int, flags: int = 0,
              shared_gate=None, want_intermediates: bool = True) -> dict:
    """One MoE layer for T tokens.  `blobs` maps expert index (shared experts
    at n_experts + i) to uint8 blobs; it must hold every expert some token
    selects (use `route` first) and the shared ones."""
    h = _c(np.atleast_2d(h), np.float64)
    T, H = h.shape
    I, E, S = shape.inter, shape.n_experts, shape.n_shared
    KS = k + S
    keep = [_c(blobs[e], np.uint8) if e in blobs else None for e in range(E + S)]
    table = (ctypes.c_void_p * (E + S))(*[None if b is None else b.ctypes.data for b in keep])
    out = dict(logits=np.empty((T, E)), idx=np.empty((T, k), dtype=np.int32),
               w=np.empty((T, k)), gamma=np.empty(T), y=np.empty((T, H)))
    if want_intermediates:
        out.update(gu=np.empty((T, KS, 2, I)), a=np.empty((T, KS, I)), d=np.empty((T, KS, H)))
    wr = _c(wr, np.uint16)
    sg = None if shared_gate is None else _c(shared_gate, np.uint16)
    rc = lib().oracle_moe_layer(ctypes.byref(shape), table, _p(wr), _p(sg), _p(h), T, k, flags,
                                _p(out["logits"]), _p(out["idx"]), _p(out["w"]),
                                _p(out["gamma"]), _p(out.get("gu")), _p(out.get("a")),
                                _p(out.get("d")), _p(out["y"]))
    if rc != 0:
        raise ValueError("oracle_moe_layer: a selected expert's blob is missing")
    return out


# ------------------------------------------------------- workload helpers

def layer_flags(cfg, renorm: bool = True) -> int:
    return (RMSNORM if cfg.rmsnorm else 0) | (0 if renorm else NO_RENORM)


def run_layer(cfg, layer: int, h: np.ndarray, want_intermediates: bool = True,
              shared_gate=None, renorm: bool = True, wr=None, blob_cache: dict | None = None) -> dict:
    """Route with the oracle, generate only the needed expert blobs from the
    seeded streams, then run the layer."""
    shape = shape_of(cfg)
    wr = synth.router(cfg, layer) if wr is None else wr
    flags = layer_flags(cfg, renorm)
    _, idx, _, _ = route(shape, wr, h, cfg.top_k, flags, shared_gate)
    need = set(int(e) for e in np.unique(idx)) | set(range(cfg.n_experts, cfg.n_slots))
    cache = {} if blob_cache is None else blob_cache
    blobs = {}
    for e in need:
        key = (layer, e)
        if key not in cache:
            cache[key] = synth.expert_blob(cfg, layer, e)
        blobs[e] = cache[key]
    return moe_layer(shape, blobs, wr, h, cfg.top_k, flags, shared_gate, want_intermediates)


def run_stack(cfg, x: np.ndarray, layers: int | None = None, first_layer: int = 0) -> dict:
    """Free-running stack of layers: h_{l+1} = layer_l(h_l).  Returns the
    per-layer input h (fp64), idx, w and the per-layer logit margin between
    the K-th and (K+1)-th ranked experts."""
    L = cfg.layers if layers is None else layers
    h = _c(np.atleast_2d(x), np.float64)
    hs, idxs, ws, margins = [h], [], [], []
    for l in range(first_layer, first_layer + L):
        out = run_layer(cfg, l, h, want_intermediates=False)
        srt = -np.sort(-out["logits"], axis=1)
        K = cfg.top_k
        margins.append(srt[:, K - 1] - srt[:, K] if K < cfg.n_experts else np.full(h.shape[0], np.inf))
        idxs.append(out["idx"])
        ws.append(out["w"])
        h = out["y"]
        hs.append(h)
    return dict(h=np.stack(hs), idx=np.stack(idxs), w=np.stack(ws), margin=np.stack(margins))
