"""Seeded synthetic workloads for the quantized MoE expert path.

Input generation only: expert blobs, router matrices and token activations,
drawn from counter-based SplitMix64 streams (see synth_host.c).  The fp64
oracle and the HIP library both take their inputs from here; this module
holds none of the path's arithmetic.

The workload shapes follow the pages: hidden 4096 with 512 experts per
layer and K=4 active experts including one shared (Flash-MoE,
fr.news.hada.io, "Architecture du modèle"), top-10 routing (openclawradar.com/fr,
first paragraph), 60 layers (same Flash-MoE section), 4-bit and 2-bit
affine experts (Flash-MoE, "Résultats de performance" and "Shaders de
calcul Metal").  Real weights and prompts are not used; seeded synthetic
values of the same shapes stand in for them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth_host.so")

# stream tensor ids (must match synth_host.c)
T_GATE_Q, T_UP_Q, T_DOWN_Q, T_GATE_SB, T_UP_SB, T_DOWN_SB = range(6)
T_ROUTER, T_TOKEN, T_SHARED_GATE = 6, 7, 8


@dataclass(frozen=True)
class MoEConfig:
    name: str
    hidden: int
    n_experts: int
    inter: int
    top_k: int            # routed experts per token
    n_shared: int         # always-active experts (0 or 1)
    tokens: int           # tokens per step
    bits: int             # 4 or 2
    group: int = 64
    s_lo: float = 0.001   # bf16 scale ~ U(s_lo, s_hi)
    s_hi: float = 0.02
    bias_mult: float = -8.0
    router_sigma: float = 0.02
    layers: int = 1
    rmsnorm: bool = False  # unit-weight RMS norm of each layer's input
    seed: int = 0

    @property
    def n_slots(self) -> int:
        return self.n_experts + self.n_shared

    @property
    def expert_bytes(self) -> int:
        q = self.hidden * self.inter * self.bits // 8
        sb = self.hidden * self.inter // self.group * 4
        return 3 * (q + sb)


_FOUR = dict(bits=4, s_lo=0.001, s_hi=0.02, bias_mult=-8.0)
_TWO = dict(bits=2, s_lo=0.004, s_hi=0.08, bias_mult=-1.5)
_THREE = dict(bits=3, s_lo=0.002, s_hi=0.04, bias_mult=-3.5)

CONFIGS = {
    # hidden 256, 8 experts, I=128, top-2 + 1 shared, 1 token
    "tiny": MoEConfig("tiny", 256, 8, 128, 2, 1, 1, **_FOUR),
    # one Flash-MoE shaped decode layer, top-3 routed + 1 shared
    "decode_4bit": MoEConfig("decode_4bit", 4096, 512, 1024, 3, 1, 1, **_FOUR),
    # same layer, 2-bit experts, top-4 + 1 shared
    "decode_2bit": MoEConfig("decode_2bit", 4096, 512, 1024, 4, 1, 1, **_TWO),
    # the same layer with 3-bit affine experts (values 0..7, bias -3.5 * scale)
    "decode_3bit": MoEConfig("decode_3bit", 4096, 512, 1024, 4, 1, 1, **_THREE),
    # batched decode, top-10 + 1 shared, 16 tokens
    "batch16_top10": MoEConfig("batch16_top10", 4096, 512, 1024, 10, 1, 16, **_FOUR),
    # 60 resident layers, 1-token decode, top-3 + 1 shared, RMS norm between layers
    "stack60_decode": MoEConfig("stack60_decode", 4096, 512, 1024, 3, 1, 1,
                                layers=60, rmsnorm=True, **_FOUR),
    # prefill variant: 2048 tokens, top-10 + 1 shared per layer
    "stack60_prefill": MoEConfig("stack60_prefill", 4096, 512, 1024, 10, 1, 2048,
                                 layers=60, rmsnorm=True, **_FOUR),
    # longer prompts through the same layers (past the MFMA ridge)
    "stack60_prefill_4k": MoEConfig("stack60_prefill_4k", 4096, 512, 1024, 10, 1, 4096,
                                    layers=60, rmsnorm=True, **_FOUR),
    "stack60_prefill_8k": MoEConfig("stack60_prefill_8k", 4096, 512, 1024, 10, 1, 8192,
                                    layers=60, rmsnorm=True, **_FOUR),
}


class _Spec(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("s_lo", ctypes.c_float), ("s_hi", ctypes.c_float),
                ("bias_mult", ctypes.c_float), ("seed", ctypes.c_uint64)]


def build(force: bool = True) -> str:
    """Compile the host generator with gcc (OpenMP, no fp contraction)."""
    src = os.path.join(_HERE, "synth_host.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fopenmp", "-o", tmp, src, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        L.synth_stream_key.restype = ctypes.c_uint64
        L.synth_stream_key.argtypes = [ctypes.c_uint64] + [ctypes.c_uint32] * 4
        L.synth_hash.restype = ctypes.c_uint64
        L.synth_hash.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.synth_expert_bytes.restype = ctypes.c_int64
        L.synth_expert_bytes.argtypes = [ctypes.POINTER(_Spec)]
        L.synth_expert_offsets.argtypes = [ctypes.POINTER(_Spec), ctypes.POINTER(ctypes.c_int64)]
        L.synth_fill_expert.argtypes = [ctypes.POINTER(_Spec), ctypes.c_uint32,
                                        ctypes.c_uint32, ctypes.c_void_p]
        L.synth_fill_experts.argtypes = [ctypes.POINTER(_Spec), ctypes.c_uint32, ctypes.c_uint32,
                                         ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p]
        L.synth_fill_gaussian_bf16.argtypes = [ctypes.c_uint64, ctypes.c_int64,
                                               ctypes.c_double, ctypes.c_void_p]
        _lib = L
    return _lib


def spec(cfg: MoEConfig) -> _Spec:
    return _Spec(cfg.hidden, cfg.inter, cfg.bits, cfg.group, cfg.s_lo, cfg.s_hi,
                 cfg.bias_mult, cfg.seed)


def stream_key(seed: int, layer: int, unit: int, tensor: int, bits: int) -> int:
    return lib().synth_stream_key(seed, layer, unit, tensor, bits)


def expert_offsets(cfg: MoEConfig) -> list[int]:
    off = (ctypes.c_int64 * 7)()
    s = spec(cfg)
    lib().synth_expert_offsets(ctypes.byref(s), off)
    return list(off)


def expert_blob(cfg: MoEConfig, layer: int, expert: int) -> np.ndarray:
    """One expert's packed blob (uint8).  Shared experts use index n_experts."""
    out = np.empty(cfg.expert_bytes, dtype=np.uint8)
    s = spec(cfg)
    lib().synth_fill_expert(ctypes.byref(s), layer, expert, out.ctypes.data)
    return out


def layer_blobs(cfg: MoEConfig, layer: int, stride: int | None = None) -> np.ndarray:
    """All n_experts + n_shared blobs of a layer as [n_slots, stride] uint8."""
    stride = stride or cfg.expert_bytes
    out = np.zeros((cfg.n_slots, stride), dtype=np.uint8)
    s = spec(cfg)
    lib().synth_fill_experts(ctypes.byref(s), layer, 0, cfg.n_slots, stride, out.ctypes.data)
    return out


def gaussian_bf16(key: int, n: int, sigma: float) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    lib().synth_fill_gaussian_bf16(key, n, sigma, out.ctypes.data)
    return out


def router(cfg: MoEConfig, layer: int) -> np.ndarray:
    """Router matrix [n_experts, hidden] as bf16 bit patterns, N(0, 0.02^2)."""
    k = stream_key(cfg.seed, layer, 0, T_ROUTER, 0)
    return gaussian_bf16(k, cfg.n_experts * cfg.hidden, cfg.router_sigma).reshape(
        cfg.n_experts, cfg.hidden)


def shared_gate_vector(cfg: MoEConfig, layer: int) -> np.ndarray:
    """Optional shared-expert gate vector [hidden] (bf16 bits), N(0, 0.02^2)."""
    k = stream_key(cfg.seed, layer, 0, T_SHARED_GATE, 0)
    return gaussian_bf16(k, cfg.hidden, cfg.router_sigma)


def tokens(cfg: MoEConfig, token_set: int, count: int | None = None) -> np.ndarray:
    """Token activations [count, hidden] as bf16 bits, iid N(0,1)."""
    count = cfg.tokens if count is None else count
    out = np.empty((count, cfg.hidden), dtype=np.uint16)
    for t in range(count):
        k = stream_key(cfg.seed, token_set, t, T_TOKEN, 0)
        out[t] = gaussian_bf16(k, cfg.hidden, 1.0)
    return out


def bf16_to_f64(a: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 exactly."""
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def with_changes(cfg: MoEConfig, **kw) -> MoEConfig:
    return replace(cfg, **kw)


# ---------------------------------------------------------------- device twin

_DEV_SO = os.path.join(_HERE, "libsynth_device.so")
_dev_lib = None


def build_device(force: bool = True) -> str:
    """Compile the HIP twin of the generator (gfx950)."""
    src = os.path.join(_HERE, "synth_device.hip")
    if force or not os.path.exists(_DEV_SO) or os.path.getmtime(_DEV_SO) < os.path.getmtime(src):
        tmp = _DEV_SO + ".tmp%d" % os.getpid()
        hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
        subprocess.check_call([hipcc, "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
                               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                               "-o", tmp, src], stderr=subprocess.DEVNULL)
        os.replace(tmp, _DEV_SO)
    return _DEV_SO


def dev_lib() -> ctypes.CDLL:
    global _dev_lib
    if _dev_lib is None:
        if not os.path.exists(_DEV_SO):
            raise ImportError(f"{_DEV_SO} is missing: call synth.build_device()")
        L = ctypes.CDLL(_DEV_SO)
        L.synth_device_fill_experts.restype = ctypes.c_int
        L.synth_device_fill_experts.argtypes = [ctypes.POINTER(_Spec), ctypes.c_uint32,
                                                ctypes.c_uint32, ctypes.c_int32, ctypes.c_int64,
                                                ctypes.c_void_p, ctypes.c_void_p]
        _dev_lib = L
    return _dev_lib


def device_fill_experts(cfg: MoEConfig, layer: int, out_ptr: int, stride: int,
                        first_expert: int = 0, count: int | None = None, stream: int = 0):
    """Fill blobs [first, first+count) of a layer into device memory at
    out_ptr + i*stride, asynchronously on `stream` (a hipStream_t value)."""
    count = cfg.n_slots - first_expert if count is None else count
    s = spec(cfg)
    rc = dev_lib().synth_device_fill_experts(ctypes.byref(s), layer, first_expert, count, stride,
                                             out_ptr, stream)
    if rc != 0:
        raise RuntimeError(f"synth_device_fill_experts failed with hipError {rc}")
