"""ctypes marshalling for libmoeq.so.  No arithmetic of the path lives here."""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_PKG, "libmoeq.so")

BF16, F32 = 0, 1
F_NO_RENORM, F_RMSNORM, F_STACK_LAYERWISE, F_STACK_NO_NORM, F_STACK_JITTER = 1, 2, 4, 8, 16

OK, E_INVALID, E_UNSUPPORTED, E_HIP, E_POOL_EXHAUSTED, E_DEVICE = 0, -1, -2, -3, -4, -5
_CODE_NAMES = {E_INVALID: "MOEQ_E_INVALID", E_UNSUPPORTED: "MOEQ_E_UNSUPPORTED", E_HIP: "MOEQ_E_HIP",
               E_POOL_EXHAUSTED: "MOEQ_E_POOL_EXHAUSTED", E_DEVICE: "MOEQ_E_DEVICE"}


class MoeqError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_CODE_NAMES.get(code, code)}: {msg}")
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("group", ctypes.c_int32)]

    @classmethod
    def of(cls, cfg) -> "Shape":
        return cls(cfg.hidden, cfg.inter, cfg.n_experts, cfg.n_shared, cfg.bits, cfg.group)

    @property
    def n_slots(self) -> int:
        return self.n_experts + self.n_shared


class _Experts(ctypes.Structure):
    _fields_ = [("blobs", ctypes.c_void_p), ("n_layers", ctypes.c_int32)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_lib = None


def library_path() -> str:
    return _SO


def lib() -> ctypes.CDLL:
    """Load libmoeq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            raise ImportError(f"{_SO} is missing: build it with "
                              "`python -m quantized_expert_gemv_router_amd.build`")
        L = ctypes.CDLL(_SO)
        S = ctypes.POINTER(Shape)
        X = ctypes.POINTER(_Experts)
        L.moeq_abi_version.restype = _I
        L.moeq_last_error.restype = ctypes.c_char_p
        L.moeq_expert_bytes.restype = ctypes.c_int64
        L.moeq_expert_bytes.argtypes = [S]
        L.moeq_workspace_bytes.argtypes = [S, _I, _I, ctypes.POINTER(ctypes.c_int64)]
        L.moe_router_topk.argtypes = [S, _P, _I, ctypes.c_uint32, _P, _P, _I, _I, _P, _P, _P, _P, _P, _P]
        L.moe_q4_expert_gemv.argtypes = [S, X, _I, _P, _I, ctypes.c_uint32, _P, _I, _I, _P, _P, _P]
        L.moe_swiglu_down_combine.argtypes = [S, X, _I, _P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P]
        L.moe_read_device_status.argtypes = [_P, _P, ctypes.POINTER(ctypes.c_int32)]
        L.moeq_last_stack_path.restype = _I
        L.moeq_stack_clock_trace.argtypes = [_P]
        L.moeq_stack_block_clock_trace.argtypes = [_P]
        L.moe_expert_stack_decode.argtypes = [S, X, _P, _I, _I, _I, _I, ctypes.c_uint32, _P, _P, _P,
                                              _P, _P]
        L.moe_expert_stack_decode_mixed.argtypes = [S, _P, X, _P, _I, _I, _I, _I, ctypes.c_uint32, _P, _P, _P,
                                                    _P, _P]
        L.moe_expert_stack_decode_noalloc.argtypes = [S, X, _P, _I, _I, _I, _I, ctypes.c_uint32, _P, _P, _P,
                                                      _P, _P]
        L.moe_expert_stack_prefill.argtypes = [S, X, _P, _I, _I, _I, _I, ctypes.c_uint32, _P, _P, _P, _P]
        L.moeq_prefill_workspace_bytes.argtypes = [S, _I, _I, ctypes.POINTER(ctypes.c_int64)]
        L.moeq_prefill_timing.argtypes = [_I]
        L.moeq_prefill_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)]
        H = ctypes.POINTER(ctypes.c_void_p)
        I64 = ctypes.c_int64
        L.moe_pool_create.argtypes = [S, _I, _P, I64, I64, _P, _P, _P, _I, H]
        L.moe_pool_make_resident.argtypes = [_P, _P]
        L.moe_pool_acquire.argtypes = [_P, _I, _P, _I, _P, X]
        L.moe_pool_release.argtypes = [_P, _I, _P]
        L.moe_pool_prefetch.argtypes = [_P, _I, _P, _I]
        L.moeq_poolsim_prefetch.argtypes = [_P, _I, _P, _I, _P, _P, ctypes.POINTER(ctypes.c_int32)]
        L.moe_pool_stats.argtypes = [_P, ctypes.POINTER(I64)]
        L.moe_pool_destroy.argtypes = [_P]
        L.moe_pool_destroy.restype = None
        L.moeq_poolsim_create.argtypes = [_I, _I, I64, H]
        L.moeq_poolsim_make_resident.argtypes = [_P]
        L.moeq_poolsim_acquire.argtypes = [_P, _I, _P, _I, _P, _P, _P, ctypes.POINTER(ctypes.c_int32)]
        L.moeq_poolsim_release.argtypes = [_P, _I]
        L.moeq_poolsim_stats.argtypes = [_P, ctypes.POINTER(I64)]
        L.moeq_poolsim_destroy.argtypes = [_P]
        L.moeq_poolsim_destroy.restype = None
        L.moeq_probe_scratch_bytes.restype = I64
        L.moeq_probe_scratch_bytes.argtypes = [_I, _I]
        L.moeq_probe_handoff.argtypes = [_I, _I, _I, _I, _I, _I, _P, I64, ctypes.POINTER(I64),
                                         ctypes.POINTER(I64), _P, _P]
        _lib = L
    return _lib


def _check(rc: int):
    if rc != OK:
        raise MoeqError(rc, lib().moeq_last_error().decode())


def moeq_abi_version() -> int:
    return lib().moeq_abi_version()


def moeq_last_error() -> str:
    return lib().moeq_last_error().decode()


def moeq_expert_bytes(shape: Shape) -> int:
    return lib().moeq_expert_bytes(ctypes.byref(shape))


def moeq_workspace_bytes(shape: Shape, T: int, k: int) -> int:
    out = ctypes.c_int64()
    _check(lib().moeq_workspace_bytes(ctypes.byref(shape), T, k, ctypes.byref(out)))
    return out.value


def new_workspace(shape: Shape, T: int, k: int, device="cuda") -> torch.Tensor:
    """Zero-filled workspace of moeq_workspace_bytes(shape, T, k) bytes."""
    return torch.zeros(moeq_workspace_bytes(shape, T, k), dtype=torch.uint8, device=device)


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoeq must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"unsupported activation dtype {t.dtype}")


class ExpertTable:
    """Device table of expert blob pointers, [n_layers][n_experts + n_shared]
    (the `moeq_experts` view).  Built from per-layer uint8 arenas whose slot
    e holds expert e's blob at byte offset e * stride."""

    def __init__(self, shape: Shape, arenas: list, stride: int, device="cuda"):
        ptrs = []
        for arena in arenas:
            base = arena.data_ptr()
            ptrs.extend(base + e * stride for e in range(shape.n_slots))
        self.table = torch.tensor(ptrs, dtype=torch.int64, device=device)
        self.arenas = arenas
        self.n_layers = len(arenas)
        self._view = _Experts(self.table.data_ptr(), self.n_layers)

    @classmethod
    def from_pointers(cls, ptr_table: torch.Tensor, n_layers: int):
        self = cls.__new__(cls)
        self.table = ptr_table
        self.arenas = []
        self.n_layers = n_layers
        self._view = _Experts(ptr_table.data_ptr(), n_layers)
        return self

    def view(self):
        return ctypes.byref(self._view)


def moe_router_topk(shape: Shape, x: torch.Tensor, w_router: torch.Tensor, k: int, flags: int = 0,
                    shared_gate: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                    want_logits: bool = False, out=None, stream=None):
    """Returns (topk_idx int32 [T,k], topk_w f32 [T,k], shared_w f32 [T], logits f64 [T,E] | None)."""
    T = x.shape[0]
    dev = x.device
    if workspace is None:
        workspace = new_workspace(shape, T, k, dev)
    if out is None:
        idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        sw = torch.empty((T,), dtype=torch.float32, device=dev)
    else:
        idx, w, sw = out
    logits = torch.empty((T, shape.n_experts), dtype=torch.float64, device=dev) if want_logits else None
    _check(lib().moe_router_topk(ctypes.byref(shape), _ptr(x), _dtype_code(x), flags, _ptr(w_router),
                                 _ptr(shared_gate), T, k, _ptr(idx), _ptr(w),
                                 _ptr(sw) if shape.n_shared else None, _ptr(logits),
                                 _ptr(workspace), _stream(stream)))
    return idx, w, sw, logits


def moe_q4_expert_gemv(shape: Shape, experts: ExpertTable, layer: int, x: torch.Tensor,
                       topk_idx: torch.Tensor, k: int, flags: int = 0,
                       workspace: torch.Tensor | None = None, gate_up: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """gate_up f32 [T, k + S, 2, I] (slot k = shared expert)."""
    T = x.shape[0]
    if workspace is None:
        workspace = new_workspace(shape, T, k, x.device)
    if gate_up is None:
        gate_up = torch.empty((T, k + shape.n_shared, 2, shape.inter), dtype=torch.float32,
                              device=x.device)
    _check(lib().moe_q4_expert_gemv(ctypes.byref(shape), experts.view(), layer, _ptr(x),
                                    _dtype_code(x), flags, _ptr(topk_idx), T, k, _ptr(workspace),
                                    _ptr(gate_up), _stream(stream)))
    return gate_up


def moe_swiglu_down_combine(shape: Shape, experts: ExpertTable, layer: int, gate_up: torch.Tensor,
                            topk_idx: torch.Tensor, topk_w: torch.Tensor,
                            shared_w: torch.Tensor | None, residual: torch.Tensor, k: int,
                            workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                            stream=None) -> torch.Tensor:
    """out f32 [T, H] = residual + sum_k w_k d_k + shared_w * d_shared."""
    T = residual.shape[0]
    if workspace is None:
        workspace = new_workspace(shape, T, k, residual.device)
    if out is None:
        out = torch.empty((T, shape.hidden), dtype=torch.float32, device=residual.device)
    _check(lib().moe_swiglu_down_combine(ctypes.byref(shape), experts.view(), layer, _ptr(gate_up),
                                         _ptr(topk_idx), _ptr(topk_w), _ptr(shared_w),
                                         _ptr(residual), _dtype_code(residual), T, k,
                                         _ptr(workspace), _ptr(out), _stream(stream)))
    return out


class RouterTable:
    """Device array of per-layer router matrix pointers ([E][H] bf16 each)."""

    def __init__(self, routers: list, device="cuda"):
        self.routers = routers
        self.table = torch.tensor([r.data_ptr() for r in routers], dtype=torch.int64, device=device)

    def ptr(self):
        return self.table.data_ptr()


def moe_expert_stack_decode(shape: Shape, experts: ExpertTable, routers: RouterTable, h: torch.Tensor,
                            k: int, layer0: int = 0, L: int | None = None, flags: int = 0,
                            workspace: torch.Tensor | None = None, trace: bool = False, stream=None):
    """Run layers [layer0, layer0 + L) in place on h (f32 [T, H]).  Returns
    (topk_trace int32 [L, T, k], h_trace f32 [L, T, H]) when trace, else None."""
    T = h.shape[0]
    L = experts.n_layers - layer0 if L is None else L
    if h.dtype != torch.float32:
        raise ValueError("the stack runs on an fp32 residual stream")
    if workspace is None:
        workspace = new_workspace(shape, T, k, h.device)
    tk = hk = None
    if trace:
        tk = torch.empty((L, T, k), dtype=torch.int32, device=h.device)
        hk = torch.empty((L, T, shape.hidden), dtype=torch.float32, device=h.device)
    _check(lib().moe_expert_stack_decode(ctypes.byref(shape), experts.view(), routers.ptr(), layer0, L, T,
                                         k, flags, _ptr(h), _ptr(tk), _ptr(hk), _ptr(workspace),
                                         _stream(stream)))
    return (tk, hk) if trace else None


def moe_expert_stack_decode_mixed(shape: Shape, layer_bits, experts: ExpertTable, routers: RouterTable,
                                  h: torch.Tensor, k: int, layer0: int = 0, flags: int = 0,
                                  workspace: torch.Tensor | None = None, trace: bool = False, stream=None):
    """moe_expert_stack_decode over layers of different widths: layer_bits[l]
    bits for layer layer0 + l.  Returns (topk_trace, h_trace) when trace."""
    T = h.shape[0]
    L = len(layer_bits)
    if workspace is None:
        workspace = new_workspace(shape, T, k, h.device)
    bits = (ctypes.c_int32 * max(L, 1))(*[int(b) for b in layer_bits])
    tk = hk = None
    if trace:
        tk = torch.empty((L, T, k), dtype=torch.int32, device=h.device)
        hk = torch.empty((L, T, shape.hidden), dtype=torch.float32, device=h.device)
    _check(lib().moe_expert_stack_decode_mixed(ctypes.byref(shape), ctypes.cast(bits, _P), experts.view(),
                                               routers.ptr(), layer0, L, T, k, flags, _ptr(h), _ptr(tk), _ptr(hk),
                                               _ptr(workspace), _stream(stream)))
    return (tk, hk) if trace else None


def moe_expert_stack_decode_noalloc(shape: Shape, experts: ExpertTable, routers: RouterTable, h: torch.Tensor,
                                    k: int, layer0: int = 0, L: int | None = None, flags: int = 0,
                                    trace: bool = False, status: torch.Tensor | None = None, stream=None):
    """moe_expert_stack_decode on the library's static scratch (no workspace,
    no allocation by the library).  `status`: optional int32 device tensor [1]
    that receives the call's status word."""
    T = h.shape[0]
    L = experts.n_layers - layer0 if L is None else L
    if h.dtype != torch.float32:
        raise ValueError("the stack runs on an fp32 residual stream")
    tk = hk = None
    if trace:
        tk = torch.empty((L, T, k), dtype=torch.int32, device=h.device)
        hk = torch.empty((L, T, shape.hidden), dtype=torch.float32, device=h.device)
    _check(lib().moe_expert_stack_decode_noalloc(ctypes.byref(shape), experts.view(), routers.ptr(), layer0, L,
                                                 T, k, flags, _ptr(h), _ptr(tk), _ptr(hk), _ptr(status),
                                                 _stream(stream)))
    return (tk, hk) if trace else None


def moeq_prefill_workspace_bytes(shape: Shape, T: int, k: int) -> int:
    out = ctypes.c_int64()
    _check(lib().moeq_prefill_workspace_bytes(ctypes.byref(shape), T, k, ctypes.byref(out)))
    return out.value


def new_prefill_workspace(shape: Shape, T: int, k: int, device="cuda") -> torch.Tensor:
    """Zero-filled workspace of moeq_prefill_workspace_bytes(shape, T, k) bytes."""
    return torch.zeros(moeq_prefill_workspace_bytes(shape, T, k), dtype=torch.uint8, device=device)


def moe_expert_stack_prefill(shape: Shape, experts, routers: RouterTable, h: torch.Tensor, k: int,
                             layer0: int = 0, L: int | None = None, flags: int = 0,
                             workspace: torch.Tensor | None = None, trace: bool = False, stream=None):
    """Prefill layers [layer0, layer0 + L) in place on h (f32 [T, H]).
    Returns topk_trace int32 [L, T, k] when trace, else None."""
    T = h.shape[0]
    L = experts.n_layers - layer0 if L is None else L
    if h.dtype != torch.float32:
        raise ValueError("the stack runs on an fp32 residual stream")
    if workspace is None:
        workspace = new_prefill_workspace(shape, T, k, h.device)
    tk = torch.empty((L, T, k), dtype=torch.int32, device=h.device) if trace else None
    _check(lib().moe_expert_stack_prefill(ctypes.byref(shape), experts.view(), routers.ptr(), layer0, L, T, k,
                                          flags, _ptr(h), _ptr(tk), _ptr(workspace), _stream(stream)))
    return tk


PREFILL_KERNELS = ("norm", "router", "topk", "group", "gate_up", "down", "combine")


def moeq_prefill_timing(enable: bool = True):
    _check(lib().moeq_prefill_timing(int(enable)))


def moeq_prefill_timing_read() -> dict:
    """{class: (summed ms, launches)} of the prefill kernels timed so far."""
    ms = (ctypes.c_double * 7)()
    n = (ctypes.c_int32 * 7)()
    _check(lib().moeq_prefill_timing_read(ms, n))
    return {k: (ms[i], n[i]) for i, k in enumerate(PREFILL_KERNELS)}


def moeq_last_stack_path() -> int:
    """1 = the last stack call ran the persistent launch, 2 = per-layer launches."""
    return lib().moeq_last_stack_path()


def moeq_stack_clock_trace(clocks: torch.Tensor) -> int:
    """Arm the diagnostic phase clock trace (int64 device tensor [L, 24])."""
    return lib().moeq_stack_clock_trace(_ptr(clocks))


def moeq_stack_block_clock_trace(clocks: torch.Tensor) -> int:
    """Arm the diagnostic per-block clock trace (int64 device tensor [blocks, L, 16])."""
    return lib().moeq_stack_block_clock_trace(_ptr(clocks))


def moeq_probe_handoff(mode: int, words_per_block: int, rounds: int, sleep: int = 1, peer: int = 1,
                       stride: int | None = None, stream=None) -> dict:
    """Diagnostic hand-off probe: {ticks (100 MHz) of all rounds, stale payload
    words, XCD id of each workgroup}."""
    stride = words_per_block if stride is None else stride
    nbytes = lib().moeq_probe_scratch_bytes(words_per_block, stride)
    if nbytes < 0:
        raise MoeqError(E_INVALID, "moeq_probe_scratch_bytes failed")
    scratch = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ticks, bad = ctypes.c_int64(), ctypes.c_int64()
    xcc = (ctypes.c_int32 * 1024)()
    _check(lib().moeq_probe_handoff(mode, words_per_block, stride, rounds, sleep, peer, _ptr(scratch), nbytes,
                                    ctypes.byref(ticks), ctypes.byref(bad), ctypes.cast(xcc, _P),
                                    _stream(stream)))
    n = torch.cuda.get_device_properties(0).multi_processor_count
    return dict(ticks=ticks.value, stale=bad.value, xcc=list(xcc[:n]))


def moe_read_device_status(workspace: torch.Tensor, stream=None) -> int:
    st = ctypes.c_int32()
    _check(lib().moe_read_device_status(_ptr(workspace), _stream(stream), ctypes.byref(st)))
    return st.value


def moe_layer(shape: Shape, experts: ExpertTable, layer: int, x: torch.Tensor,
              w_router: torch.Tensor, k: int, flags: int = 0, shared_gate=None, workspace=None,
              stream=None) -> dict:
    """The three calls of one decode layer, in order, on one stream."""
    T = x.shape[0]
    if workspace is None:
        workspace = new_workspace(shape, T, k, x.device)
    idx, w, sw, logits = moe_router_topk(shape, x, w_router, k, flags, shared_gate, workspace,
                                         want_logits=True, stream=stream)
    gu = moe_q4_expert_gemv(shape, experts, layer, x, idx, k, flags, workspace, stream=stream)
    out = moe_swiglu_down_combine(shape, experts, layer, gu, idx, w,
                                  sw if shape.n_shared else None, x, k, workspace, stream=stream)
    return dict(idx=idx, w=w, shared_w=sw, logits=logits, gate_up=gu, y=out)


_STATS = ("hits", "misses", "bytes_copied", "evictions")


def _int32_host(ids) -> ctypes.Array:
    vals = [int(v) for v in ids]
    return (ctypes.c_int32 * max(len(vals), 1))(*vals)


class PoolView:
    """The moeq_experts view a pool acquire returns (the pool's pointer table)."""

    def __init__(self, ex: _Experts, pool):
        self._ex = ex
        self.pool = pool
        self.n_layers = ex.n_layers

    def view(self):
        return ctypes.byref(self._ex)


class Pool:
    """moe_pool_*: expert slots in a device arena, filled on demand from pinned
    host blobs, least recently used slot evicted.  `host` is either one
    pinned uint8 CPU tensor laid out blob (l, e) at (l * (E + S) + e) *
    slot_bytes, or a list of per-layer pinned tensors [E + S slots of
    slot_bytes], or a list of n_layers * (E + S) host addresses of pinned
    blobs; `table` an int64 device tensor of n_layers * (E + S) entries (the
    pointer table the pool writes); `copy_stream` one stream or a list of
    them (misses are spread over them)."""

    def __init__(self, shape: Shape, n_layers: int, arena: torch.Tensor, n_slots: int, slot_bytes: int,
                 host, table: torch.Tensor, copy_stream=None):
        self._h = ctypes.c_void_p()
        self.shape, self.arena, self.host, self.table = shape, arena, host, table
        per = shape.n_slots
        if isinstance(host, torch.Tensor):
            base = host.data_ptr()
            ptrs = [base + i * slot_bytes for i in range(n_layers * per)]
        elif len(host) and isinstance(host[0], torch.Tensor):
            ptrs = [t.data_ptr() + e * slot_bytes for t in host for e in range(per)]
        else:
            ptrs = [int(v) for v in host]
        if len(ptrs) != n_layers * per:
            raise ValueError(f"host blobs: {len(ptrs)} given, {n_layers * per} needed")
        self._ptrs = (ctypes.c_void_p * len(ptrs))(*ptrs)
        streams = copy_stream if isinstance(copy_stream, (list, tuple)) else [copy_stream]
        self.copy_streams = streams
        self._streams = (ctypes.c_void_p * len(streams))(*[_stream(st) for st in streams])
        _check(lib().moe_pool_create(ctypes.byref(shape), n_layers, _ptr(arena), n_slots, slot_bytes,
                                     ctypes.cast(self._ptrs, _P), _ptr(table), ctypes.cast(self._streams, _P),
                                     len(streams), ctypes.byref(self._h)))

    def make_resident(self, stream=None):
        _check(lib().moe_pool_make_resident(self._h, _stream(stream)))

    def acquire(self, layer: int, ids, stream=None) -> PoolView:
        arr = _int32_host(ids)
        ex = _Experts()
        _check(lib().moe_pool_acquire(self._h, layer, ctypes.cast(arr, _P), len(ids), _stream(stream),
                                      ctypes.byref(ex)))
        return PoolView(ex, self)

    def release(self, layer: int, stream=None):
        _check(lib().moe_pool_release(self._h, layer, _stream(stream)))

    def prefetch(self, layer: int, ids):
        arr = _int32_host(ids)
        _check(lib().moe_pool_prefetch(self._h, layer, ctypes.cast(arr, _P), len(ids)))

    def stats(self) -> dict:
        out = (ctypes.c_int64 * 4)()
        _check(lib().moe_pool_stats(self._h, out))
        return dict(zip(_STATS, list(out)))

    def destroy(self):
        if self._h:
            lib().moe_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


class PoolSim:
    """moeq_poolsim_*: the pool's placement and eviction decisions alone."""

    def __init__(self, n_layers: int, per_layer: int, n_slots: int):
        self._h = ctypes.c_void_p()
        _check(lib().moeq_poolsim_create(n_layers, per_layer, n_slots, ctypes.byref(self._h)))

    def make_resident(self):
        _check(lib().moeq_poolsim_make_resident(self._h))

    def acquire(self, layer: int, ids) -> list:
        """[(slot, evicted entry or -1, missed)] per distinct id, first-appearance order."""
        n = len(ids)
        arr = _int32_host(ids)
        slots, ev, miss = ((ctypes.c_int32 * max(n, 1))() for _ in range(3))
        n_out = ctypes.c_int32()
        _check(lib().moeq_poolsim_acquire(self._h, layer, ctypes.cast(arr, _P), n, slots, ev, miss,
                                          ctypes.byref(n_out)))
        return [(slots[i], ev[i], bool(miss[i])) for i in range(n_out.value)]

    def prefetch(self, layer: int, ids) -> list:
        """[(slot, evicted entry or -1)] per copy the prefetch plans."""
        n = len(ids)
        arr = _int32_host(ids)
        slots, ev = ((ctypes.c_int32 * max(n, 1))() for _ in range(2))
        n_out = ctypes.c_int32()
        _check(lib().moeq_poolsim_prefetch(self._h, layer, ctypes.cast(arr, _P), n, slots, ev, ctypes.byref(n_out)))
        return [(slots[i], ev[i]) for i in range(n_out.value)]

    def release(self, layer: int):
        _check(lib().moeq_poolsim_release(self._h, layer))

    def stats(self) -> dict:
        out = (ctypes.c_int64 * 4)()
        _check(lib().moeq_poolsim_stats(self._h, out))
        return dict(zip(_STATS, list(out)))

    def __del__(self):
        try:
            if self._h:
                lib().moeq_poolsim_destroy(self._h)
        except Exception:
            pass
