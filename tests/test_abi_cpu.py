"""CPU checks of the C ABI: the library loads, exports every function the
headers declare, and refuses bad or unsupported arguments with the
documented codes before touching the GPU."""
import ctypes
import os
import re

import pytest

import quantized_expert_gemv_router_amd as q
import synth
from quantized_expert_gemv_router_amd._binding import E_INVALID, E_UNSUPPORTED, OK, _Experts

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    inc = os.path.join(ROOT, "include")
    for f in sorted(os.listdir(inc)):
        if not f.endswith(".h"):
            continue
        text = open(os.path.join(inc, f)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(moe\w*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert "moe_router_topk" in names and "moe_q4_expert_gemv" in names
    assert "moe_swiglu_down_combine" in names
    L = q.lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_expert_bytes():
    assert q.moeq_expert_bytes(q.Shape(4096, 1024, 512, 1, 4, 64)) == 7_077_888
    assert q.moeq_expert_bytes(q.Shape(4096, 1024, 512, 1, 2, 64)) == 3_932_160
    assert q.moeq_expert_bytes(q.Shape(256, 128, 8, 1, 4, 64)) == 55_296
    assert q.moeq_expert_bytes(q.Shape(4096, 1024, 512, 1, 3, 64)) == 5_505_024
    assert q.moeq_expert_bytes(q.Shape(4096, 1024, 512, 1, 5, 64)) == -1
    assert q.moeq_expert_bytes(q.Shape(4096, 1088, 512, 1, 3, 64)) == -1   # 3-bit rows need multiples of 128
    for cfg in synth.CONFIGS.values():
        assert q.moeq_expert_bytes(q.Shape.of(cfg)) == cfg.expert_bytes


def _ws(shape, T, k):
    out = ctypes.c_int64()
    rc = q.lib().moeq_workspace_bytes(ctypes.byref(shape), T, k, ctypes.byref(out))
    return rc, out.value


@pytest.mark.parametrize("shape,T,k,code", [
    ((4096, 1024, 512, 1, 4, 64), 1, 3, OK),
    ((4096, 1024, 512, 1, 2, 64), 16, 10, OK),
    ((4096, 1024, 512, 1, 4, 64), -1, 3, E_INVALID),
    ((4096, 1024, 512, 1, 4, 64), 1, -1, E_INVALID),
    ((4096, 1024, 8, 1, 4, 64), 1, 9, E_INVALID),
    ((4096, 1024, 512, 1, 4, 64), 1, 17, E_UNSUPPORTED),
    ((4096, 1024, 512, 1, 4, 64), 65, 3, E_UNSUPPORTED),
    ((4096, 1024, 512, 1, 3, 64), 1, 3, OK),
    ((4096, 1088, 512, 1, 3, 64), 1, 3, E_UNSUPPORTED),
    ((4096, 1024, 512, 1, 5, 64), 1, 3, E_UNSUPPORTED),
    ((4096, 1024, 512, 1, 8, 64), 1, 3, E_UNSUPPORTED),
    ((4096, 1024, 512, 1, 4, 32), 1, 3, E_UNSUPPORTED),
    ((4100, 1024, 512, 1, 4, 64), 1, 3, E_UNSUPPORTED),
    ((4096, 1000, 512, 1, 4, 64), 1, 3, E_UNSUPPORTED),
    ((16384, 1024, 512, 1, 4, 64), 1, 3, E_UNSUPPORTED),
    ((4096, 1024, 8192, 1, 4, 64), 1, 3, E_UNSUPPORTED),
    ((4096, 1024, 512, 2, 4, 64), 1, 3, E_UNSUPPORTED),
    ((0, 1024, 512, 1, 4, 64), 1, 3, E_INVALID),
])
def test_workspace_validation(shape, T, k, code):
    rc, nbytes = _ws(q.Shape(*shape), T, k)
    assert rc == code, q.moeq_last_error()
    if code == OK:
        assert nbytes > 0 and q.moeq_last_error() == ""
    else:
        assert q.moeq_last_error() != ""


def test_workspace_grows_with_batch():
    s = q.Shape(4096, 1024, 512, 1, 4, 64)
    assert _ws(s, 16, 10)[1] > _ws(s, 1, 3)[1]


def test_router_validation_without_gpu():
    L = q.lib()
    s = q.Shape(4096, 1024, 512, 1, 4, 64)
    fake = ctypes.c_void_p(0x1000)
    # T == 0 is a no-op and succeeds without touching the device
    assert L.moe_router_topk(ctypes.byref(s), fake, 0, 0, fake, None, 0, 3, fake, fake, None, None,
                             fake, None) == OK
    assert L.moe_router_topk(ctypes.byref(s), None, 0, 0, fake, None, 1, 3, fake, fake, None, None,
                             fake, None) == E_INVALID
    assert L.moe_router_topk(ctypes.byref(s), fake, 7, 0, fake, None, 1, 3, fake, fake, None, None,
                             fake, None) == E_UNSUPPORTED
    assert L.moe_router_topk(ctypes.byref(s), fake, 0, 0x80, fake, None, 1, 3, fake, fake, None,
                             None, fake, None) == E_UNSUPPORTED
    assert "flag" in q.moeq_last_error()
    assert L.moe_router_topk(ctypes.byref(s), fake, 0, 0, fake, None, 1, 0, fake, fake, None, None,
                             fake, None) == E_INVALID
    s0 = q.Shape(4096, 1024, 512, 0, 4, 64)
    assert L.moe_router_topk(ctypes.byref(s0), fake, 0, 0, fake, fake, 1, 3, fake, fake, None,
                             None, fake, None) == E_INVALID


def test_expert_call_validation_without_gpu():
    L = q.lib()
    s = q.Shape(4096, 1024, 512, 1, 4, 64)
    fake = ctypes.c_void_p(0x1000)
    ex = _Experts(0x2000, 2)
    assert L.moe_q4_expert_gemv(ctypes.byref(s), None, 0, fake, 0, 0, fake, 1, 3, fake, fake,
                                None) == E_INVALID
    assert L.moe_q4_expert_gemv(ctypes.byref(s), ctypes.byref(ex), 2, fake, 0, 0, fake, 1, 3, fake,
                                fake, None) == E_INVALID
    assert L.moe_q4_expert_gemv(ctypes.byref(s), ctypes.byref(ex), 0, fake, 0, 0, fake, 0, 3, fake,
                                fake, None) == OK
    assert L.moe_swiglu_down_combine(ctypes.byref(s), ctypes.byref(ex), 0, fake, fake, fake, None,
                                     fake, 9, 1, 3, fake, fake, None) == E_UNSUPPORTED
    assert L.moe_swiglu_down_combine(ctypes.byref(s), ctypes.byref(ex), 0, None, fake, fake, None,
                                     fake, 1, 1, 3, fake, fake, None) == E_INVALID
    assert L.moe_swiglu_down_combine(ctypes.byref(s), ctypes.byref(ex), 0, fake, fake, fake, None,
                                     fake, 1, 0, 3, fake, fake, None) == OK
    s0 = q.Shape(4096, 1024, 512, 0, 4, 64)
    assert L.moe_swiglu_down_combine(ctypes.byref(s0), ctypes.byref(ex), 0, fake, fake, fake, None,
                                     fake, 1, 1, 0, fake, fake, None) == E_UNSUPPORTED


def test_abi_version():
    assert q.moeq_abi_version() >= 1


def test_noalloc_rejects_workspace_above_static_scratch_without_gpu():
    """The allocation-free stack decode refuses shapes whose workspace does not
    fit its static scratch (before any device call), and bad counts."""
    L = q.lib()
    big = q.Shape(8192, 8192, 4096, 1, 4, 64)
    assert L.moe_expert_stack_decode_noalloc(ctypes.byref(big), None, None, 0, 1, 64, 16, 0, None, None,
                                             None, None, None) == E_UNSUPPORTED
    assert b"static scratch" in L.moeq_last_error()
    s = q.Shape(4096, 1024, 512, 1, 4, 64)
    assert L.moe_expert_stack_decode_noalloc(ctypes.byref(s), None, None, 0, 1, -1, 3, 0, None, None,
                                             None, None, None) == E_INVALID
    assert L.moe_expert_stack_decode_noalloc(ctypes.byref(s), None, None, 0, 1, 1, 17, 0, None, None,
                                             None, None, None) == E_UNSUPPORTED
