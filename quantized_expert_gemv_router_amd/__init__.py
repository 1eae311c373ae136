"""quantized_expert_gemv_router_amd: the quantized MoE expert forward at
decode on AMD MI355X (gfx950).

This package is a thin ctypes binding over libmoeq.so (HIP kernels + C ABI,
declared in include/moeq.h).  The functions keep the C names and only
marshal arguments: torch tensors provide device memory and the current HIP
stream; every step of the path runs in the library's kernels.  If the
library has not been built the import of the binding functions fails
loudly; there is no CPU fallback.
"""
from ._binding import (  # noqa: F401
    BF16, F32, F_NO_RENORM, F_RMSNORM, F_STACK_LAYERWISE, F_STACK_NO_NORM, F_STACK_JITTER,
    MoeqError, E_UNSUPPORTED, Shape, ExpertTable, RouterTable, lib, library_path,
    moeq_abi_version, moeq_expert_bytes, moeq_workspace_bytes, moeq_last_error,
    moe_router_topk, moe_q4_expert_gemv, moe_swiglu_down_combine, moe_read_device_status,
    moe_expert_stack_decode, moe_expert_stack_decode_mixed, moe_expert_stack_decode_noalloc, moeq_last_stack_path, moeq_stack_clock_trace, moeq_stack_block_clock_trace,
    new_workspace, moe_layer, Pool, PoolSim, PoolView,
    moe_expert_stack_prefill, moeq_prefill_workspace_bytes, new_prefill_workspace,
    moeq_prefill_timing, moeq_prefill_timing_read, PREFILL_KERNELS, moeq_probe_handoff,
)
