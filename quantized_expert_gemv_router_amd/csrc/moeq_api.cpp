// C-ABI entry points of libmoeq: argument validation, workspace layout and
// kernel dispatch.  The arithmetic lives in the .hip kernels.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "moeq.h"
#include "moeq_internal.hpp"

namespace moeq {

namespace {
thread_local std::string g_last_error;
thread_local int g_last_stack_path = 0;
thread_local int64_t* g_stack_clocks = nullptr;   // diagnostic phase stamps for this thread's next persistent launch
thread_local int64_t* g_stack_bclocks = nullptr;  // the same, every block
}  // namespace

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return MOEQ_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MOEQ_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

int check_shape(const moeq_shape* s) {
  if (!s) return fail(MOEQ_E_INVALID, "shape is NULL");
  if (s->hidden <= 0 || s->inter <= 0 || s->n_experts <= 0 || s->n_shared < 0)
    return fail(MOEQ_E_INVALID, "shape sizes must be positive (hidden=%d inter=%d n_experts=%d n_shared=%d)",
                s->hidden, s->inter, s->n_experts, s->n_shared);
  if (s->bits != 4 && s->bits != 3 && s->bits != 2)
    return fail(MOEQ_E_UNSUPPORTED, "bits=%d: only 4-, 3- and 2-bit experts are implemented", s->bits);
  if (s->group != 64)
    return fail(MOEQ_E_UNSUPPORTED, "group=%d: only groups of 64 are implemented", s->group);
  if (s->hidden % 64 || s->inter % 64)
    return fail(MOEQ_E_UNSUPPORTED, "hidden=%d inter=%d must be multiples of 64", s->hidden, s->inter);
  if (s->bits == 3 && (s->hidden % 128 || s->inter % 128))
    return fail(MOEQ_E_UNSUPPORTED, "3-bit experts need hidden=%d and inter=%d to be multiples of 128 "
                "(16-byte aligned rows)", s->hidden, s->inter);
  if (s->hidden > MOEQ_MAX_HIDDEN || s->inter > MOEQ_MAX_INTER)
    return fail(MOEQ_E_UNSUPPORTED, "hidden=%d inter=%d exceed %d/%d", s->hidden, s->inter,
                MOEQ_MAX_HIDDEN, MOEQ_MAX_INTER);
  if (s->n_experts > MOEQ_MAX_EXPERTS)
    return fail(MOEQ_E_UNSUPPORTED, "n_experts=%d exceeds %d", s->n_experts, MOEQ_MAX_EXPERTS);
  if (s->n_shared > 1)
    return fail(MOEQ_E_UNSUPPORTED, "n_shared=%d: at most one shared expert", s->n_shared);
  return MOEQ_OK;
}

namespace {

int check_tk(const moeq_shape* s, int T, int k) {
  if (T < 0) return fail(MOEQ_E_INVALID, "T=%d is negative", T);
  if (k < 0) return fail(MOEQ_E_INVALID, "k=%d is negative", k);
  if (k > s->n_experts) return fail(MOEQ_E_INVALID, "k=%d exceeds n_experts=%d", k, s->n_experts);
  if (k > MOEQ_MAX_TOPK) return fail(MOEQ_E_UNSUPPORTED, "k=%d exceeds %d", k, MOEQ_MAX_TOPK);
  if (T > MOEQ_MAX_DECODE_TOKENS)
    return fail(MOEQ_E_UNSUPPORTED, "T=%d exceeds the decode batch limit %d", T, MOEQ_MAX_DECODE_TOKENS);
  return MOEQ_OK;
}

int check_dtype(int d, const char* what) {
  if (d != MOEQ_BF16 && d != MOEQ_F32)
    return fail(MOEQ_E_UNSUPPORTED, "%s dtype %d: expected MOEQ_BF16 or MOEQ_F32", what, d);
  return MOEQ_OK;
}

int check_experts(const moeq_shape* s, const moeq_experts* ex, int layer) {
  if (!ex || !ex->blobs) return fail(MOEQ_E_INVALID, "experts view or its blob table is NULL");
  if (layer < 0 || layer >= ex->n_layers)
    return fail(MOEQ_E_INVALID, "layer=%d outside [0, %d)", layer, ex->n_layers);
  (void)s;
  return MOEQ_OK;
}

}  // namespace

WorkspaceLayout workspace_layout(const moeq_shape& s, int T, int k) {
  WorkspaceLayout w;
  const int64_t KS = (int64_t)k + s.n_shared;
  w.counters = 0;
  w.logits = 4096;
  w.dbuf = w.logits + align_up((int64_t)T * (s.n_experts + 1) * 8);
  w.st_bar = w.dbuf + align_up((int64_t)T * KS * s.hidden * 4);
  w.st_logits = w.st_bar + align_up((int64_t)stack_barrier_words() * 4);
  w.st_abuf = w.st_logits + align_up((int64_t)2 * s.n_experts * 16);
  w.st_h = w.st_abuf + align_up(2 * KS * s.inter * 8);
  w.st_idx = w.st_h + align_up((int64_t)2 * s.hidden * 8);
  w.st_w = w.st_idx + align_up((int64_t)T * k * 4);
  w.st_sw = w.st_w + align_up((int64_t)T * k * 4);
  w.st_gu = w.st_sw + align_up((int64_t)T * 4);
  w.total = w.st_gu + align_up((int64_t)T * KS * 2 * s.inter * 4);
  return w;
}

}  // namespace moeq

using namespace moeq;

extern "C" {

int moeq_abi_version(void) { return 2; }

const char* moeq_last_error(void) { return g_last_error.c_str(); }

int64_t moeq_expert_bytes(const moeq_shape* s) {
  if (check_shape(s) != MOEQ_OK) return -1;
  const int64_t q = (int64_t)s->hidden * s->inter * s->bits / 8;
  const int64_t sb = (int64_t)s->hidden * s->inter / s->group * 4;
  return 3 * (q + sb);
}

int moeq_workspace_bytes(const moeq_shape* s, int T, int k, int64_t* bytes) {
  if (int rc = check_shape(s)) return rc;
  if (int rc = check_tk(s, T, k)) return rc;
  if (!bytes) return fail(MOEQ_E_INVALID, "bytes is NULL");
  *bytes = workspace_layout(*s, T, k).total;
  return ok();
}

int moe_router_topk(const moeq_shape* s, const void* x, int x_dtype, uint32_t flags,
                    const uint16_t* w_router, const uint16_t* shared_gate, int T, int k,
                    int32_t* topk_idx, float* topk_w, float* shared_w, double* logits,
                    void* workspace, void* stream) {
  if (int rc = check_shape(s)) return rc;
  if (int rc = check_tk(s, T, k)) return rc;
  if (int rc = check_dtype(x_dtype, "x")) return rc;
  if (flags & ~(uint32_t)(MOEQ_F_NO_RENORM | MOEQ_F_RMSNORM))
    return fail(MOEQ_E_UNSUPPORTED, "unknown flag bits 0x%x", flags);
  if (k < 1) return fail(MOEQ_E_INVALID, "router needs k >= 1 (got %d)", k);
  if (T == 0) return ok();
  if (!x || !w_router || !topk_idx || !topk_w || !workspace)
    return fail(MOEQ_E_INVALID, "x, w_router, topk_idx, topk_w and workspace must be non-NULL");
  if (shared_gate && s->n_shared == 0)
    return fail(MOEQ_E_INVALID, "shared_gate given but n_shared == 0");
  const WorkspaceLayout L = workspace_layout(*s, T, k);
  char* ws = static_cast<char*>(workspace);
  RouterArgs a{};
  a.x = x;
  a.x_f32 = x_dtype == MOEQ_F32;
  a.rmsnorm = (flags & MOEQ_F_RMSNORM) != 0;
  a.no_renorm = (flags & MOEQ_F_NO_RENORM) != 0;
  a.w_router = w_router;
  a.shared_gate = shared_gate;
  a.H = s->hidden; a.E = s->n_experts; a.T = T; a.k = k;
  a.topk_idx = topk_idx; a.topk_w = topk_w; a.shared_w = shared_w;
  a.logits = reinterpret_cast<double*>(ws + L.logits);
  a.logits_out = logits;
  a.counter = reinterpret_cast<uint32_t*>(ws + L.counters) + kCounterRouter;
  hipError_t e = launch_router_topk(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "router kernel launch");
  return ok();
}

int moe_q4_expert_gemv(const moeq_shape* s, const moeq_experts* ex, int layer, const void* x,
                       int x_dtype, uint32_t flags, const int32_t* topk_idx, int T, int k,
                       void* workspace, float* gate_up, void* stream) {
  if (int rc = check_shape(s)) return rc;
  if (int rc = check_tk(s, T, k)) return rc;
  if (int rc = check_dtype(x_dtype, "x")) return rc;
  if (int rc = check_experts(s, ex, layer)) return rc;
  if (flags & ~(uint32_t)(MOEQ_F_NO_RENORM | MOEQ_F_RMSNORM))
    return fail(MOEQ_E_UNSUPPORTED, "unknown flag bits 0x%x", flags);
  if (T == 0 || k + s->n_shared == 0) return ok();
  if (!x || !gate_up || !workspace || (k > 0 && !topk_idx))
    return fail(MOEQ_E_INVALID, "x, topk_idx, gate_up and workspace must be non-NULL");
  const WorkspaceLayout L = workspace_layout(*s, T, k);
  char* ws = static_cast<char*>(workspace);
  GemvArgs a{};
  a.x = x;
  a.x_f32 = x_dtype == MOEQ_F32;
  a.rmsnorm = (flags & MOEQ_F_RMSNORM) != 0;
  a.blobs = ex->blobs + (int64_t)layer * (s->n_experts + s->n_shared);
  a.topk_idx = topk_idx;
  a.H = s->hidden; a.I = s->inter; a.E = s->n_experts; a.S = s->n_shared;
  a.T = T; a.k = k; a.bits = s->bits;
  a.gate_up = gate_up;
  a.status = reinterpret_cast<int32_t*>(ws + L.counters) + kCounterStatus;
  hipError_t e = launch_expert_gemv(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gate/up kernel launch");
  return ok();
}

int moe_swiglu_down_combine(const moeq_shape* s, const moeq_experts* ex, int layer,
                            const float* gate_up, const int32_t* topk_idx, const float* topk_w,
                            const float* shared_w, const void* residual, int res_dtype, int T,
                            int k, void* workspace, float* out, void* stream) {
  if (int rc = check_shape(s)) return rc;
  if (int rc = check_tk(s, T, k)) return rc;
  if (int rc = check_dtype(res_dtype, "residual")) return rc;
  if (int rc = check_experts(s, ex, layer)) return rc;
  if (T == 0) return ok();
  if (!gate_up || !residual || !out || !workspace || (k > 0 && (!topk_idx || !topk_w)))
    return fail(MOEQ_E_INVALID, "gate_up, topk_idx, topk_w, residual, out and workspace must be non-NULL");
  if (k + s->n_shared == 0) {
    return fail(MOEQ_E_UNSUPPORTED, "k == 0 without a shared expert: the layer is the identity");
  }
  const WorkspaceLayout L = workspace_layout(*s, T, k);
  char* ws = static_cast<char*>(workspace);
  DownArgs a{};
  a.gate_up = gate_up;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.shared_w = shared_w;
  a.residual = residual;
  a.res_f32 = res_dtype == MOEQ_F32;
  a.blobs = ex->blobs + (int64_t)layer * (s->n_experts + s->n_shared);
  a.H = s->hidden; a.I = s->inter; a.E = s->n_experts; a.S = s->n_shared;
  a.T = T; a.k = k; a.bits = s->bits;
  a.out = out;
  a.dbuf = reinterpret_cast<float*>(ws + L.dbuf);
  a.status = reinterpret_cast<int32_t*>(ws + L.counters) + kCounterStatus;
  hipError_t e = launch_down_combine(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "down/combine kernel launch");
  return ok();
}

int moe_expert_stack_decode(const moeq_shape* s, const moeq_experts* ex,
                            const uint16_t* const* w_router, int layer0, int L, int T, int k,
                            uint32_t flags, float* h, int32_t* topk_trace, float* h_trace,
                            void* workspace, void* stream) {
  if (int rc = check_shape(s)) return rc;
  if (int rc = check_tk(s, T, k)) return rc;
  if (flags & ~(uint32_t)(MOEQ_F_NO_RENORM | MOEQ_F_STACK_LAYERWISE | MOEQ_F_STACK_NO_NORM | MOEQ_F_STACK_JITTER))
    return fail(MOEQ_E_UNSUPPORTED, "unknown or inapplicable flag bits 0x%x", flags);
  if (!ex || !ex->blobs) return fail(MOEQ_E_INVALID, "experts view or its blob table is NULL");
  if (L < 0 || layer0 < 0 || layer0 + L > ex->n_layers)
    return fail(MOEQ_E_INVALID, "layers [%d, %d) outside [0, %d)", layer0, layer0 + L, ex->n_layers);
  if (k < 1) return fail(MOEQ_E_INVALID, "k=%d: the stack needs k >= 1", k);
  if (T == 0 || L == 0) return ok();
  if (!w_router || !h || !workspace)
    return fail(MOEQ_E_INVALID, "w_router, h and workspace must be non-NULL");
  const WorkspaceLayout W = workspace_layout(*s, T, k);
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* status = reinterpret_cast<int32_t*>(ws + W.counters) + kCounterStatus;

  if (T == 1 && !(flags & MOEQ_F_STACK_LAYERWISE)) {
    StackArgs a{};
    a.blobs = ex->blobs;
    a.routers = w_router;
    a.layer0 = layer0; a.L = L;
    a.H = s->hidden; a.I = s->inter; a.E = s->n_experts; a.S = s->n_shared; a.K = k;
    a.bits = s->bits;
    a.no_renorm = (flags & MOEQ_F_NO_RENORM) != 0;
    a.no_norm = (flags & MOEQ_F_STACK_NO_NORM) != 0;
    a.jitter = (flags & MOEQ_F_STACK_JITTER) != 0;
    a.h = h;
    a.topk_trace = topk_trace;
    a.h_trace = h_trace;
    a.lwords = reinterpret_cast<uint64_t*>(ws + W.st_logits);
    a.awords = reinterpret_cast<uint64_t*>(ws + W.st_abuf);
    a.hwords = reinterpret_cast<uint64_t*>(ws + W.st_h);
    a.bar = reinterpret_cast<uint32_t*>(ws + W.st_bar);
    a.status = status;
    a.clocks = g_stack_clocks;
    a.bclocks = g_stack_bclocks;
    g_stack_clocks = nullptr;
    g_stack_bclocks = nullptr;
    hipError_t e = launch_stack_decode(a, st);
    if (e == hipSuccess) {
      g_last_stack_path = 1;
      return ok();
    }
    // no persistent instantiation for this shape, or the device cannot hold
    // the whole grid at once: run the layers one launch sequence at a time
    if (e != hipErrorNotSupported && e != hipErrorCooperativeLaunchTooLarge)
      return hip_fail(e, "persistent stack kernel launch");
    (void)hipGetLastError();
    if (flags & MOEQ_F_STACK_JITTER)
      return fail(MOEQ_E_UNSUPPORTED, "delay injection has no persistent instantiation for this shape");
  }
  if (flags & MOEQ_F_STACK_JITTER)
    return fail(MOEQ_E_UNSUPPORTED, "delay injection applies to the persistent one-token launch only");

  // per-layer path: router -> gate/up -> down/combine per layer, in place on h
  const int KS = k + s->n_shared;
  int32_t* idx = reinterpret_cast<int32_t*>(ws + W.st_idx);
  float* w = reinterpret_cast<float*>(ws + W.st_w);
  float* sw = reinterpret_cast<float*>(ws + W.st_sw);
  float* gu = reinterpret_cast<float*>(ws + W.st_gu);
  const uint32_t norm = (flags & MOEQ_F_STACK_NO_NORM) ? 0u : (uint32_t)MOEQ_F_RMSNORM;
  const uint32_t lf = norm | (flags & MOEQ_F_NO_RENORM);
  for (int l = 0; l < L; ++l) {
    const int layer = layer0 + l;
    if (h_trace) {
      hipError_t e = hipMemcpyAsync(h_trace + (int64_t)l * T * s->hidden, h,
                                    sizeof(float) * (size_t)T * s->hidden, hipMemcpyDeviceToDevice, st);
      if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync h_trace");
    }
    int32_t* idx_l = topk_trace ? topk_trace + (int64_t)l * T * k : idx;
    {
      // the router kernel reads this layer's matrix pointer from the device table
      RouterArgs a{};
      a.x = h;
      a.x_f32 = 1;
      a.rmsnorm = norm != 0;
      a.no_renorm = (lf & MOEQ_F_NO_RENORM) != 0;
      a.w_table = w_router;
      a.w_layer = layer;
      a.H = s->hidden; a.E = s->n_experts; a.T = T; a.k = k;
      a.topk_idx = idx_l; a.topk_w = w; a.shared_w = s->n_shared ? sw : nullptr;
      a.logits = reinterpret_cast<double*>(ws + W.logits);
      a.counter = reinterpret_cast<uint32_t*>(ws + W.counters) + kCounterRouter;
      hipError_t e = launch_router_topk(a, st);
      if (e != hipSuccess) return hip_fail(e, "router kernel launch");
    }
    int rc = moe_q4_expert_gemv(s, ex, layer, h, MOEQ_F32, norm, idx_l, T, k, workspace, gu, stream);
    if (rc) return rc;
    rc = moe_swiglu_down_combine(s, ex, layer, gu, idx_l, w, s->n_shared ? sw : nullptr, h, MOEQ_F32, T,
                                 k, workspace, h, stream);
    if (rc) return rc;
  }
  (void)KS;
  g_last_stack_path = 2;
  return ok();
}

int moe_expert_stack_decode_mixed(const moeq_shape* s, const int32_t* layer_bits, const moeq_experts* ex,
                                  const uint16_t* const* w_router, int layer0, int L, int T, int k, uint32_t flags,
                                  float* h, int32_t* topk_trace, float* h_trace, void* workspace, void* stream) {
  if (int rc = check_shape(s)) return rc;
  if (L < 0) return fail(MOEQ_E_INVALID, "L=%d is negative", L);
  if (L > 0 && !layer_bits) return fail(MOEQ_E_INVALID, "layer_bits is NULL");
  for (int l = 0; l < L; ++l) {
    moeq_shape sl = *s;
    sl.bits = layer_bits[l];
    if (int rc = check_shape(&sl)) return rc;
  }
  // maximal runs of layers of equal width, each one stack call
  int paths = 0;
  for (int l = 0; l < L;) {
    int e = l + 1;
    while (e < L && layer_bits[e] == layer_bits[l]) ++e;
    moeq_shape sl = *s;
    sl.bits = layer_bits[l];
    int rc = moe_expert_stack_decode(&sl, ex, w_router, layer0 + l, e - l, T, k, flags, h,
                                     topk_trace ? topk_trace + (int64_t)l * T * k : nullptr,
                                     h_trace ? h_trace + (int64_t)l * T * s->hidden : nullptr, workspace, stream);
    if (rc != MOEQ_OK) return rc;
    paths |= 1 << g_last_stack_path;
    l = e;
  }
  g_last_stack_path = paths == (1 << 1) ? 1 : (paths == (1 << 2) ? 2 : (paths ? 3 : 0));
  return ok();
}

int moeq_last_stack_path(void) { return g_last_stack_path; }

int moeq_stack_clock_trace(int64_t* clocks) {
  g_stack_clocks = clocks;
  return kStackClockEvents;
}

int moeq_stack_block_clock_trace(int64_t* clocks) {
  g_stack_bclocks = clocks;
  return kBlockClockEvents;
}

int moe_read_device_status(void* workspace, void* stream, int32_t* status) {
  if (!workspace || !status) return fail(MOEQ_E_INVALID, "workspace and status must be non-NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* word = reinterpret_cast<int32_t*>(workspace) + kCounterStatus;
  hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  e = hipMemcpy(status, word, sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy status");
  const int32_t zero = 0;
  e = hipMemcpy(word, &zero, sizeof(int32_t), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy clear status");
  return ok();
}

int64_t moeq_probe_scratch_bytes(int words_per_block, int stride) {
  const int nb = device_cus();
  if (nb < 1 || words_per_block < 1 || stride < words_per_block) return -1;
  return probe_scratch_bytes(nb, words_per_block, stride);
}

int moeq_probe_handoff(int mode, int words_per_block, int stride, int rounds, int sleep, int peer,
                       void* scratch, int64_t scratch_bytes, int64_t* ticks, int64_t* mismatches,
                       int32_t* xcc_ids, void* stream) {
  const int nb = device_cus();
  if (nb < 1) return fail(MOEQ_E_HIP, "no device");
  if (nb > 1024) return fail(MOEQ_E_UNSUPPORTED, "the probe handles at most 1024 CUs");
  if (mode < 0 || mode > 7) return fail(MOEQ_E_INVALID, "mode=%d outside [0, 7]", mode);
  if (mode == 7 && (stride < 2 * words_per_block || nb > 511))
    return fail(MOEQ_E_UNSUPPORTED, "the reduction needs stride >= 2 * words_per_block (three buffers) and < 512 CUs");
  if (mode == 6 && words_per_block * nb > 4 * 512)
    return fail(MOEQ_E_UNSUPPORTED, "pipelined polls handle at most 2048 words");
  if (words_per_block < 1 || (int64_t)words_per_block * nb > probe_max_words())
    return fail(MOEQ_E_UNSUPPORTED, "words_per_block=%d: the probe polls at most %d words", words_per_block,
                probe_max_words());
  if (stride < words_per_block) return fail(MOEQ_E_INVALID, "stride=%d < words_per_block", stride);
  if (rounds < 1 || rounds > (1 << 24)) return fail(MOEQ_E_INVALID, "rounds=%d outside [1, 2^24]", rounds);
  if (mode == 2 && (peer < 1 || peer >= nb)) return fail(MOEQ_E_INVALID, "peer=%d outside [1, %d)", peer, nb);
  if ((mode == 4 || mode == 5) && (peer < 1 || peer > 64))
    return fail(MOEQ_E_INVALID, "copies=%d outside [1, 64]", peer);
  const int64_t need = probe_scratch_bytes(nb, words_per_block, stride);
  if (!scratch || !ticks || scratch_bytes < need)
    return fail(MOEQ_E_INVALID, "scratch (>= moeq_probe_scratch_bytes) and ticks must be given");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemsetAsync(scratch, 0, (size_t)need, st);
  if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync probe scratch");
  e = launch_probe(mode, words_per_block, stride, rounds, sleep, peer, scratch, nb, st);
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "probe synchronise");
  uint32_t ctl[4];
  int32_t status = 0;
  const char* s = static_cast<const char*>(scratch);
  if ((e = hipMemcpy(ctl, s, sizeof ctl, hipMemcpyDeviceToHost)) != hipSuccess ||
      (e = hipMemcpy(&status, s + 64, sizeof status, hipMemcpyDeviceToHost)) != hipSuccess ||
      (e = hipMemcpy(ticks, s + 128, sizeof(int64_t), hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "probe read-back");
  if (xcc_ids && (e = hipMemcpy(xcc_ids, s + 4096, sizeof(int32_t) * nb, hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "probe read-back");
  if (xcc_ids)
    for (int i = 0; i < nb; ++i) xcc_ids[i] -= 1;
  if (mismatches) *mismatches = ctl[3];
  if (status != 0) return fail(MOEQ_E_DEVICE, "probe wait timed out (status %d)", status);
  return ok();
}

}  // extern "C"
