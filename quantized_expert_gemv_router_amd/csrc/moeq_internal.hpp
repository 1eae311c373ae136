// Host-side internals shared by the moeq translation units: workspace
// layout, kernel argument blocks and launcher prototypes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moeq.h"

namespace moeq {

constexpr int64_t kAlign = 256;
inline int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Workspace layout (offsets in bytes from the workspace base):
//   [0, 4096)        u32 words: [0] router arrival counter, [1] status word,
//                    [64 .. 64 + n_rowblocks) down-combine row-block counters
//   logits           f64 [T][E + 1]   (last column: shared-gate logit)
//   dbuf             f32 [T][k + S][H] per-slot down outputs (multi-token)
struct WorkspaceLayout {
  int64_t counters = 0;
  int64_t logits = 0;
  int64_t dbuf = 0;
  int64_t total = 0;
};

constexpr int kCounterRouter = 0;
constexpr int kCounterStatus = 1;
constexpr int kCounterRowBlocks = 64;
constexpr int kMaxRowBlockCounters = 1024 - kCounterRowBlocks;

WorkspaceLayout workspace_layout(const moeq_shape& s, int T, int k);

// ----------------------------------------------------------------- router
struct RouterArgs {
  const void* x;
  int x_f32;
  int rmsnorm;
  int no_renorm;
  const uint16_t* w_router;
  const uint16_t* shared_gate;
  int H, E, T, k;
  int32_t* topk_idx;
  float* topk_w;
  float* shared_w;
  double* logits;      // [T][E + 1] scratch (workspace)
  double* logits_out;  // [T][E] or null
  uint32_t* counter;
};
hipError_t launch_router_topk(const RouterArgs& a, hipStream_t stream);

// ------------------------------------------------------------ gate / up
struct GemvArgs {
  const void* x;
  int x_f32;
  int rmsnorm;
  const void* const* blobs;   // this layer's row of the pointer table
  const int32_t* topk_idx;
  int H, I, E, S, T, k, bits;
  float* gate_up;
  int32_t* status;
};
hipError_t launch_expert_gemv(const GemvArgs& a, hipStream_t stream);

// ------------------------------------------------------ down + combine
struct DownArgs {
  const float* gate_up;
  const int32_t* topk_idx;
  const float* topk_w;
  const float* shared_w;
  const void* residual;
  int res_f32;
  const void* const* blobs;
  int H, I, E, S, T, k, bits;
  float* out;
  float* dbuf;
  uint32_t* rb_counters;
  int32_t* status;
};
hipError_t launch_down_combine(const DownArgs& a, hipStream_t stream);

}  // namespace moeq
