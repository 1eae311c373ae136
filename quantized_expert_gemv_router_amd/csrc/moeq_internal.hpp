// Host-side internals shared by the moeq translation units: workspace
// layout, kernel argument blocks and launcher prototypes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moeq.h"

namespace moeq {

// Error reporting shared by the entry points: fail() records the message
// returned by moeq_last_error() and returns `code`; ok() clears it.
int fail(int code, const char* fmt, ...);
int ok();
int hip_fail(hipError_t e, const char* what);
int check_shape(const moeq_shape* s);

constexpr int64_t kAlign = 256;
inline int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Workspace layout (offsets in bytes from the workspace base):
//   [0, 4096)        u32 words: [0] router arrival counter, [1] status word
//   logits           f64 [T][E + 1]   (last column: shared-gate logit)
//   dbuf             f32 [T][k + S][H] per-slot down outputs (multi-token)
//   stack area       barrier words, tagged words double-buffered by layer
//                    parity (fp64 logit halves [2][E][2], activations
//                    [2][k + S][I], hidden state [2][H]), and the
//                    per-layer path's routing
//                    (idx [T][k], w [T][k], shared w [T]) and gate_up
//                    [T][k + S][2][I]
struct WorkspaceLayout {
  int64_t counters = 0;
  int64_t logits = 0;
  int64_t dbuf = 0;
  int64_t st_bar = 0;
  int64_t st_logits = 0;
  int64_t st_abuf = 0;
  int64_t st_h = 0;
  int64_t st_idx = 0;
  int64_t st_w = 0;
  int64_t st_sw = 0;
  int64_t st_gu = 0;
  int64_t total = 0;
};

constexpr int kCounterRouter = 0;
constexpr int kCounterStatus = 1;
constexpr int32_t kStatusTimeout = 2;   // a grid barrier or handoff wait gave up

WorkspaceLayout workspace_layout(const moeq_shape& s, int T, int k);

// ----------------------------------------------------------------- router
struct RouterArgs {
  const void* x;
  int x_f32;
  int rmsnorm;
  int no_renorm;
  const uint16_t* w_router;
  const uint16_t* const* w_table;  // if set, the router matrix is w_table[w_layer] (device)
  int w_layer;
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
  float* dbuf;         // [T][k + S][H] per-slot rows (batches)
  int32_t* status;
};
hipError_t launch_down_combine(const DownArgs& a, hipStream_t stream);

// ------------------------------------------------------------- prefill
// Prefill workspace (offsets in bytes): status word, 1/rms [T] f64, x fp16
// [T][H] (permuted), logits [T][E] f64, idx [T][k] i32, w [T][k] f32,
// per-expert counts / list offsets / tile offsets, the row-tile table,
// pair lists [T*(k+S)],
// activations fp16 [T*(k+S)][I], per-pair down rows f32 [T*(k+S)][H].
struct PrefillLayout {
  int64_t status = 0, inv = 0, xh = 0, logits = 0, idx = 0, w = 0, counts = 0, offs = 0, mtoff = 0,
          tiles = 0, lists = 0, abuf = 0, dbuf = 0, total = 0;
};
PrefillLayout prefill_layout(const moeq_shape& s, int T, int k);

// ----------------------------------------------- persistent stack decode
struct StackArgs {
  const void* const* blobs;        // pointer table base, [n_layers][E + S]
  const uint16_t* const* routers;  // device array [n_layers] of [E][H] bf16
  int layer0, L;
  int H, I, E, S, K, bits;
  int no_renorm;
  int no_norm;                     // layer input taken as is (no RMS norm)
  int jitter;                      // diagnostic delay injection before every hand-off publish
  int router_rows;                 // set by the launcher
  float* h;                        // [H] in/out
  int32_t* topk_trace;             // [L][K] or null
  float* h_trace;                  // [L][H] or null
  uint64_t* lwords;                // [2][E][2] tagged halves of the fp64 logits (by layer parity)
  uint64_t* awords;                // [2][K + S][I] words: tagged activation pairs in the first (K + S) I / 2
  uint64_t* hwords;                // [2][H] tagged hidden state between layers
  uint32_t* bar;                   // barrier counters (stack_barrier_words())
  int32_t* status;
  int64_t* clocks;                 // diagnostic: [L][kStackClockEvents] wall-clock stamps of block 0, or null
  int64_t* bclocks;                // diagnostic: [blocks][L][kBlockClockEvents] stamps of every block, or null
};
constexpr int kStackClockEvents = 24;
constexpr int kBlockClockEvents = 16;
int stack_barrier_words();
// hipErrorNotSupported: no persistent instantiation for this shape.
hipError_t launch_stack_decode(StackArgs& a, hipStream_t stream);

// ------------------------------------------------ hand-off probe (diagnostic)
int64_t probe_scratch_bytes(int nb, int W, int stride);
int probe_max_words();
hipError_t launch_probe(int mode, int W, int stride, int rounds, int sleep, int peer, void* scratch, int nb,
                        hipStream_t stream);
int device_cus();

}  // namespace moeq
