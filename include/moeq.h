/*
 * moeq: the quantized Mixture-of-Experts expert forward at decode, for
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The path (per layer, per token):
 *   router logits over E experts -> top-K -> softmax of the K selected
 *   -> for each selected expert and the shared expert: group-wise affine
 *      4-bit or 2-bit dequantised mat-vec for gate and up -> SwiGLU ->
 *      dequantised down mat-vec -> weighted combine with the shared expert
 *      and the residual.
 * Sources: Flash-MoE (fr.news.hada.io), sections "Architecture du modèle"
 * (512 experts, K=4 active including one shared, hidden 4096, 60 layers),
 * "Noyau de déquantification optimisé FMA" (weight = value*scale + bias),
 * "Shaders de calcul Metal" (4-bit/2-bit dequant mat-vec, SwiGLU, MoE
 * combine + residual + gate), "Deferred GPU Expert Compute" (combine, norm
 * and residual stay on the GPU and feed the next layer); openclawradar.com/fr
 * (top-10 routing over 512 experts; experts kept in a bounded set of
 * resident slots and loaded on router demand).
 *
 * Conventions (all entry points):
 *   - Every call returns MOEQ_OK (0) or a negative MOEQ_E_* code and then
 *     sets a thread-local message readable with moeq_last_error().
 *     Unsupported inputs are refused with MOEQ_E_UNSUPPORTED, never
 *     silently ignored.
 *   - Pointers marked "device" are HIP device pointers owned by the caller
 *     and must stay valid until the work queued on `stream` completes.
 *     `stream` is a hipStream_t passed as void* (NULL = null stream).
 *   - Calls validate their arguments on the host, enqueue kernels on
 *     `stream` and return without synchronising; no entry point allocates
 *     device memory except moe_pool_create (host metadata + events).
 *   - `workspace` is caller-owned device memory of moeq_workspace_bytes()
 *     bytes, zero-filled once after allocation; the kernels leave it ready
 *     for the next call.  Calls sharing one workspace must not overlap.
 *   - Results are bit-reproducible run to run: no floating-point atomics.
 *
 * Expert blob layout (one contiguous blob per expert, 256-byte aligned):
 *   [gate.q | up.q | down.q | gate.sb | up.sb | down.sb]
 *   gate.q, up.q: inter rows x hidden values; down.q: hidden rows x inter
 *   values; each row packs 32/bits unsigned values per little-endian u32,
 *   value j at bit bits*(j mod (32/bits)) of word j/(32/bits).
 *   *.sb: one u32 per (row, group of 64 consecutive inputs): bf16 scale in
 *   the low 16 bits, bf16 bias in the high 16 bits.  w = value*scale + bias.
 */
#ifndef MOEQ_H
#define MOEQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOEQ_OK = 0,
  MOEQ_E_INVALID = -1,        /* bad argument (null pointer, negative size, ...) */
  MOEQ_E_UNSUPPORTED = -2,    /* valid but outside what the kernels implement */
  MOEQ_E_HIP = -3,            /* a HIP runtime call failed */
  MOEQ_E_POOL_EXHAUSTED = -4, /* every pool slot is pinned by the current layer */
  MOEQ_E_DEVICE = -5          /* a kernel flagged bad data (see moe_read_device_status) */
};

enum { MOEQ_BF16 = 0, MOEQ_F32 = 1 };   /* activation dtypes */

enum {
  /* Weights = full softmax over all E logits read at the selected experts
   * (default: softmax over the K selected logits). */
  MOEQ_F_NO_RENORM = 1u,
  /* The layer input is normalised as x / sqrt(mean(x^2) + 1e-6) (unit-weight
   * RMS norm) before the router and the experts; the residual stays x. */
  MOEQ_F_RMSNORM = 2u,
  /* moe_expert_stack_decode only: run the layers one launch sequence at a
   * time (router, gate/up, down per layer) instead of the persistent kernel. */
  MOEQ_F_STACK_LAYERWISE = 4u,
  /* moe_expert_stack_decode only: each layer takes its input h as is (no
   * RMS norm): one layer of this call computes what moe_router_topk,
   * moe_q4_expert_gemv and moe_swiglu_down_combine compute without
   * MOEQ_F_RMSNORM (for a single decode layer in one launch). */
  MOEQ_F_STACK_NO_NORM = 8u,
  /* moe_expert_stack_decode only, diagnostic: the persistent launch runs a
   * delay-injection build of its kernel, in which every wave sleeps a
   * pseudo-random 0..~13 us before each hand-off publish.  The results must
   * be bit-identical to the plain launch.  MOEQ_E_UNSUPPORTED where the
   * shape has no such build (hidden 4096 / 512 experts / top-3 + 1 at
   * 4 bits, and the small test shape), for T > 1 and with
   * MOEQ_F_STACK_LAYERWISE. */
  MOEQ_F_STACK_JITTER = 16u
};

/* Limits of the current kernels (larger values return MOEQ_E_UNSUPPORTED). */
#define MOEQ_MAX_HIDDEN 8192
#define MOEQ_MAX_INTER 8192
#define MOEQ_MAX_EXPERTS 4096
#define MOEQ_MAX_TOPK 16
#define MOEQ_MAX_DECODE_TOKENS 64

typedef struct moeq_shape {
  int32_t hidden;     /* H, multiple of 64 */
  int32_t inter;      /* I, multiple of 64 */
  int32_t n_experts;  /* E routed experts per layer */
  int32_t n_shared;   /* S always-active experts per layer, 0 or 1 */
  int32_t bits;       /* 4, 3 or 2 (3: hidden and inter multiples of 128) */
  int32_t group;      /* 64 */
} moeq_shape;

/* Where the expert blobs of each layer live.  `blobs` is a device array of
 * n_layers * (n_experts + n_shared) device pointers, row-major by layer;
 * shared experts follow the routed ones.  Only the entries of experts that
 * a call actually reads need to be valid. */
typedef struct moeq_experts {
  const void* const* blobs;
  int32_t n_layers;
} moeq_experts;

/* Bytes of one expert blob: 3 * (H*I*bits/8 + H*I/64*4).  7,077,888 for
 * H=4096, I=1024, 4-bit (6.75 MiB, the per-expert size given in Flash-MoE,
 * "SSD Expert Streaming"); 3,932,160 at 2-bit.  Returns -1 for a bad shape. */
int64_t moeq_expert_bytes(const moeq_shape* shape);

/* Workspace bytes needed by the calls below for T tokens and top-k. */
int moeq_workspace_bytes(const moeq_shape* shape, int T, int k, int64_t* bytes);

/* Message of the last failed call on this thread ("" if none). */
const char* moeq_last_error(void);

/* ABI version of this header (bumped on incompatible change). */
int moeq_abi_version(void);

/* Router and top-K (Flash-MoE, "Architecture du modèle": K of 512 experts
 * active per token; openclawradar.com/fr: top-10 routing).
 *   x             device [T][H] in x_dtype (MOEQ_BF16 or MOEQ_F32)
 *   w_router      device [E][H] bf16 router matrix, row-major
 *   shared_gate   device [H] bf16 or NULL: if given, the shared expert's
 *                 weight is sigmoid(shared_gate . xhat), else 1
 *   flags         MOEQ_F_RMSNORM, MOEQ_F_NO_RENORM
 *   topk_idx      device [T][k] int32 out: experts by logit descending,
 *                 ties to the lower index
 *   topk_w        device [T][k] f32 out: softmax weights of the selection
 *   shared_w      device [T] f32 out (may be NULL when n_shared == 0)
 *   logits        device [T][E] f64 out, or NULL
 * Logits accumulate in fp64 (bf16 x bf16/fp32 products are exact there),
 * so the selection equals an fp64 evaluation except at gaps near 1e-15.
 * T == 0 is a no-op.  1 <= k <= min(E, 16); T <= 64. */
int moe_router_topk(const moeq_shape* shape, const void* x, int x_dtype, uint32_t flags,
                    const uint16_t* w_router, const uint16_t* shared_gate, int T, int k,
                    int32_t* topk_idx, float* topk_w, float* shared_w, double* logits,
                    void* workspace, void* stream);

/* Gate and up projections of every selected expert and the shared expert
 * (Flash-MoE, "Noyau de déquantification optimisé FMA" and "Shaders de
 * calcul Metal": dequantised 4-bit / 2-bit mat-vec).  Each expert's rows
 * are streamed once per call for every 4 of the (token, slot) pairs routed
 * to it (once, for most experts of a decode batch) and applied to those
 * tokens.
 *   x         device [T][H] in x_dtype; with MOEQ_F_RMSNORM normalised first
 *   topk_idx  device [T][k] int32 (ids outside [0, E) are skipped, their
 *             outputs left unwritten, and the workspace status word is set)
 *   gate_up   device [T][k + S][2][I] f32 out: slot s < k is the s-th
 *             selected expert, slot k the shared expert; [.][0] = gate,
 *             [.][1] = up
 * Bits 2 and 4 are both handled (the name keeps the 4-bit case). */
int moe_q4_expert_gemv(const moeq_shape* shape, const moeq_experts* experts, int layer,
                       const void* x, int x_dtype, uint32_t flags, const int32_t* topk_idx,
                       int T, int k, void* workspace, float* gate_up, void* stream);

/* SwiGLU, down projection and combine (Flash-MoE, "Shaders de calcul
 * Metal": SwiGLU and MoE combine + residual + gate; "Deferred GPU Expert
 * Compute"):
 *   out[t] = residual[t] + sum_s topk_w[t][s] * d_s + shared_w[t] * d_shared
 *   d_s = Wd_s (silu(g_s) * u_s), summed in slot order.
 *   gate_up   device [T][k + S][2][I] f32 (from moe_q4_expert_gemv)
 *   shared_w  device [T] f32 or NULL (= 1)
 *   residual  device [T][H] in res_dtype
 *   out       device [T][H] f32 (may alias residual when res_dtype is f32) */
int moe_swiglu_down_combine(const moeq_shape* shape, const moeq_experts* experts, int layer,
                            const float* gate_up, const int32_t* topk_idx, const float* topk_w,
                            const float* shared_w, const void* residual, int res_dtype,
                            int T, int k, void* workspace, float* out, void* stream);

/* L stacked decode layers [layer0, layer0 + L) on a resident fp32 residual
 * stream h, in place (Flash-MoE, fr.news.hada.io, "Architecture du
 * modèle": 60 layers, each with 512 experts, K active including one shared;
 * "Deferred GPU Expert Compute": combine + norm + residual stay on the GPU
 * and feed the next layer).  Per layer: xhat = h / sqrt(mean(h^2) + 1e-6)
 * (unit-weight RMS norm), router + top-k + softmax on xhat, experts on xhat,
 * h <- h + sum_s w_s d_s + d_shared.
 *   w_router    device array [n_layers] of device pointers to [E][H] bf16
 *   h           device [T][H] f32, in/out
 *   topk_trace  device [L][T][k] int32 out, or NULL
 *   h_trace     device [L][T][H] f32 out (the input of each layer), or NULL
 *   flags       MOEQ_F_NO_RENORM, MOEQ_F_STACK_LAYERWISE, MOEQ_F_STACK_NO_NORM,
 *               MOEQ_F_STACK_JITTER
 * T == 1 runs one persistent launch for all L layers (no host
 * involvement: the workgroups hand the logits, the activations and the
 * hidden state to each other through tagged words in the workspace) when
 * the shape has a persistent instantiation; the launch is an ordinary one
 * (it can be captured in a HIP graph and replayed) whose workgroups, one
 * per compute unit, must all be resident at once, so persistent launches
 * on one GPU must not overlap in time (a launch that cannot fill the GPU
 * ends with status bit 2 instead of hanging).  On that path each fp64
 * logit is handed to the other workgroups rounded to a 36-bit significand
 * (2^-37 relative) and the activations as fp16 under a shared power of two
 * (the precision they are staged in anyway).  Otherwise, or with
 * MOEQ_F_STACK_LAYERWISE or T > 1, it enqueues the three per-layer calls
 * for each layer.  A wait between workgroups that lasts too long sets
 * status bit 2 (see moe_read_device_status) and the launch ends early. */
int moe_expert_stack_decode(const moeq_shape* shape, const moeq_experts* experts,
                            const uint16_t* const* w_router, int layer0, int L, int T, int k,
                            uint32_t flags, float* h, int32_t* topk_trace, float* h_trace,
                            void* workspace, void* stream);

/* moe_expert_stack_decode with no workspace argument and no allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The workspace is a
 * static device array of MOEQ_NOALLOC_SCRATCH_BYTES per GPU, held by the
 * library until the process ends; its address is taken once per device (the
 * first call on a device, with that device current, also clears it on
 * `stream`).  Arguments as moe_expert_stack_decode, plus
 *   status_out  device int32 or NULL: receives the call's status word
 *               (0 = clean, bits as in moe_read_device_status), which is
 *               then cleared for the next call.
 * MOEQ_E_UNSUPPORTED when the shape's workspace (moeq_workspace_bytes for T
 * and k) exceeds MOEQ_NOALLOC_SCRATCH_BYTES (8 MiB: T = 1 fits every shape
 * within the other limits, and so does a 16-token batch at hidden 4096,
 * intermediate 1024, 512 experts, top-10).  All calls on one GPU share the array: calls that
 * overlap in time on one GPU (several streams or host threads) race and
 * must be serialised by the caller. */
#define MOEQ_NOALLOC_SCRATCH_BYTES (8 << 20)
int moe_expert_stack_decode_noalloc(const moeq_shape* shape, const moeq_experts* experts,
                                    const uint16_t* const* w_router, int layer0, int L, int T, int k,
                                    uint32_t flags, float* h, int32_t* topk_trace, float* h_trace,
                                    int32_t* status_out, void* stream);

/* moe_expert_stack_decode over layers of different widths (per-layer mixes
 * of 4-, 3- and 2-bit experts; Flash-MoE, fr.news.hada.io, "Résultats de
 * performance": 4-bit and 2-bit expert sets; openclawradar.com/ru,
 * "Эффективные оптимизации": lower-bit experts).  layer_bits: host [L],
 * layer layer0 + l holds blobs of layer_bits[l] bits; every other argument
 * as moe_expert_stack_decode with shape.bits ignored.  Each maximal run of
 * layers of one width is one moe_expert_stack_decode call (persistent
 * where the width has a persistent instantiation, else per-layer
 * launches); moeq_last_stack_path then reports 1 or 2 if every run took
 * that path, 3 if they differed. */
int moe_expert_stack_decode_mixed(const moeq_shape* shape, const int32_t* layer_bits, const moeq_experts* experts,
                                  const uint16_t* const* w_router, int layer0, int L, int T, int k,
                                  uint32_t flags, float* h, int32_t* topk_trace, float* h_trace,
                                  void* workspace, void* stream);

/* Prefill: T tokens (any T >= 1; the configured workload is 2048) through
 * the stacked layers [layer0, layer0 + L) on the fp32 residual stream h
 * [T][H], in place; per layer and token the same computation as
 * moe_expert_stack_decode (unit-weight RMS norm, router, top-k + softmax,
 * experts, combine).  Flash-MoE (fr.news.hada.io), "Architecture du
 * modèle"; openclawradar.com/fr (top-10 over 512 experts).  Tokens are
 * grouped by expert so each expert's weights are streamed once per layer
 * (per 64 tokens routed to it) into dequantise-on-load MFMA GEMMs with fp16
 * operands and fp32 accumulation; the router stays fp64.
 *   topk_trace  device [L][T][k] int32 out, or NULL
 *   flags       MOEQ_F_NO_RENORM
 *   workspace   moeq_prefill_workspace_bytes(shape, T, k) bytes
 * 4-bit experts only; hidden and inter multiples of 128; scales and biases
 * must be representable in fp16 (they are converted from bf16 for the
 * MFMA operands). */
int moe_expert_stack_prefill(const moeq_shape* shape, const moeq_experts* experts,
                             const uint16_t* const* w_router, int layer0, int L, int T, int k,
                             uint32_t flags, float* h, int32_t* topk_trace, void* workspace, void* stream);

/* Workspace bytes of moe_expert_stack_prefill for T tokens and top-k
 * (about 440 MB at T=2048, k=10, hidden 4096, inter 1024, 512+1 experts). */
int moeq_prefill_workspace_bytes(const moeq_shape* shape, int T, int k, int64_t* bytes);

/* Diagnostic timing of the prefill kernels: with enable != 0, every later
 * moe_expert_stack_prefill layer records HIP events on its stream around
 * each kernel class (0 norm, 1 router, 2 top-K, 3 grouping, 4 gate/up GEMM,
 * 5 down GEMM, 6 combine).  moeq_prefill_timing_read waits for them and
 * returns, per class, the summed milliseconds ms[7] and the number of
 * timed launches launches[7], then discards the events; timing stays on
 * until moeq_prefill_timing(0). */
int moeq_prefill_timing(int enable);
int moeq_prefill_timing_read(double* ms, int32_t* launches);

/* Which path the last successful moe_expert_stack_decode on this thread
 * took: 1 = persistent launch, 2 = per-layer launches, 0 = none yet. */
int moeq_last_stack_path(void);

/* Diagnostic: the calling thread's next persistent moe_expert_stack_decode
 * launch writes
 * wall-clock stamps (100 MHz device counter) of its phase boundaries, as
 * seen by workgroup 0, to the device array `clocks` [L][n] where n is the
 * return value (24).  The pointer is consumed by that launch. */
int moeq_stack_clock_trace(int64_t* clocks);

/* Diagnostic: the calling thread's next persistent moe_expert_stack_decode
 * launch writes, for every workgroup, n = 16 (the return value) entries per
 * layer to the device array `clocks` [blocks][L][n], blocks = the device's
 * compute units: stamps of the same clock at 0 layer start, 1 h polled,
 * 2 own logits published, 3 logits polled, 4 top-K, 5 routed gate/up dot
 * products, 6 routed activations published, 7 shared activations polled and
 * applied, 8 routed activations polled (thread 0's view, no extra
 * barriers), 9 h published (the workgroup's last wave); then thread 0's
 * poll rounds for 10 h, 11 logits, 12 shared and 13 routed activations.
 * The pointer is consumed by that launch. */
int moeq_stack_block_clock_trace(int64_t* clocks);

/* Synchronise `stream` and read the workspace status word: 0 = clean,
 * else a bitmask (1 = an expert id outside [0, E) or a NULL blob pointer
 * was seen, 2 = a wait between workgroups of the persistent stack kernel
 * timed out).  Clears it. */
int moe_read_device_status(void* workspace, void* stream, int32_t* status);

/* Diagnostic: latency of cross-workgroup hand-offs on this device.  One
 * workgroup of 512 threads per CU (cooperative launch) runs `rounds` rounds
 * of one pattern after a start barrier:
 *   mode 0  tagged all-gather: every workgroup publishes words_per_block
 *           64-bit words carrying the round's tag (writer j's words from
 *           word j * stride); every workgroup polls all of them (the words
 *           are their own flags);
 *   mode 1  flag + payload: payload words, then one tagged flag word per
 *           workgroup; readers poll the flags, then read the payload once;
 *   mode 2  ping-pong: workgroups 0 and `peer` bounce one tagged word (two
 *           one-way hand-offs per round);
 *   mode 3  counter barrier: one atomic counter, polled until every
 *           workgroup has added its round;
 *   mode 4  gather + broadcast: only workgroup 0 polls the published words,
 *           then writes the round's tag to `peer` go words (4 KiB apart)
 *           that the other workgroups poll (workgroup id mod peer);
 *   mode 5  mode 4, then every workgroup reads all the words once;
 *   mode 6  mode 0 with `peer` (2 or 4) staggered loads of every polled
 *           word in flight (at most 2048 words);
 *   mode 7  fixed-point reduction: every workgroup adds to each of the
 *           CUs * words_per_block 64-bit accumulators with agent-scope
 *           atomics (a count in bits 55-63, its id mod 256 below) and polls
 *           them until every count reads CUs; sums are checked (a wrong
 *           sum counts in *mismatches); accumulators triple-buffered by
 *           round, so stride >= 2 * words_per_block; fewer than 512 CUs.
 * `sleep` (0..3) is the back-off between polls (s_sleep 0, 1, 2, 4).
 * scratch: device, moeq_probe_scratch_bytes(words_per_block, stride) bytes,
 * cleared by the call.  Synchronises `stream`; *ticks = 100 MHz wall-clock
 * ticks of all rounds as seen by workgroup 0; *mismatches (may be NULL) =
 * payload words read with a stale tag in mode 1; xcc_ids (host [CUs], may
 * be NULL) receives the XCD id each workgroup ran on.  MOEQ_E_DEVICE if a
 * wait gave up.  words_per_block * (CUs) <= 8192, stride >= words_per_block. */
int64_t moeq_probe_scratch_bytes(int words_per_block, int stride);
int moeq_probe_handoff(int mode, int words_per_block, int stride, int rounds, int sleep, int peer,
                       void* scratch, int64_t scratch_bytes, int64_t* ticks, int64_t* mismatches,
                       int32_t* xcc_ids, void* stream);

/* ------------------------------------------------------------------ pool
 * Expert slot pool (openclawradar.com/fr, Flash-MoE write-up: experts kept
 * in a bounded number of resident slots and loaded when the router asks for
 * them, the engine's copies split over several I/O streams in the
 * openclawradar.com/ru article, "Эффективные оптимизации"; fr.news.hada.io,
 * Flash-MoE, "SSD Expert Streaming": one contiguous 6.75 MiB read per
 * expert).  The pool owns the placement of experts in a caller-provided
 * device arena of n_slots slots and writes the device pointer table that the
 * expert calls read (entries of non-resident experts are NULL).  Misses are
 * copied from pinned host memory by hipMemcpyAsync, spread round robin over
 * the caller's copy streams; the compute stream is made to wait on an event
 * of each, so no kernel reads a slot before its copy lands.  The least
 * recently acquired unpinned slot is evicted first, and only after the
 * last layer that used it was released (its release event is awaited on
 * the copy stream of the miss and on the stream that edits the table).  A
 * pool is used from one host thread. */
typedef struct moeq_pool moeq_pool;

#define MOEQ_POOL_MAX_COPY_STREAMS 8

/*   n_layers        layers in the host table and the device table
 *   arena           device, n_slots * slot_bytes bytes, 256-byte aligned
 *   slot_bytes      multiple of 256, >= moeq_expert_bytes(shape)
 *   host_blobs      host array [n_layers * (E + S)] of pointers to pinned host
 *                   memory (hipHostMalloc, pinned tensors), one expert blob
 *                   each, entry (l, e) at index l * (E + S) + e; the blobs
 *                   need not be contiguous.  The array is copied; the blobs
 *                   stay caller-owned.
 *   table           device array [n_layers][E + S] of pointers, set to NULL here
 *   copy_streams    host array of n_copy_streams (1 .. 8) streams for the
 *                   copies; the first also carries the table edits
 * The arena, host blobs, table and streams stay caller-owned and must
 * outlive the pool.  The pool allocates its host metadata and events.
 * MOEQ_E_INVALID if a host blob is not pinned. */
int moe_pool_create(const moeq_shape* shape, int n_layers, void* arena, int64_t n_slots, int64_t slot_bytes,
                    const void* const* host_blobs, const void** table, void* const* copy_streams,
                    int n_copy_streams, moeq_pool** out);

/* Every expert resident, blob i in slot i (needs n_slots >= n_layers*(E+S));
 * `stream` waits for the copy. */
int moe_pool_make_resident(moeq_pool* pool, void* stream);

/* Makes the experts `ids` (host int32 [n], duplicates allowed, the shared
 * expert is id E) of `layer` resident and pins them until moe_pool_release
 * for the layer.  Queues the copies of the misses; `compute_stream` waits
 * for them.  `view` receives the table to pass to the expert calls.
 * MOEQ_E_POOL_EXHAUSTED (nothing changed) when the misses need more slots
 * than are unpinned; MOEQ_E_INVALID for a bad id or a layer acquired twice
 * without a release. */
int moe_pool_acquire(moeq_pool* pool, int layer, const int32_t* ids, int n, void* compute_stream,
                     moeq_experts* view);

/* Temporal prefetch (openclawradar.com/ru, "Эффективные оптимизации": the
 * next token reuses many of the previous token's experts, so their loads
 * can start before routing resolves): copies the experts `ids` (host int32
 * [n]) of `layer` that are not resident into unpinned slots (empty first,
 * else least recently used) on the first copy stream, without pinning them;
 * resident ones become most recently used.  Stops quietly when no unpinned
 * slot is left.  A later acquire that finds them is a hit whose compute
 * stream waits for these copies.  The copies count in the bytes-copied
 * statistic; hits and misses count at acquire. */
int moe_pool_prefetch(moeq_pool* pool, int layer, const int32_t* ids, int n);

/* Unpins the layer's slots once the work queued so far on compute_stream is
 * done (an event is recorded there). */
int moe_pool_release(moeq_pool* pool, int layer, void* compute_stream);

/* out[4]: hits, misses, bytes copied, evictions. */
int moe_pool_stats(const moeq_pool* pool, int64_t* out);

/* Synchronises the copy stream and frees the pool's host state. */
void moe_pool_destroy(moeq_pool* pool);

/* The pool's placement and eviction decisions alone, with no device: same
 * policy object as moe_pool_*, for host-side checks.  acquire writes, for
 * each distinct id in first-appearance order, its slot, the entry
 * (layer * per_layer + expert) it evicted or -1, and 1 if it missed;
 * n_out = number of distinct ids.  stats: hits, misses, 0, evictions. */
typedef struct moeq_poolsim moeq_poolsim;
int moeq_poolsim_create(int n_layers, int per_layer, int64_t n_slots, moeq_poolsim** out);
int moeq_poolsim_make_resident(moeq_poolsim* pool);
int moeq_poolsim_acquire(moeq_poolsim* pool, int layer, const int32_t* ids, int n, int32_t* slots,
                         int32_t* evicted, int32_t* missed, int32_t* n_out);
int moeq_poolsim_prefetch(moeq_poolsim* pool, int layer, const int32_t* ids, int n, int32_t* slots,
                          int32_t* evicted, int32_t* n_out);
int moeq_poolsim_release(moeq_poolsim* pool, int layer);
int moeq_poolsim_stats(const moeq_poolsim* pool, int64_t* out);
void moeq_poolsim_destroy(moeq_poolsim* pool);

#ifdef __cplusplus
}
#endif

#endif /* MOEQ_H */
