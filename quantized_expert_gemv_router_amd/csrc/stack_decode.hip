// One decode token through L stacked MoE layers in a single persistent
// launch (Flash-MoE, fr.news.hada.io, "Deferred GPU Expert Compute": the
// combined output, norm and residual stay on the GPU and feed the next
// layer; removing per-layer submission cost, ~30 us per layer on the Metal
// engine of the openclawradar.com/ru page ("CMD2"), is what a single
// launch does here).
//
// Per layer l, with h the residual stream (fp32, resident):
//   xhat = h / sqrt(mean(h^2) + 1e-6)           unit-weight RMS norm
//   logits = Wr_l xhat (fp64), top-K, softmax   router
//   for each selected expert and the shared one: g, u (dequant mat-vec),
//   a = silu(g) u, d = Wd a;  h <- h + sum_k w_k d_k + d_shared
//
// Grid: one workgroup of 8 waves per CU, all resident at once (the
// launcher checks that the occupancy allows one workgroup per CU).  Three all-to-all steps per layer, each a handoff of tagged
// words (payload + layer tag in one 64-bit word, polled by the readers; no
// grid barrier or fence between the phases):
//   h:       each block publishes its rows of h_{l+1}; every block polls all
//            of h, takes sum(h^2), max|h| and its router rows' partial dot
//            products from the polled registers, and after one block
//            barrier publishes its logits
//   logits:  (one tagged word each) every block polls all E logits and
//            selects top-K itself (one
//            wave: a selection network over truncated keys, else rounds on
//            the keys' high words), then streams its gate/up rows
//   a:       each block publishes silu(g)*u for its gate/up rows (two per
//            word, fp16 under a shared power of two); every block
//            polls all activations (shared and routed slots in one take),
//            then applies its down rows and the combine with the residual.
//            The shared expert does not wait for routing: its gate/up rows
//            are applied while wave 0 selects (wave 0's own row once the
//            routed rows are requested), its activations published while
//            the routed rows stream in, and its down rows requested right
//            after that publish.
// Loads are issued as early as their addresses are known and their data
// does not compete with loads on the critical path: the router and
// shared-expert pointers of every layer are cached in LDS at start; the
// next layer's router rows are requested right after h is published, the
// shared expert's gate/up rows right after the layer's logits are
// published and its down rows right after its activations are (requested
// with the router rows, both held the h poll back); its gate/up is
// computed while the routed rows stream in; the routed down rows are
// requested once the gate/up rows are consumed.  A poll's loads complete
// after every load the wave issued before them (the vector memory counter
// is in order), so whatever is requested just before a poll delays it:
// the layer's loads were placed by measurement (requesting the down rows
// with the routed gate/up rows, or the next layer's rows before the
// activation poll, both cost more than they save).  Each block owns fixed,
// contiguous rows of every matrix:
//   router rows  e in [b E/NB, (b+1) E/NB) (every thread takes the columns
//   of the h values it polls);
//   gate/up rows in pairs: rows [2p, 2p + 2) for p in [b I/2NB,
//   (b+1) I/2NB) of every selected expert (a = silu(g)*u is formed locally,
//   a pair's two activations travel in one word);
//   down rows    r in [b H/NB, (b+1) H/NB) of every selected expert (each
//   lane weights its share of every slot, one sum per row, no atomics).
// Every wait is bounded: on time-out a block sets the status word and an
// abort flag, and every block leaves the kernel.
#include "moeq_device.hpp"
#include "moeq_internal.hpp"
#include "topk.hpp"

namespace moeq {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kSpinLimit = 1 << 18;        // polls before a wait gives up
constexpr int kActPollBackoff = 3;         // s_sleep 8 (512 clocks) steps before the activation poll
constexpr int kMaxKS = 8;                  // selected + shared experts per layer
constexpr int kActSums = 4;                // per staged activation chunk: X, 1024 X', undo, pad
constexpr int kMaxLayers = 128;            // per persistent launch
constexpr int kTblPer = 8;                 // pointer-table entries per thread (E + S <= 4096)
constexpr int kTopkSlots = 8;              // logits per lane in a one-wave top-K (E <= 512)
static_assert(kWaves * MOEQ_MAX_TOPK <= 64 * 2, "top-K merge holds two candidates per lane");
static_assert(2 * kWaves >= MOEQ_MAX_TOPK, "threshold top-K: at most two samples per wave");

// ------------------------------------------------------- launch numbers
// Control words in the workspace (zero-filled once when it is allocated):
//   [32]    abort word: holds the launch's abort value while it aborts;
//   [64 + b] workgroup b's launch count: every launch runs all NB
//           workgroups once (the grid is the device's CU count, and calls
//           on one workspace do not overlap), so at the n-th launch every
//           count reads n and each workgroup derives the same launch number
//           from its own word, read and rewritten by it alone: no atomic
//           that all workgroups contend for.
// Tags are 32 bits: (n mod 2^24) << 8 in the high 24 bits and the layer
// index within the launch + 1 (1 .. 128) in the low 8 bits; the value with
// low bits 0 marks a word cleared by this launch and low bits 255 the abort
// value.  A word written by another launch therefore never carries a tag
// this launch waits for, so no grid barrier is needed between launches or
// at a launch's start: each block rewrites its own words with the cleared
// value first (which also bounds the age of every word by one launch, so
// the 24-bit launch number cannot wrap onto a stale word).  Activation words
// carry the tag's low 24 bits (16 bits of launch number), which the same
// argument covers.
constexpr int kMaxCus = 1024;                     // workgroups with a launch-count word
constexpr int kBarCounts = 64;                   // first launch-count word
constexpr int kBarWords = kBarCounts + kMaxCus;
constexpr uint32_t kAbortLow = 255u;

__device__ __forceinline__ uint32_t tag_abort_value(uint32_t tag) { return tag | kAbortLow; }

// ------------------------------------------------------------ tagged words
// A value handed from one block to the others travels as one 64-bit word:
// the payload in the low half, the tag of the layer that wrote it in the
// high half.  Readers poll the word until the tag they expect shows up, so
// the word is its own flag and no fence or grid barrier sits between the
// writer and its readers.  Each word has one writing block for the whole
// launch.  The words are double-buffered by layer parity, so a word read
// for layer l is next overwritten with layer l+2's value.  Every block owns
// at least one row of h (the launcher requires H >= blocks), and a block
// publishes its h rows of layer l+1 only after it has read everything of
// layer l (h, logits, activations); every writer of a layer-(l+2) value has
// first polled all of layer l+1's h.  So no word is overwritten before
// every block has read it, and a reader never sees a tag newer than the
// one it waits for.
__device__ __forceinline__ void put_tagged(uint64_t* p, uint32_t payload, uint32_t tag) {
  st_agent(p, ((uint64_t)tag << 32) | payload);
}

// Activations travel two to a word: the pair as fp16 values scaled by a
// shared power of two 2^s (the larger magnitude lands in [2^14, 2^15)),
// the byte s + 128, and the low 24 bits of the tag above them:
//   tag24 << 40 | (s + 128) << 32 | fp16 pair.
// fp16 keeps each value's 11 significant bits, the same rounding the staged
// chunk applies under its own power of two, so staging the decoded values
// is exact and stages what the fp32 values would (values more than 2^28
// below the pair's or the chunk's largest aside, which both forms flush).
constexpr uint32_t kActTagMask = 0xFFFFFFu;
__device__ __forceinline__ uint64_t act_cleared(uint32_t tbase) {
  return ((uint64_t)(tbase & kActTagMask) << 40) | (128ull << 32);
}
__device__ __forceinline__ void put_act_pair(uint64_t* p, float a0, float a1, uint32_t tag) {
  const float m = fmaxf(fabsf(a0), fabsf(a1));
  int sc = 0;
  if (m > 0.0f && isfinite(m)) sc = min(14 - ilogbf(m), 126);
  const float f = ldexpf(1.0f, sc);
  const uint32_t pr = pack_half2(a0 * f, a1 * f);
  st_agent(p, ((uint64_t)(tag & kActTagMask) << 40) | ((uint64_t)(uint32_t)(sc + 128) << 32) | pr);
}
__device__ __forceinline__ void act_pair_values(uint64_t w, float& a0, float& a1) {
  const int sc = (int)((uint32_t)(w >> 32) & 0xFFu) - 128;
  const float g = ldexpf(1.0f, -sc);
  a0 = half_lo((uint32_t)w) * g;
  a1 = half_hi((uint32_t)w) * g;
}

// Polls the words base[idx(i)] for the bits i set in `valid` until each
// passes match() (carries the tag the reader waits for); the words land in
// out[i].  Bounded: gives up (and raises the launch's abort value for
// `tag`) after kSpinLimit polls, or when another block has raised it.
template <int N, typename Idx, typename Match>
__device__ __forceinline__ bool take_match(const uint64_t* base, Idx idx, uint32_t valid, Match match, uint32_t tag,
                                           uint64_t (&out)[N], uint32_t* abort, int32_t* status, int& rounds) {
  uint32_t pending = valid;
  for (int spins = 0;; ++spins) {
    uint64_t v[N];
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = ((pending >> i) & 1) ? ld_agent(base + idx(i)) : 0ull;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (((pending >> i) & 1) && match(v[i])) {
        out[i] = v[i];
        pending &= ~(1u << i);
      }
    }
    if (pending == 0) {
      rounds = spins + 1;
      return true;
    }
    if ((spins & 15) == 15 && ld_agent(abort) == tag_abort_value(tag)) return false;
    if (spins > kSpinLimit) {
      set_status(status, kStatusTimeout);
      st_agent(abort, tag_abort_value(tag));
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Words whose high bits from SHIFT up carry the tag (SHIFT 32: the tag;
// SHIFT 40: its low 24 bits, the activation pairs).
template <int N, int SHIFT, typename Idx>
__device__ __forceinline__ bool take_tagged_w(const uint64_t* base, Idx idx, uint32_t valid, uint32_t tag,
                                              uint64_t (&out)[N], uint32_t* abort, int32_t* status,
                                              int& rounds) {
  const uint32_t want = SHIFT == 32 ? tag : (tag & (0xFFFFFFFFu >> (SHIFT - 32)));
  return take_match<N>(base, idx, valid, [&](uint64_t v) { return (uint32_t)(v >> SHIFT) == want; }, tag, out,
                       abort, status, rounds);
}

// Router logits travel one to a word: the fp64 logit rounded to a 36-bit
// significand (nearest, ties to even) with the tag's low 16 bits (8 bits of
// launch number above the layer byte) in the freed low bits.  Every block
// selects from the same rounded logits; the rounding (2^-37 relative) only
// decides ties closer than the fp64 sums' own order differences reach.
constexpr uint64_t kLogitTagMask = 0xFFFFull;
__device__ __forceinline__ uint64_t logit_cleared(uint32_t tbase) { return (uint64_t)(tbase & 0xFFFFu); }
__device__ __forceinline__ uint64_t logit_word(double v, uint32_t tag) {
  const uint64_t bits = (uint64_t)__double_as_longlong(v);
  return ((bits + 0x7FFFull + ((bits >> 16) & 1ull)) & ~kLogitTagMask) | (tag & 0xFFFFu);
}
__device__ __forceinline__ double logit_value(uint64_t w) { return __longlong_as_double((long long)(w & ~kLogitTagMask)); }

// Tagged 32-bit payloads: out[i] receives the payload of word idx(i).
template <int N, typename Idx>
__device__ __forceinline__ bool take_tagged(const uint64_t* base, Idx idx, uint32_t valid, uint32_t tag,
                                            uint32_t (&out)[N], uint32_t* abort, int32_t* status,
                                            int& rounds) {
  uint64_t w[N];
#pragma unroll
  for (int i = 0; i < N; ++i) w[i] = (uint64_t)out[i];
  const bool ok = take_tagged_w<N, 32>(base, idx, valid, tag, w, abort, status, rounds);
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = (uint32_t)w[i];
  return ok;
}

// Delay injection (diagnostic instantiations, JIT = 1): before each of its
// hand-off publishes a wave sleeps a pseudo-random 0 .. 63 times s_sleep 8
// (up to ~13 us), a different amount per (workgroup, wave, layer, site).
// The hand-offs carry their own ordering, so the results must not change.
template <int JIT>
__device__ __forceinline__ void jitter(int b, int wave, int li, int site) {
  if constexpr (JIT != 0) {
    uint32_t h = (uint32_t)b * 0x9E3779B1u ^ (uint32_t)(li * 4 + site) * 0x85EBCA77u ^ (uint32_t)wave * 0xC2B2AE3Du;
    h ^= h >> 15;
    h *= 0x2C1B3C6Du;
    h ^= h >> 12;
    const int n = (int)(h & 63u);
    for (int i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(8);
  }
}

// ------------------------------------------------------------------ layout
struct StackLds {
  int hs, xp, xs, ap, as, gres, lg, tbl, clk, total;
};

__host__ __device__ inline int al16(int v) { return (v + 15) & ~15; }

// Most gate/up rows a block owns: rows are handed out in pairs, contiguous
// and balanced over the blocks.
__host__ __device__ inline int gu_rows_max(int I, int nb) { return 2 * ((I / 2 + nb - 1) / nb); }

__host__ __device__ inline StackLds stack_lds_layout(int H, int I, int E, int S, int KS, int PC,
                                                     int RG, int RD, int clk_entries) {
  StackLds L;
  L.hs = 0;
  L.xp = al16(L.hs + 4 * H);
  L.xs = al16(L.xp + 2 * H);
  L.ap = al16(L.xs + 4 * kChunkSums * (H / PC));
  L.as = al16(L.ap + KS * 2 * I);
  L.gres = al16(L.as + 4 * kActSums * KS * (I / PC));
  L.lg = al16(L.gres + 4 * KS * 2 * RG);
  L.tbl = al16(L.lg + 8 * E);
  L.clk = al16(L.tbl + 8 * (E + S));
  L.total = al16(L.clk + 8 * clk_entries);
  return L;
}

// Stage word w (PW values, scaled by f) of a vector of nch chunks into its
// fp16 pairs; returns the word's share of the chunk sums {X, 1024 X'} (the
// caller folds the four words of a chunk with lane shuffles).
// Sum over the four lanes of a quad (the four words of a chunk).
__device__ __forceinline__ float2 quad_sum(float2 s) {
  s.x += __shfl_xor(s.x, 1, 64);
  s.y += __shfl_xor(s.y, 1, 64);
  s.x += __shfl_xor(s.x, 2, 64);
  s.y += __shfl_xor(s.y, 2, 64);
  return s;
}

template <int BITS>
__device__ __forceinline__ float2 stage_word(const float* v, float f, uint32_t* vec, int w, int nch) {
  constexpr int HP = Pack<BITS>::kPairsPerWord;
  uint32_t pr[HP];
  float X = 0.0f, Xs = 0.0f;
  pack_word<BITS>(v, f, pr, X, Xs);
  store_word<BITS>(vec, w, nch, pr);
  return make_float2(X, Xs);
}

template <int BITS, int CPLR, int CPLG, int RPWG, int LPRD, int CPLD, int STEPSD, int HW, int JIT>
__global__ __launch_bounds__(kThreads) void stack_kernel(StackArgs a) {
  constexpr int PC = Pack<BITS>::kPerChunk, PW = Pack<BITS>::kPerWord;
  constexpr int RPSD = 64 / LPRD;          // down rows per wave step
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ double rpart[CPLR * kWaves];
  __shared__ double ssum[kWaves];
  __shared__ float hmax[kWaves];
  __shared__ int sel[MOEQ_MAX_TOPK];
  __shared__ const uint8_t* selp[MOEQ_MAX_TOPK];   // the selected experts' blobs (null: missing)
  __shared__ double selv[MOEQ_MAX_TOPK];
  __shared__ int64_t candk[kWaves * 64];
  __shared__ int candi[kWaves * 64];
  __shared__ float selw[MOEQ_MAX_TOPK];
  __shared__ const uint16_t* rtr[kMaxLayers];
  __shared__ const uint8_t* shp[kMaxLayers];
  __shared__ float undo_x;
  __shared__ uint32_t s_tbase;
  __shared__ int fail_flag;

  int tid = threadIdx.x, lane = tid & 63;   // re-derived opaquely each layer, as b
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NB = gridDim.x;
  int b = blockIdx.x;   // re-derived opaquely each layer (see the layer loop)
  const int H = a.H, I = a.I, E = a.E, K = a.K, S = a.S, KS = K + S, L = a.L;
  const int nchG = H / PC, nchD = I / PC;
  const int RG = gu_rows_max(I, NB), RD = (H + NB - 1) / NB;

  const int clk0 = a.clocks ? L * kStackClockEvents : 0;
  const StackLds LL = stack_lds_layout(H, I, E, S, KS, PC, RG, RD, clk0 + (a.bclocks ? L * kBlockClockEvents : 0));
  float* hs = reinterpret_cast<float*>(smem + LL.hs);               // [H]
  uint32_t* xp = reinterpret_cast<uint32_t*>(smem + LL.xp);         // [H/2]
  float* xs = reinterpret_cast<float*>(smem + LL.xs);               // [H/PC][kChunkSums]
  uint32_t* ap = reinterpret_cast<uint32_t*>(smem + LL.ap);         // [KS][I/2]
  float* as = reinterpret_cast<float*>(smem + LL.as);               // [KS][I/PC][kActSums]
  float* gres = reinterpret_cast<float*>(smem + LL.gres);           // [KS][2][RG]
  double* lg = reinterpret_cast<double*>(smem + LL.lg);             // [E]
  const uint8_t** tbl = reinterpret_cast<const uint8_t**>(smem + LL.tbl);  // [E + S], this layer
  int64_t* clk = reinterpret_cast<int64_t*>(smem + LL.clk);         // [L][kStackClockEvents] if timed
  int64_t* bclk = clk + clk0;                                        // [L][kBlockClockEvents] if timed

  // this launch's number, from the workgroup's own launch count (first, so
  // that it is back by the time the tags are needed)
  if (tid == 0) {
    uint32_t* const count = a.bar + kBarCounts + blockIdx.x;
    const uint32_t n = ld_agent(count);
    st_agent(count, n + 1u);
    s_tbase = n << 8;
  }

  // This block's rows, contiguous and balanced: router rows [rlo, rhi),
  // gate/up rows [glo, ghi), rows of h [dlo, dhi) (at least one when H >=
  // blocks).  Contiguous ownership keeps a tagged 128-byte line to few
  // writing blocks (one for h) while readers still poll in address order.
  int rlo, rhi, glo, ghi, dlo, dhi;
  auto set_rows = [&]() {
    rlo = b * E / NB;
    rhi = (b + 1) * E / NB;
    glo = 2 * (b * (I / 2) / NB);   // in pairs: a pair of activations travels in one word
    ghi = 2 * ((b + 1) * (I / 2) / NB);
    dlo = b * H / NB;
    dhi = (b + 1) * H / NB;
  };
  set_rows();
  // router: RW (<= CPLR) rows per block, rows rlo + k; each thread takes
  // the columns of the h values it polls (2p, 2p+1 for p = tid + i*kThreads)
  const int RW = a.router_rows;
  const int tbl_n = E + S;

  uint32_t wr[CPLR][HW];
  u32x4 qg[RPWG][CPLG];
  uint32_t sg[RPWG][CPLG];
  uint2 qhg[RPWG][CPLG];           // 3-bit: the chunks' high-bit plane words
  u32x4 qd[STEPSD][CPLD];          // routed slots' down rows
  uint32_t sd[STEPSD][CPLD];
  uint2 qhd[STEPSD][CPLD];
  u32x4 qsh[CPLD];                 // the shared expert's down rows
  uint32_t ssh[CPLD];
  uint2 qhsh[CPLD];
  const uint8_t* tnext[kTblPer];   // this layer's pointer-table row, in flight to LDS

  // gate/up rows: register slot m = 0 holds the shared expert's rows (task
  // u = wave), slots m >= 1 the routed slots' (task u = (m - 1) * kWaves +
  // wave, slot u / 2RG); within a slot, task u % 2RG is section (gate, up)
  // and row glo + i.  The shared rows are requested a layer ahead and
  // stay in their registers while the routed rows are requested.
  auto gu_task = [&](int m, int& j, int& sec, int& row) -> bool {
    int u;
    bool valid;
    if (m == 0) {
      u = wave;
      j = K;
      valid = S > 0 && u < 2 * RG;
    } else {
      u = (m - 1) * kWaves + wave;
      j = u / (2 * RG);
      valid = j < K;
    }
    const int tj = u % (2 * RG);
    sec = tj / RG;
    row = glo + tj % RG;
    return valid && row < ghi;
  };
  // Loads are planned (every LDS read they need) before any is issued: an
  // LDS read between loads makes the compiler wait for the loads in flight.
  // Every lane issues its loads unconditionally; what a lane does not need
  // is outside its buffer range (zeros, no memory access) or re-reads a
  // valid address, and the dot products skip it.
  rsrc_t rplan[CPLR];              // this block's router rows (empty range: no row)
  auto plan_router = [&](int li) {
    const uint16_t* base = uniform_ptr(rtr[li]);
#pragma unroll
    for (int k = 0; k < CPLR; ++k) {
      const int r = rlo + k;
      const bool have = k < RW && r < rhi;
      rplan[k] = make_rsrc(base + (int64_t)(have ? r : 0) * H, have ? (uint32_t)H * 2u : 0u);
    }
  };
  auto issue_router = [&]() {
#pragma unroll
    for (int k = 0; k < CPLR; ++k)
#pragma unroll
      for (int i = 0; i < HW; ++i) wr[k][i] = load_rsrc_b32(rplan[k], (uint32_t)(tid + i * kThreads) * 4u);
  };
  // gate/up rows of the register slots m in [mlo, mhi) (constants at every
  // call); gu_task is uniform over a wave, so each row is one scalar buffer
  // resource
  rsrc_t gq[RPWG];               // the task's expert blob, or an empty range: no task
  uint32_t gqo[RPWG], gso[RPWG]; // byte offsets of its quantized row and scale/bias words
  bool ghave[RPWG];
  auto plan_gu = [&](int mlo, int mhi, const uint8_t* shared_blob) {
    const uint32_t row_bytes = (uint32_t)H * BITS / 8;
    const uint32_t gpr = H / 64;
    const uint32_t sb_off = 3u * (uint32_t)H * I * BITS / 8;
    const uint32_t blob_bytes = sb_off + 3u * (uint32_t)(H / 64) * I * 4u;
#pragma unroll
    for (int m = 0; m < RPWG; ++m) {
      if (m < mlo || m >= mhi) continue;
      int j, sec, row;
      ghave[m] = gu_task(m, j, sec, row);
      // routed slots: the selection; the shared slot: shared_blob.  A missing expert (null) loads nothing.
      const int jj = ghave[m] ? j : K;
      const uint8_t* blob = uniform_ptr(jj < K ? selp[jj] : shared_blob);
      const uint32_t r = ghave[m] ? (uint32_t)(sec * I + row) : 0u;   // row of [gate; up]
      gq[m] = make_rsrc(blob, ghave[m] && blob != nullptr ? blob_bytes : 0u);
      gqo[m] = r * row_bytes;
      gso[m] = sb_off + r * gpr * 4u;
    }
  };
  // chunk-major: the dots take one staged x chunk at a time against every
  // row of the wave, so each chunk is read from LDS once
  auto issue_gu = [&](int mlo, int mhi) {
#pragma unroll
    for (int c = 0; c < CPLG; ++c) {
      const int cc = min(lane + 64 * c, nchG - 1);   // past the row: the dots skip it
#pragma unroll
      for (int m = 0; m < RPWG; ++m) {
        if (m < mlo || m >= mhi) continue;
        qg[m][c] = load_rsrc_b128(gq[m], gqo[m] + (uint32_t)cc * 16u);
        if constexpr (BITS == 3)   // a 3-bit row: the 2-bit low plane, then the high-bit plane
          qhg[m][c] = load_rsrc_b64(gq[m], gqo[m] + (uint32_t)H / 4u + (uint32_t)cc * 8u);
        sg[m][c] = load_rsrc_b32(gq[m], gso[m] + (uint32_t)(cc * PC / 64) * 4u);
      }
    }
    issue_fence();
  };
  auto gu_dots = [&](int mlo, int mhi) {
    bool live[RPWG];
    bool any = false;
#pragma unroll
    for (int m = 0; m < RPWG; ++m) {
      int j, sec, row;
      live[m] = m >= mlo && m < mhi && gu_task(m, j, sec, row);
      any = any || live[m];
    }
    if (!any) return;
    float part[RPWG];
#pragma unroll
    for (int m = 0; m < RPWG; ++m) part[m] = 0.0f;
#pragma unroll
    for (int c = 0; c < CPLG; ++c) {
      const int cc = lane + 64 * c;
      const int ccl = min(cc, nchG - 1);
      const XChunk<BITS> x = load_xchunk<BITS>(xp, ccl, nchG);
      const float2 xsum = *reinterpret_cast<const float2*>(xs + kChunkSums * ccl);
#pragma unroll
      for (int m = 0; m < RPWG; ++m)
        if (live[m] && cc < nchG) part[m] += chunk_term<BITS>(chunk_dot_q<BITS>(qg[m][c], qhg[m][c], x), sg[m][c], xsum);
    }
    const float ux = undo_x;
#pragma unroll
    for (int m = 0; m < RPWG; ++m) {
      if (!live[m]) continue;
      int j, sec, row;
      gu_task(m, j, sec, row);
      const float v = wave_sum_dpp(part[m]) * ux;
      if (lane == 0) gres[(j * 2 + sec) * RG + (row - glo)] = v;
    }
  };
  // down rows: a wave owns RPSD of the block's output rows (LPRD lanes
  // each), for every slot: step s is routed slot s, so the combine of a row
  // stays in the wave; the shared expert's rows have their own registers
  rsrc_t dsrc[STEPSD];       // routed slot s's expert blob, or an empty range
  const uint32_t blob_bytes_all = 3u * (uint32_t)H * I * BITS / 8 + 3u * (uint32_t)(H / 64) * I * 4u;
  auto down_row = [&](int& row) {
    const int i = wave * RPSD + lane / LPRD;
    row = i < RD && dlo + i < dhi ? dlo + i : H;   // H: no row
  };
  auto plan_down = [&]() {   // from the selection
#pragma unroll
    for (int s = 0; s < STEPSD; ++s) {
      const uint8_t* blob = uniform_ptr(s < K ? selp[s] : nullptr);
      dsrc[s] = make_rsrc(blob, blob != nullptr ? blob_bytes_all : 0u);
    }
  };
  auto down_load = [&](rsrc_t src, u32x4 (&q)[CPLD], uint32_t (&sbw)[CPLD], uint2 (&qh)[CPLD]) {
    const uint32_t row_bytes = (uint32_t)I * BITS / 8;
    const uint32_t gpr = I / 64;
    const uint32_t q_off = 2u * (uint32_t)H * I * BITS / 8;
    const uint32_t sb_off = 3u * (uint32_t)H * I * BITS / 8 + 2u * (uint32_t)H * (I / 64) * 4u;
    const int sub = lane % LPRD;
    int row;
    down_row(row);
    if (row >= H) row = 0;   // padding lane: re-reads a valid row, skipped by the dots
#pragma unroll
    for (int c = 0; c < CPLD; ++c) {
      const int cc = min(sub + LPRD * c, nchD - 1);
      q[c] = load_rsrc_b128(src, q_off + (uint32_t)row * row_bytes + (uint32_t)cc * 16u);
      if constexpr (BITS == 3)
        qh[c] = load_rsrc_b64(src, q_off + (uint32_t)row * row_bytes + (uint32_t)I / 4u + (uint32_t)cc * 8u);
      sbw[c] = load_rsrc_b32(src, sb_off + ((uint32_t)row * gpr + (uint32_t)(cc * PC / 64)) * 4u);
    }
  };
  auto issue_down = [&]() {
#pragma unroll
    for (int s = 0; s < STEPSD; ++s) down_load(dsrc[s], qd[s], sd[s], qhd[s]);
    issue_fence();
  };
  auto issue_down_shared = [&](const uint8_t* sblob) {   // the layer's shared expert (at most one)
    const uint8_t* blob = uniform_ptr(sblob);
    down_load(make_rsrc(blob, blob != nullptr ? blob_bytes_all : 0u), qsh, ssh, qhsh);
    issue_fence();
  };
  auto load_tbl_row = [&](int layer) {   // into registers; stored to LDS after the next barrier
    const void* const* row = a.blobs + (int64_t)layer * tbl_n;
#pragma unroll
    for (int i = 0; i < kTblPer; ++i) {
      const int e = tid + i * kThreads;
      tnext[i] = e < tbl_n ? static_cast<const uint8_t*>(row[e]) : nullptr;
    }
  };
  auto store_tbl_row = [&]() {
#pragma unroll
    for (int i = 0; i < kTblPer; ++i) {
      const int e = tid + i * kThreads;
      if (e < tbl_n) tbl[e] = tnext[i];
    }
  };
  // diagnostic phase stamps (block 0, after a block-wide barrier)
  auto stamp = [&](int li, int ev) {
    if (a.clocks && b == 0) {
      block_sync_lds();
      if (tid == 0) clk[li * kStackClockEvents + ev] = (int64_t)wall_clock64();
    }
  };
  // diagnostic stamps from wave 0 alone (no block barrier)
  auto stamp0 = [&](int li, int ev) {
    if (a.clocks && b == 0 && tid == 0) clk[li * kStackClockEvents + ev] = (int64_t)wall_clock64();
  };
  // diagnostic stamps of every block, by thread 0 (no block barrier):
  // 0 layer start, 1 h polled, 2 own logits published, 3 logits polled,
  // 4 top-K (after its barrier), 5 routed gate/up dots, 6 routed activations
  // published, 7 top-K selected (wave 0, before the barrier), 8 activations
  // polled, 9 h published (the last wave's), 14 routed gate/up rows
  // requested, 15 shared activations published; poll rounds (most over the
  // threads): 10 h, 11 logits, 12 shared activations, 13 routed activations
  auto bstamp = [&](int li, int ev) {
    if (a.bclocks && tid == 0) bclk[li * kBlockClockEvents + ev] = (int64_t)wall_clock64();
  };
  auto bcount = [&](int li, int ev, int n) {   // maximum over the block's threads (one LDS atomic per wave)
    if (a.bclocks) {
      const int m = wave_max_i32(n);
      if (lane == 0)
        atomicMax(reinterpret_cast<unsigned long long*>(bclk + li * kBlockClockEvents + ev), (unsigned long long)m);
    }
  };

  // prologue: router and shared-expert pointers of every layer, first rows
  for (int li = tid; li < L; li += kThreads) {
    rtr[li] = a.routers[a.layer0 + li];
    shp[li] = S > 0 ? static_cast<const uint8_t*>(a.blobs[(int64_t)(a.layer0 + li) * tbl_n + E]) : nullptr;
  }
  if (tid == 0) fail_flag = 0;
  if (a.bclocks)
    for (int i = tid; i < L * kBlockClockEvents; i += kThreads) bclk[i] = 0;
  block_sync_lds();
  // tags of this launch: tbase + layer + 1
  const uint32_t tbase = __builtin_amdgcn_readfirstlane(s_tbase);
  const uint64_t cleared = (uint64_t)tbase << 32;
  // this block's tagged words carry this launch's cleared value before any
  // layer's write; only the block's own later stores need ordering after
  // the clears (other launches' tags never match), so each thread waits for
  // its clears to complete and one block barrier follows: no grid barrier
  for (int par = 0; par < 2; ++par) {
    uint64_t* lw = a.lwords + (int64_t)par * 2 * E;
    uint64_t* aw = a.awords + (int64_t)par * KS * I;
    uint64_t* hw = a.hwords + (int64_t)par * H;
    for (int j = tid; j < RW; j += kThreads) {
      const int r = rlo + j;
      if (r < rhi) st_agent(lw + r, logit_cleared(tbase));
    }
    for (int t = tid; t < KS * (RG / 2); t += kThreads) {
      const int j = t / (RG / 2), r0 = glo + 2 * (t - j * (RG / 2));
      if (r0 < ghi) st_agent(aw + (int64_t)j * (I / 2) + r0 / 2, act_cleared(tbase));
    }
    for (int i = tid; i < RD; i += kThreads) {
      const int row = dlo + i;
      if (row < dhi) st_agent(hw + row, cleared);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  block_sync_lds();
  plan_router(0);
  issue_router();
  uint32_t* const abort_word = a.bar + 32;
  auto block_failed = [&](bool ok) -> bool {   // whole block
    if (!ok) fail_flag = 1;
    block_sync_lds();
    return fail_flag != 0;
  };

  for (int li = 0; li < L; ++li) {
    // Row offsets and addresses derived from the block and thread indices
    // are cheap to recompute; hoisted out of the loop they stay live across
    // all phases and push registers into scratch, whose reloads are memory
    // round trips.
    {
      int zero;
      asm volatile("s_mov_b32 %0, 0" : "=s"(zero));
      b = (int)blockIdx.x + zero;
      asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
      lane = tid & 63;
      set_rows();
    }
    stamp(li, 0);
    bstamp(li, 0);
    const int par = li & 1;
    const uint64_t* hw_in = a.hwords + (int64_t)par * H;
    uint64_t* hw_out = a.hwords + (int64_t)(par ^ 1) * H;
    uint64_t* lw = a.lwords + (int64_t)par * 2 * E;
    uint64_t* aw = a.awords + (int64_t)par * KS * I;
    // ------------------------------------------------------------ phase R
    // h -> LDS with sum of squares (fp64) and max |h|
    {
      uint64_t hv[HW];
      bool ok = true;
      if (li == 0) {
        const uint64_t* src = reinterpret_cast<const uint64_t*>(a.h);
#pragma unroll
        for (int i = 0; i < HW; ++i) {
          const int p = tid + i * kThreads;
          hv[i] = (2 * p < H) ? ld_agent(src + p) : 0ull;
        }
      } else {
        uint32_t hw[2 * HW];
        uint32_t valid = 0;
#pragma unroll
        for (int i = 0; i < HW; ++i) {
          hw[2 * i] = hw[2 * i + 1] = 0u;
          if (2 * (tid + i * kThreads) < H) valid |= 3u << (2 * i);
        }
        int nr = 0;
        ok = take_tagged<2 * HW>(hw_in, [&](int i) { return 2 * (tid + (i >> 1) * kThreads) + (i & 1); },
                                 valid, tbase + (uint32_t)li, hw, abort_word, a.status, nr);
        bcount(li, 10, nr);
#pragma unroll
        for (int i = 0; i < HW; ++i) hv[i] = ((uint64_t)hw[2 * i + 1] << 32) | hw[2 * i];
      }
      if (block_failed(ok)) return;
      // sum of squares and max |h| (for the norm and the fp16 rescale) and
      // this thread's share of the router rows' dot products, from the
      // polled registers: one barrier then completes the logits
      double ss = 0.0;
      double racc[CPLR];
#pragma unroll
      for (int k = 0; k < CPLR; ++k) racc[k] = 0.0;
      float mx = 0.0f;
#pragma unroll
      for (int i = 0; i < HW; ++i) {
        const int p = tid + i * kThreads;
        const float lo = __uint_as_float((uint32_t)hv[i]), hi = __uint_as_float((uint32_t)(hv[i] >> 32));
        if (2 * p < H) {
          *reinterpret_cast<float2*>(hs + 2 * p) = make_float2(lo, hi);
          ss = fma((double)lo, (double)lo, ss);
          ss = fma((double)hi, (double)hi, ss);
          mx = fmaxf(mx, fmaxf(fabsf(lo), fabsf(hi)));
        }
#pragma unroll
        for (int k = 0; k < CPLR; ++k) {   // zeros past the row (buffer range)
          racc[k] = fma((double)bf16_lo(wr[k][i]), (double)lo, racc[k]);
          racc[k] = fma((double)bf16_hi(wr[k][i]), (double)hi, racc[k]);
        }
      }
      ss = wave_sum_f64_dpp(ss);
      mx = wave_max_dpp(mx);
#pragma unroll
      for (int k = 0; k < CPLR; ++k) racc[k] = wave_sum_f64_dpp(racc[k]);
      if (lane == 0) {
        ssum[wave] = ss;
        hmax[wave] = mx;
#pragma unroll
        for (int k = 0; k < CPLR; ++k) rpart[k * kWaves + wave] = racc[k];
      }
    }
    block_sync_lds();
    stamp(li, 1);
    bstamp(li, 1);
    double ss = 0.0;
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) { ss += ssum[i]; mx = fmaxf(mx, hmax[i]); }
    const double inv = a.no_norm ? 1.0 : 1.0 / sqrt(ss / (double)H + 1e-6);
    const uint32_t tag = tbase + (uint32_t)li + 1u;
    jitter<JIT>(b, wave, li, 0);
    if (tid < RW && rlo + tid < rhi) {   // this block's logits, one word each
      double d = 0.0;
      for (int w = 0; w < kWaves; ++w) d += rpart[tid * kWaves + w];
      st_agent(lw + rlo + tid, logit_word(d * inv, tag));
    }
    bstamp(li, 2);
    // the shared expert's gate/up rows, in flight while x is staged, the
    // logits are polled and top-K runs (requested before the h poll they
    // held it back)
    if (S > 0) {
      plan_gu(0, 1, shp[li]);
      issue_gu(0, 1);
    }
    // xhat -> fp16 pairs, one packed word per thread; the norm and the
    // rescale come from the h pass above, so no further reductions
    {
      const float mul = (float)inv;
      const float p = pow2_stage_factor(mx * mul);
      const float f = mul * p;
      if (tid == 0) undo_x = 1.0f / p;
      const int nw = H / PW;
      for (int w0 = 0; w0 < nw; w0 += kThreads) {
        const int w = w0 + tid;
        float2 s = make_float2(0.0f, 0.0f);
        if (w < nw) {
          float v[PW];
#pragma unroll
          for (int j = 0; j < PW; ++j) v[j] = hs[w * PW + j];
          s = stage_word<BITS>(v, f, xp, w, nchG);
        }
        s = quad_sum(s);
        if ((tid & 3) == 0 && w < nw) *reinterpret_cast<float2*>(xs + kChunkSums * (w >> 2)) = s;
      }
    }
    block_sync_lds();
    stamp(li, 2);

    // ------------------------------------------------------------ phase G
    // this layer's pointer-table row lands while the logits are polled
    load_tbl_row(a.layer0 + li);
    for (int e0 = 0; e0 < E; e0 += kThreads) {   // one logit (one word) per thread per pass
      const int e = e0 + tid;
      uint64_t w[1] = {0ull};
      int nr = 0;
      const uint32_t t16 = tag & 0xFFFFu;
      const bool ok = take_match<1>(lw + e, [](int i) { return i; }, e < E ? 1u : 0u,
                                    [&](uint64_t v) { return (uint32_t)(v & kLogitTagMask) == t16; }, tag, w,
                                    abort_word, a.status, nr);
      bcount(li, 11, nr);
      if (e < E) lg[e] = logit_value(w[0]);
      // the table row's loads were issued before the poll's, so they are in;
      // the barrier below publishes both to every wave
      if (e0 + kThreads >= E) store_tbl_row();
      if (block_failed(ok)) return;
    }
    stamp0(li, 12);
    bstamp(li, 3);
    // top-K: wave 0 selects from all E logits (up to eight per lane; one
    // wave alone on its SIMD finishes sooner than eight sharing four), one
    // barrier hands the selection to the block; beyond 512 experts the
    // waves select together.  Up to four experts the selection network
    // (one pass of sorted four-lists through the wave) decides whenever
    // the truncated keys separate the K best from the rest; rounds of wave
    // maxima on the full keys decide otherwise.
    if (E <= 64 * kTopkSlots) {
      if (wave == 0) {
        int win;
        if (K <= 4 && wave_topk_net(lg, E, K, win)) {
          if (lane < K) sel[lane] = win;
        } else {
          int64_t kk[kTopkSlots];
#pragma unroll
          for (int i = 0; i < kTopkSlots; ++i) {
            const int e = lane + 64 * i;
            kk[i] = e < E ? order_key(lg[e]) : kNoKey;
          }
          wave_select_hi<kTopkSlots>(kk, K, [&](int r, int w) { sel[r] = w; });
        }
        // the selected blobs, so the routed loads are planned from one read
        if (lane < K) {
          const int e = sel[lane];
          selp[lane] = (unsigned)e < (unsigned)E ? tbl[e] : nullptr;
        }
        bstamp(li, 7);
      } else if (S > 0) {
        gu_dots(0, 1);   // the other waves apply their shared rows meanwhile
      }
      block_sync_lds();
    } else {
      block_topk_keys<kWaves, kTblPer, 2>(lg, E, K, candk, candi, sel, selv);
      if (tid < K) {
        const int e = sel[tid];
        selp[tid] = (unsigned)e < (unsigned)E ? tbl[e] : nullptr;
      }
      block_sync_lds();
    }
    stamp0(li, 14);
    bstamp(li, 4);
    plan_gu(1, RPWG, nullptr);       // routed gate/up rows
    issue_gu(1, RPWG);
    bstamp(li, 14);
    stamp0(li, 5);
    // while they arrive: wave 0 checks the selected experts' blobs and
    // records the trace
    if (wave == 0 && lane < K) {
      const int e = sel[lane];
      if (selp[lane] == nullptr) set_status(a.status, kStatusBadExpert);
      if (b == 0 && a.topk_trace) a.topk_trace[(int64_t)li * K + lane] = e;
    }
    stamp0(li, 15);
    // the shared expert's gate/up rows (requested a layer ahead) while the
    // routed rows arrive, and its activations published at once
    if (S > 0) {
      if (wave == 0 || E > 64 * kTopkSlots) gu_dots(0, 1);   // (the other waves took theirs during top-K)
      stamp0(li, 3);
      block_sync_lds();
      jitter<JIT>(b, wave, li, 1);
      for (int t = tid; t < RG / 2; t += kThreads) {
        const int i = 2 * t, r0 = glo + i;
        if (r0 < ghi) {
          const float g0 = gres[(K * 2) * RG + i], u0 = gres[(K * 2 + 1) * RG + i];
          const float g1 = gres[(K * 2) * RG + i + 1], u1 = gres[(K * 2 + 1) * RG + i + 1];
          put_act_pair(aw + (int64_t)K * (I / 2) + r0 / 2, g0 / (1.0f + __expf(-g0)) * u0,
                       g1 / (1.0f + __expf(-g1)) * u1, tag);
        }
      }
      stamp0(li, 4);
      bstamp(li, 15);
      // its down rows, in flight while the routed rows are applied
      issue_down_shared(shp[li]);
    }
    gu_dots(1, RPWG);
    stamp0(li, 13);
    bstamp(li, 5);
    block_sync_lds();
    stamp(li, 6);
    jitter<JIT>(b, wave, li, 2);
    for (int t = tid; t < K * (RG / 2); t += kThreads) {
      const int j = t / (RG / 2), i = 2 * (t - j * (RG / 2)), r0 = glo + i;
      if (r0 < ghi) {
        const float g0 = gres[(j * 2) * RG + i], u0 = gres[(j * 2 + 1) * RG + i];
        const float g1 = gres[(j * 2) * RG + i + 1], u1 = gres[(j * 2 + 1) * RG + i + 1];
        put_act_pair(aw + (int64_t)j * (I / 2) + r0 / 2, g0 / (1.0f + __expf(-g0)) * u0,
                     g1 / (1.0f + __expf(-g1)) * u1, tag);
      }
    }
    bstamp(li, 6);
    // down rows of every slot, in flight while the activations arrive (not
    // earlier: they would share the memory system with the gate/up rows
    // every block is waiting for, or hold back the publish above)
    plan_down();
    issue_down();
    stamp0(li, 7);
    stamp(li, 8);

    // ------------------------------------------------------------ phase D
    // activations of slots [s0, s0 + ns): one packed word of one slot per
    // thread, staged with a power-of-two scale per 16-byte chunk (the four
    // threads of a chunk agree on it with two lane shuffles), so staging
    // needs no block-wide maximum; the block barrier after it also settles
    // a failed poll
    auto take_acts = [&](int s0, int ns, int count_ev) -> bool {
      const int nwa = I / PW;
      const int total = ns * nwa;
      bool got_all = true;
      for (int t0 = 0; t0 < total; t0 += kThreads) {
        const int t = t0 + tid;
        const bool ok = t < total;
        const int m = ok ? s0 + t / nwa : s0, w = ok ? t - (m - s0) * nwa : 0;
        constexpr int PP = PW / 2;   // activation pairs per word
        float v[PW];
        uint64_t raw[PP];
#pragma unroll
        for (int j = 0; j < PP; ++j) raw[j] = 128ull << 32;   // zeros under scale 2^0
        const uint64_t* src = aw + (int64_t)m * (I / 2) + (int64_t)w * PP;
        int nr = 0;
        const bool got = take_tagged_w<PP, 40>(src, [](int j) { return j; },
                                               ok ? (uint32_t)((1ull << PP) - 1) : 0u, tag, raw, abort_word,
                                               a.status, nr);
        bcount(li, count_ev, nr);
        got_all = got_all && got;
        float lm = 0.0f;
#pragma unroll
        for (int j = 0; j < PP; ++j) {
          act_pair_values(raw[j], v[2 * j], v[2 * j + 1]);
          lm = fmaxf(lm, fmaxf(fabsf(v[2 * j]), fabsf(v[2 * j + 1])));
        }
        lm = fmaxf(lm, __shfl_xor(lm, 1, 64));
        lm = fmaxf(lm, __shfl_xor(lm, 2, 64));
        const float p = pow2_stage_factor(lm);
        float2 sums = make_float2(0.0f, 0.0f);
        if (ok) sums = stage_word<BITS>(v, p, ap + (int64_t)m * (I / 2), w, nchD);
        sums = quad_sum(sums);
        if (ok && (tid & 3) == 0)
          *reinterpret_cast<float4*>(as + kActSums * (m * nchD + (w >> 2))) =
              make_float4(sums.x, sums.y, 1.0f / p, 0.0f);
      }
      return !block_failed(got_all);
    };
    // this lane's share of one slot's down row against its staged
    // activations (the LPRD lanes of a row group hold the row's chunks)
    auto down_part = [&](int s, const u32x4 (&q)[CPLD], const uint32_t (&sbw)[CPLD], const uint2 (&qh)[CPLD],
                         bool ok) -> float {
      const int sub = lane % LPRD;
      float part = 0.0f;
#pragma unroll
      for (int c = 0; c < CPLD; ++c) {
        const int cc = min(sub + LPRD * c, nchD - 1);
        const XChunk<BITS> x = load_xchunk<BITS>(ap + (int64_t)s * (I / 2), cc, nchD);
        const float4 xsm = *reinterpret_cast<const float4*>(as + kActSums * (s * nchD + cc));
        if (ok && sub + LPRD * c < nchD)
          part += chunk_term<BITS>(chunk_dot_q<BITS>(q[c], qh[c], x), sbw[c], make_float2(xsm.x, xsm.y)) * xsm.z;
      }
      return part;
    };
    const int sub = lane % LPRD;
    // shared and routed activations in one take
    // back-off before the first activation poll: issued at once, its first
    // round reads the words before the slowest blocks have published them
    // and, queued behind the down rows, returns late, so a second round is
    // needed; ~0.64 us later the first round mostly finds them all
    // wave 0 takes the softmax weights first (read by the combine after the
    // activation take's block barrier), off the path of the routed rows
    if (wave == 0) {
      if (lane < K) {
        const int e = sel[lane];
        selv[lane] = (unsigned)e < (unsigned)E ? lg[e] : -INFINITY;
      }
      const float w = a.no_renorm ? wave_softmax_weight(lg, E, K, selv, true)
                                  : wave_softmax_selected(selv, K);
      if (lane < K) selw[lane] = w;
    }
    for (int d = 0; d < kActPollBackoff; ++d) __builtin_amdgcn_s_sleep(8);
    if (!take_acts(0, KS, 13)) return;
    stamp0(li, 17);
    bstamp(li, 8);
    stamp(li, 9);
    jitter<JIT>(b, wave, li, 3);
    {
      int drow;
      down_row(drow);
      const bool dok = drow < H;
      // every slot's share weighted in the lane (the shared expert first,
      // then the slots in rank order), then one sum over the row group:
      // valid in lane LPRD-1
      float part = S > 0 ? down_part(K, qsh, ssh, qhsh, dok) : 0.0f;
#pragma unroll
      for (int s = 0; s < STEPSD; ++s) {
        if (s >= K) break;
        part = fmaf(selw[s], down_part(s, qd[s], sd[s], qhd[s], dok), part);
      }
      const float dsum = group_sum_dpp<LPRD>(part);
      const float acc = dok ? hs[drow] + dsum : 0.0f;
      if (dok && sub == LPRD - 1) {
        if (a.h_trace) a.h_trace[(int64_t)li * H + drow] = hs[drow];
        if (li + 1 == L) a.h[drow] = acc;   // complete when the launch ends
        else put_tagged(hw_out + drow, __float_as_uint(acc), tag);
      }
    }
    stamp0(li, 18);
    if (a.bclocks && lane == 0)
      atomicMax(reinterpret_cast<unsigned long long*>(bclk + li * kBlockClockEvents + 9),
                (unsigned long long)wall_clock64());
    stamp(li, 10);
    if (li + 1 == L) break;
    // next layer: router rows, in flight while h arrives (the shared
    // expert's gate/up rows follow the logits publish, its down rows its
    // activations' publish)
    plan_router(li + 1);
    issue_router();
    stamp0(li, 11);
  }
  if (a.clocks && b == 0) {   // stamps were kept in LDS so taking them adds no memory traffic
    block_sync_lds();
    for (int i = tid; i < L * kStackClockEvents; i += kThreads) a.clocks[i] = clk[i];
  }
  if (a.bclocks) {
    block_sync_lds();
    for (int i = tid; i < L * kBlockClockEvents; i += kThreads)
      a.bclocks[(int64_t)b * L * kBlockClockEvents + i] = bclk[i];
  }
}

// The workgroups wait on each other's words, so the whole grid must be
// resident at once: one workgroup per compute unit, which the occupancy of
// the instantiation at this LDS size must allow (checked once per
// instantiation and size).  The launch is an ordinary one (capturable in a
// graph); the per-workgroup launch counts replace any per-launch reset.
template <int BITS, int CPLR, int CPLG, int RPWG, int LPRD, int CPLD, int STEPSD, int HW, int JIT = 0>
hipError_t launch_t(const StackArgs& a, int nb, size_t lds, hipStream_t stream) {
  auto* kern = &stack_kernel<BITS, CPLR, CPLG, RPWG, LPRD, CPLD, STEPSD, HW, JIT>;
  static thread_local size_t checked_lds = 0;
  if (checked_lds != lds) {
    int per_cu = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreads, lds);
    if (e != hipSuccess) return e;
    if (per_cu < 1 || nb > device_cus()) return hipErrorCooperativeLaunchTooLarge;
    checked_lds = lds;
  }
  StackArgs args = a;
  void* params[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(kern), dim3(nb), dim3(kThreads), params, lds, stream);
}

}  // namespace

int device_cus() {
  static int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return cus;
  }();
  return n;
}

namespace {

// Does instantiation <BITS, CPLR, CPLG, RPWG, LPRD, CPLD, STEPSD, HW> cover
// this shape on nb blocks?
struct Geometry {
  int nb, rw, H, I, E, S, K, KS, bits;
  bool fits(int BITS, int CPLR, int CPLG, int RPWG, int LPRD, int CPLD, int STEPSD, int HW) const {
    if (bits != BITS) return false;
    // expert blobs are addressed with 32-bit byte offsets
    if ((int64_t)3 * H * I * BITS / 8 + (int64_t)3 * (H / 64) * I * 4 >= (int64_t{1} << 31)) return false;
    const int PC = BITS == 3 ? 64 : 128 / BITS;   // values per 16-byte unit (of the low plane at 3 bits)
    const int PW = BITS == 4 ? 8 : 16;            // values per staged word
    if (rw > CPLR) return false;
    if (H / PC > 64 * CPLG) return false;
    const int RG = gu_rows_max(I, nb), RD = (H + nb - 1) / nb;
    if (S > 0 && 2 * RG > kWaves) return false;              // shared rows: register slot 0
    if (K * 2 * RG > kWaves * (RPWG - 1)) return false;      // routed rows: slots 1 ..
    const int nchd = I / PC;
    if (nchd > LPRD * CPLD) return false;
    if (KS * (I / PW) > kThreads) return false;    // one activation word per thread
    if (BITS == 3 && (H % 128 != 0 || I % 128 != 0)) return false;   // whole high-plane words per row
    if (K > STEPSD) return false;                  // one down step per routed slot
    if (H < nb) return false;                      // every block owns a row of h (hand-off safety)
    if (RD > kWaves * (64 / LPRD)) return false;   // every output row owned by a wave
    if (H > 2 * kThreads * HW) return false;
    if (E + S > kTblPer * kThreads) return false;
    return true;
  }
};

}  // namespace

int stack_barrier_words() { return kBarWords; }

// Geometry check and dispatch.  Returns hipErrorNotSupported (without
// launching) when no persistent instantiation covers the shape; the caller
// then runs the layers one launch sequence at a time.
hipError_t launch_stack_decode(StackArgs& a, hipStream_t stream) {
  const int nb = device_cus();
  if (nb < 1) return hipErrorNoDevice;
  if (nb > kMaxCus) return hipErrorNotSupported;   // one launch-count word per workgroup
  const int KS = a.K + a.S;
  if (a.K < 1 || KS > kMaxKS || a.L > kMaxLayers) return hipErrorNotSupported;
  const int rw_need = (a.E + nb - 1) / nb;
  int rw = 1;
  while (rw < rw_need) rw <<= 1;
  if (rw > kWaves) return hipErrorNotSupported;
  a.router_rows = rw;
  const int PC = a.bits == 3 ? 64 : 128 / a.bits;
  const int RG = gu_rows_max(a.I, nb), RD = (a.H + nb - 1) / nb;
  const size_t lds =
      (size_t)stack_lds_layout(a.H, a.I, a.E, a.S, KS, PC, RG, RD,
                               (a.clocks ? a.L * kStackClockEvents : 0) + (a.bclocks ? a.L * kBlockClockEvents : 0))
          .total;
  if (lds > 96 * 1024) return hipErrorNotSupported;
  const Geometry g{nb, rw, a.H, a.I, a.E, a.S, a.K, KS, a.bits};
  // hidden 4096, intermediate 1024, 512 experts on 256 CUs: 4-bit K+S <= 4,
  // 2-bit and 3-bit K+S <= 5; a small shape for tests; else the per-layer path.
  if (a.jitter) {   // delay-injection instantiations: the 60-layer shape and the small test shape
    if (g.fits(4, 2, 2, 4, 32, 1, 3, 4)) return launch_t<4, 2, 2, 4, 32, 1, 3, 4, 1>(a, nb, lds, stream);
    if (g.fits(4, 1, 1, 2, 64, 1, 3, 1)) return launch_t<4, 1, 1, 2, 64, 1, 3, 1, 1>(a, nb, lds, stream);
    return hipErrorNotSupported;
  }
  if (g.fits(4, 2, 2, 4, 32, 1, 3, 4)) return launch_t<4, 2, 2, 4, 32, 1, 3, 4>(a, nb, lds, stream);
  if (g.fits(2, 2, 1, 5, 32, 1, 4, 4)) return launch_t<2, 2, 1, 5, 32, 1, 4, 4>(a, nb, lds, stream);
  if (g.fits(3, 2, 1, 5, 32, 1, 4, 4)) return launch_t<3, 2, 1, 5, 32, 1, 4, 4>(a, nb, lds, stream);
  if (g.fits(4, 1, 1, 2, 64, 1, 3, 1)) return launch_t<4, 1, 1, 2, 64, 1, 3, 1>(a, nb, lds, stream);
  return hipErrorNotSupported;
}

}  // namespace moeq
