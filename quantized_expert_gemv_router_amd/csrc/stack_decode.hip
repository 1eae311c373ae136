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
// Grid: one workgroup of 8 waves per CU, all co-resident (cooperative
// launch).  Three all-to-all steps per layer, each a handoff of tagged
// words (payload + layer tag in one 64-bit word, polled by the readers; no
// grid barrier or fence between the phases):
//   h:       each block publishes its rows of h_{l+1}; every block polls all
//            of h, takes sum(h^2), max|h| and its router rows' partial dot
//            products from the polled registers, and after one block
//            barrier publishes its logits
//   logits:  every block polls all E logits and selects top-K itself
//            (threshold on the keys' high words, every wave keeps its own
//            copy of the selection), then streams its gate/up rows
//   a:       each block publishes silu(g)*u for its gate/up rows; every block
//            polls all activations of the K + S slots, then its down rows
//            and the combine with the residual.
// Loads are issued as early as their addresses are known and their data
// does not compete with loads on the critical path: the router and
// shared-expert pointers of every layer are cached in LDS at start; the
// next layer's router rows and shared-expert gate/up rows are requested
// right after h is published, and the shared expert's gate/up is computed
// while the logits travel; the down rows are requested once the gate/up
// rows are consumed.  A poll's loads complete after every load the wave
// issued before them (the vector memory counter is in order), which is why
// nothing large is requested just before a poll that is on the critical
// path.  Each block owns fixed rows of every matrix:
//   router rows  e = b + NB*k (every thread takes the columns of the h
//   values it polls);
//   gate/up rows r = b + NB*i of every selected expert (a = silu(g)*u is
//   formed locally);
//   down rows    r = b + NB*i of every selected expert (the combine is a
//   per-row sum in slot order, no atomics).
// Every wait is bounded: on time-out a block sets the status word and an
// abort flag, and every block leaves the kernel.
#include "moeq_device.hpp"
#include "moeq_internal.hpp"
#include "topk.hpp"

namespace moeq {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kGroups = 8;                 // barrier tree: groups of blocks
constexpr int kBarWords = 32 * (kGroups + 2);
constexpr int kSpinLimit = 1 << 18;        // polls before a barrier gives up
constexpr int kMaxKS = 8;                  // selected + shared experts per layer
constexpr int kActSums = 4;                // per staged activation chunk: X, 1024 X', undo, pad
constexpr int kMaxLayers = 128;            // per persistent launch
constexpr int kTblPer = 8;                 // pointer-table entries per thread (E + S <= 4096)
static_assert(kWaves * MOEQ_MAX_TOPK <= 64 * 2, "top-K merge holds two candidates per lane");
static_assert(2 * kWaves >= MOEQ_MAX_TOPK, "threshold top-K: at most two samples per wave");

// ------------------------------------------------------------------ barrier
struct GridBarrier {
  uint32_t* base;       // [0]: top counter, [32*(1+g)]: group g, [32*(1+kGroups)]: abort
  int group, gsize, ngroups;
  uint32_t epoch;

  // Thread 0 arrives for the whole block.  The caller has drained the
  // block's global stores and passed a block barrier after that.
  __device__ __forceinline__ void arrive() {
    if (threadIdx.x == 0) {
      ++epoch;
      uint32_t* gc = base + 32 * (1 + group);
      const uint32_t old = atomic_add_agent(gc, 1u);
      if (old == epoch * (uint32_t)gsize - 1u) atomic_add_agent(base, 1u);
    }
  }

  // Whole block: waits until every block has arrived.  Global loads issued
  // between arrive() and wait() stay in flight across the wait.  Returns
  // false if the grid is aborting.
  __device__ __forceinline__ bool wait(int32_t* status, int* flag) {
    if (threadIdx.x == 0) {
      const uint32_t* top = base;
      uint32_t* abort = base + 32 * (1 + kGroups);
      const uint32_t target = epoch * (uint32_t)ngroups;
      int ok = 1;
      for (int spins = 0; ld_agent(top) < target; ++spins) {
        if ((spins & 63) == 63 && ld_agent(abort) != 0u) { ok = 0; break; }
        if (spins > kSpinLimit) {
          set_status(status, kStatusTimeout);
          st_agent(abort, 1u);
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      *flag = ok;
    }
    block_sync_lds();
    return *flag != 0;
  }

  // Whole block: drain, arrive, wait.
  __device__ __forceinline__ bool sync(int32_t* status, int* flag) {
    drain_memory();
    __syncthreads();
    arrive();
    return wait(status, flag);
  }
};

// ------------------------------------------------------------ tagged words
// A value handed from one block to the others travels as one 64-bit word:
// the payload in the low half, the tag of the layer that wrote it in the
// high half.  Readers poll the word until the tag they expect shows up, so
// the word is its own flag and no fence or grid barrier sits between the
// writer and its readers.  Each word has one writing block for the whole
// launch, and a block writes layer l+1's value only after every block has
// read layer l's (each layer's three handoffs form a chain), so a reader
// never sees a tag newer than the one it waits for.
__device__ __forceinline__ void put_tagged(uint64_t* p, uint32_t payload, uint32_t tag) {
  st_agent(p, ((uint64_t)tag << 32) | payload);
}

// Polls the words base[idx(i)] for the bits i set in `valid` until each
// carries `tag`; payloads land in out[i].  Bounded: gives up (and raises
// the grid's abort flag) after kSpinLimit polls, or when another block has
// raised it.
template <int N, typename Idx>
__device__ __forceinline__ bool take_tagged(const uint64_t* base, Idx idx, uint32_t valid, uint32_t tag,
                                            uint32_t (&out)[N], uint32_t* abort, int32_t* status) {
  uint32_t pending = valid;
  for (int spins = 0;; ++spins) {
    uint64_t v[N];
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = ((pending >> i) & 1) ? ld_agent(base + idx(i)) : 0ull;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (((pending >> i) & 1) && (uint32_t)(v[i] >> 32) == tag) {
        out[i] = (uint32_t)v[i];
        pending &= ~(1u << i);
      }
    }
    if (pending == 0) return true;
    if ((spins & 15) == 15 && ld_agent(abort) != 0u) return false;
    if (spins > kSpinLimit) {
      set_status(status, kStatusTimeout);
      st_agent(abort, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// ------------------------------------------------------------------ layout
struct StackLds {
  int hs, xp, xs, ap, as, gres, lg, tbl, clk, total;
};

__host__ __device__ inline int al16(int v) { return (v + 15) & ~15; }

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

template <int BITS, int CPLR, int CPLG, int RPWG, int LPRD, int CPLD, int STEPSD, int HW>
__global__ __launch_bounds__(kThreads) void stack_kernel(StackArgs a) {
  constexpr int PC = Pack<BITS>::kPerChunk, PW = Pack<BITS>::kPerWord;
  constexpr int RPSD = 64 / LPRD;          // down rows per wave step
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ double rpart[CPLR * kWaves];
  __shared__ double ssum[kWaves];
  __shared__ float hmax[kWaves];
  __shared__ int sel[MOEQ_MAX_TOPK];
  __shared__ double selv[MOEQ_MAX_TOPK];
  __shared__ int64_t candk[kWaves * 64];
  __shared__ int candi[kWaves * 64];
  __shared__ int sample_k[2 * kWaves];
  __shared__ int cand_cnt[kWaves];
  __shared__ int wsel[kWaves][MOEQ_MAX_TOPK];   // each wave's copy of the selection
  __shared__ float selw[MOEQ_MAX_TOPK];
  __shared__ const uint8_t* eblob[kMaxKS];
  __shared__ const uint16_t* rtr[kMaxLayers];
  __shared__ const uint8_t* shp[kMaxLayers];
  __shared__ float undo_x;
  __shared__ int bar_flag;
  __shared__ int fail_flag;

  int tid = threadIdx.x, lane = tid & 63;   // re-derived opaquely each layer, as b
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NB = gridDim.x;
  int b = blockIdx.x;   // re-derived opaquely each layer (see the layer loop)
  const int H = a.H, I = a.I, E = a.E, K = a.K, S = a.S, KS = K + S, L = a.L;
  const int nchG = H / PC, nchD = I / PC;
  const int RG = (I + NB - 1) / NB, RD = (H + NB - 1) / NB;

  const StackLds LL = stack_lds_layout(H, I, E, S, KS, PC, RG, RD, a.clocks ? L * kStackClockEvents : 0);
  float* hs = reinterpret_cast<float*>(smem + LL.hs);               // [H]
  uint32_t* xp = reinterpret_cast<uint32_t*>(smem + LL.xp);         // [H/2]
  float* xs = reinterpret_cast<float*>(smem + LL.xs);               // [H/PC][kChunkSums]
  uint32_t* ap = reinterpret_cast<uint32_t*>(smem + LL.ap);         // [KS][I/2]
  float* as = reinterpret_cast<float*>(smem + LL.as);               // [KS][I/PC][kActSums]
  float* gres = reinterpret_cast<float*>(smem + LL.gres);           // [KS][2][RG]
  double* lg = reinterpret_cast<double*>(smem + LL.lg);             // [E]
  const uint8_t** tbl = reinterpret_cast<const uint8_t**>(smem + LL.tbl);  // [E + S], this layer
  int64_t* clk = reinterpret_cast<int64_t*>(smem + LL.clk);         // [L][kStackClockEvents] if timed

  GridBarrier bar;
  bar.base = a.bar;
  bar.ngroups = min(kGroups, NB);
  bar.group = b % bar.ngroups;
  bar.gsize = (NB - bar.group + bar.ngroups - 1) / bar.ngroups;
  bar.epoch = 0;

  // router: RW (<= CPLR) rows per block, rows b + NB*k; each thread takes
  // the columns of the h values it polls (2p, 2p+1 for p = tid + i*kThreads)
  const int RW = a.router_rows;
  const int tbl_n = E + S;

  uint32_t wr[CPLR][HW];
  u32x4 qg[RPWG][CPLG];
  uint32_t sg[RPWG][CPLG];
  u32x4 qd[STEPSD][CPLD];
  uint32_t sd[STEPSD][CPLD];
  const uint8_t* tnext[kTblPer];   // this layer's pointer-table row, in flight to LDS

  // gate/up rows: task t = m * kWaves + wave, the shared experts' rows first,
  // then the routed ones, so every wave takes part in both phases
  auto gu_task = [&](int m, int& j, int& sec, int& row) -> bool {
    const int t = m * kWaves + wave, nsh = S * 2 * RG;
    const bool shared = t < nsh;
    const int u = shared ? t : t - nsh;
    j = (shared ? K : 0) + u / (2 * RG);
    const int tj = u % (2 * RG);
    sec = tj / RG;
    row = b + NB * (tj % RG);
    return (shared ? j < KS : j < K) && row < I;
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
      const int r = b + NB * k;
      const bool have = k < RW && r < E;
      rplan[k] = make_rsrc(base + (int64_t)(have ? r : 0) * H, have ? (uint32_t)H * 2u : 0u);
    }
  };
  auto issue_router = [&]() {
#pragma unroll
    for (int k = 0; k < CPLR; ++k)
#pragma unroll
      for (int i = 0; i < HW; ++i) wr[k][i] = load_rsrc_b32(rplan[k], (uint32_t)(tid + i * kThreads) * 4u);
  };
  // gate/up rows of the tasks whose slot is in [jlo, jhi); gu_task is
  // uniform over a wave, so each row is one scalar buffer resource
  rsrc_t gq[RPWG];               // the task's expert blob, or an empty range: no task
  uint32_t gqo[RPWG], gso[RPWG]; // byte offsets of its quantized row and scale/bias words
  bool ghave[RPWG];
  auto plan_gu = [&](int jlo, int jhi) {
    const uint32_t row_bytes = (uint32_t)H * BITS / 8;
    const uint32_t gpr = H / 64;
    const uint32_t sb_off = 3u * (uint32_t)H * I * BITS / 8;
    const uint32_t blob_bytes = sb_off + 3u * (uint32_t)(H / 64) * I * 4u;
#pragma unroll
    for (int m = 0; m < RPWG; ++m) {
      int j, sec, row;
      const bool ok = gu_task(m, j, sec, row);
      ghave[m] = ok && j >= jlo && j < jhi;
      // routed slots: this wave's own copy of the selection; the shared one
      // from eblob.  A missing expert (null) loads nothing.
      const int jj = ghave[m] ? j : K;
      const int e = jj < K ? wsel[wave][jj] : 0;
      const uint8_t* blob = uniform_ptr(jj < K ? ((unsigned)e < (unsigned)E ? tbl[e] : nullptr)
                                               : eblob[min(jj, KS - 1)]);
      const uint32_t r = ghave[m] ? (uint32_t)(sec * I + row) : 0u;   // row of [gate; up]
      gq[m] = make_rsrc(blob, ghave[m] && blob != nullptr ? blob_bytes : 0u);
      gqo[m] = r * row_bytes;
      gso[m] = sb_off + r * gpr * 4u;
    }
  };
  // chunk-major: the dots take one staged x chunk at a time against every
  // row of the wave, so each chunk is read from LDS once
  auto issue_gu = [&]() {
#pragma unroll
    for (int c = 0; c < CPLG; ++c) {
      const int cc = min(lane + 64 * c, nchG - 1);   // past the row: the dots skip it
#pragma unroll
      for (int m = 0; m < RPWG; ++m) {
        qg[m][c] = load_rsrc_b128(gq[m], gqo[m] + (uint32_t)cc * 16u);
        sg[m][c] = load_rsrc_b32(gq[m], gso[m] + (uint32_t)(cc * PC / 64) * 4u);
      }
    }
    issue_fence();
  };
  auto gu_dots = [&](int jlo, int jhi) {
    bool live[RPWG];
    bool any = false;
#pragma unroll
    for (int m = 0; m < RPWG; ++m) {
      int j, sec, row;
      live[m] = gu_task(m, j, sec, row) && j >= jlo && j < jhi;
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
        if (live[m] && cc < nchG) part[m] += chunk_affine(chunk_dot<BITS>(qg[m][c], x), sg[m][c], xsum);
    }
    const float ux = undo_x;
#pragma unroll
    for (int m = 0; m < RPWG; ++m) {
      if (!live[m]) continue;
      int j, sec, row;
      gu_task(m, j, sec, row);
      const float v = wave_sum_dpp(part[m]) * ux;
      if (lane == 0) gres[(j * 2 + sec) * RG + (row - b) / NB] = v;
    }
  };
  // down rows: a wave owns RPSD of the block's output rows (LPRD lanes
  // each), for every slot: step s is slot s, so the combine of a row stays
  // in the wave
  rsrc_t dsrc[STEPSD];       // slot s's expert blob, or an empty range
  auto down_row = [&](int s, int& j, int& row) {
    j = s;
    const int i = wave * RPSD + lane / LPRD;
    row = i < RD ? b + NB * i : H;   // H: no row
  };
  auto plan_down = [&]() {
    const uint32_t blob_bytes = 3u * (uint32_t)H * I * BITS / 8 + 3u * (uint32_t)(H / 64) * I * 4u;
#pragma unroll
    for (int s = 0; s < STEPSD; ++s) {
      const uint8_t* blob = s < KS ? uniform_ptr(eblob[s]) : nullptr;
      dsrc[s] = make_rsrc(blob, blob != nullptr ? blob_bytes : 0u);
    }
  };
  auto issue_down = [&]() {
    const uint32_t row_bytes = (uint32_t)I * BITS / 8;
    const uint32_t gpr = I / 64;
    const uint32_t q_off = 2u * (uint32_t)H * I * BITS / 8;
    const uint32_t sb_off = 3u * (uint32_t)H * I * BITS / 8 + 2u * (uint32_t)H * (I / 64) * 4u;
    const int sub = lane % LPRD;
#pragma unroll
    for (int s = 0; s < STEPSD; ++s) {
      int j, row;
      down_row(s, j, row);
      if (row >= H) row = 0;   // padding lane: re-reads a valid row, skipped by the dots
#pragma unroll
      for (int c = 0; c < CPLD; ++c) {
        const int cc = min(sub + LPRD * c, nchD - 1);
        qd[s][c] = load_rsrc_b128(dsrc[s], q_off + (uint32_t)row * row_bytes + (uint32_t)cc * 16u);
        sd[s][c] = load_rsrc_b32(dsrc[s], sb_off + ((uint32_t)row * gpr + (uint32_t)(cc * PC / 64)) * 4u);
      }
    }
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

  // prologue: router and shared-expert pointers of every layer, first rows
  for (int li = tid; li < L; li += kThreads) {
    rtr[li] = a.routers[a.layer0 + li];
    shp[li] = S > 0 ? static_cast<const uint8_t*>(a.blobs[(int64_t)(a.layer0 + li) * tbl_n + E]) : nullptr;
  }
  if (tid == 0) fail_flag = 0;
  // this block's tagged words start at tag 0 (no layer's); one grid
  // barrier puts every clear before any layer's write
  for (int j = tid; j < RW; j += kThreads) {
    const int r = b + NB * j;
    if (r < E) { st_agent(a.lwords + 2 * r, uint64_t{0}); st_agent(a.lwords + 2 * r + 1, uint64_t{0}); }
  }
  for (int t = tid; t < KS * RG; t += kThreads) {
    const int j = t / RG, row = b + NB * (t - j * RG);
    if (row < I) st_agent(a.awords + (int64_t)j * I + row, uint64_t{0});
  }
  for (int i = tid; i < RD; i += kThreads) {
    const int row = b + NB * i;
    if (row < H) st_agent(a.hwords + row, uint64_t{0});
  }
  if (tid < S) eblob[K + tid] = shp[0];
  if (!bar.sync(a.status, &bar_flag)) return;
  block_sync_lds();
  plan_router(0);
  plan_gu(K, KS);
  issue_router();
  issue_gu();
  uint32_t* const abort_word = a.bar + 32 * (1 + kGroups);
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
    }
    stamp(li, 0);
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
        ok = take_tagged<2 * HW>(a.hwords, [&](int i) { return 2 * (tid + (i >> 1) * kThreads) + (i & 1); },
                                 valid, (uint32_t)li, hw, abort_word, a.status);
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
    __syncthreads();
    stamp(li, 1);
    double ss = 0.0;
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) { ss += ssum[i]; mx = fmaxf(mx, hmax[i]); }
    const double inv = 1.0 / sqrt(ss / (double)H + 1e-6);
    const uint32_t tag = (uint32_t)li + 1u;
    if (tid < RW && b + NB * tid < E) {   // logits of this block's router rows
      double d = 0.0;
      for (int w = 0; w < kWaves; ++w) d += rpart[tid * kWaves + w];
      const int r = b + NB * tid;
      const uint64_t bits = (uint64_t)__double_as_longlong(d * inv);
      put_tagged(a.lwords + 2 * r, (uint32_t)bits, tag);
      put_tagged(a.lwords + 2 * r + 1, (uint32_t)(bits >> 32), tag);
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
    __syncthreads();
    stamp(li, 2);
    gu_dots(K, KS);                 // the shared expert's rows are already here
    stamp(li, 3);
    stamp(li, 4);

    // ------------------------------------------------------------ phase G
    // this layer's pointer-table row lands while the logits are polled
    load_tbl_row(a.layer0 + li);
    int64_t key = kNoKey;   // this thread's logit (E <= kThreads)
    for (int e0 = 0; e0 < E; e0 += kThreads) {   // one logit (two words) per thread per pass
      const int e = e0 + tid;
      uint32_t w[2] = {0u, 0u};
      const bool ok = take_tagged<2>(a.lwords + 2 * e, [](int i) { return i; }, e < E ? 3u : 0u, tag, w,
                                     abort_word, a.status);
      if (e < E) {
        const double v = __longlong_as_double((long long)(((uint64_t)w[1] << 32) | w[0]));
        lg[e] = v;
        key = order_key(v);
      }
      if (E <= kThreads) topk_samples<kWaves>(key, K, sample_k);
      if (block_failed(ok)) return;
    }
    store_tbl_row();
    stamp0(li, 12);
    // top-K: every wave ends with its own copy of the selection, so the
    // gate/up rows are requested without another block barrier
    bool fast = false;
    if (E <= kThreads) {
      topk_candidates<kWaves>(key, tid, K, sample_k, candk, candi, cand_cnt);
      __syncthreads();
      fast = topk_select<kWaves>(K, candk, candi, cand_cnt, [&](int r, int win) { wsel[wave][r] = win; });
    } else {
      __syncthreads();
    }
    if (!fast) {   // block-uniform
      if (E <= kThreads) block_topk_keys<kWaves, 1, 2>(lg, E, K, candk, candi, sel, selv);
      else block_topk_keys<kWaves, kTblPer, 2>(lg, E, K, candk, candi, sel, selv);
      if (lane < K) wsel[wave][lane] = sel[lane];
    }
    stamp0(li, 14);
    plan_gu(0, K);                   // routed gate/up rows
    issue_gu();
    stamp0(li, 5);
    // while they arrive: wave 0 takes the softmax weights and the blob
    // pointers the down rows use (read after the next block barrier)
    if (wave == 0) {
      if (lane < K) selv[lane] = (unsigned)wsel[0][lane] < (unsigned)E ? lg[wsel[0][lane]] : -INFINITY;
      const float w = a.no_renorm ? wave_softmax_weight(lg, E, K, selv, true)
                                  : wave_softmax_selected(selv, K);
      if (lane < K) {
        selw[lane] = w;
        const int e = wsel[0][lane];
        const uint8_t* bp = (unsigned)e < (unsigned)E ? tbl[e] : nullptr;
        eblob[lane] = bp;
        if (bp == nullptr) set_status(a.status, kStatusBadExpert);
        if (b == 0 && a.topk_trace) a.topk_trace[(int64_t)li * K + lane] = e;
      }
    }
    stamp0(li, 15);
    gu_dots(0, K);
    stamp0(li, 13);
    __syncthreads();
    stamp(li, 6);
    plan_down();                     // every slot's down rows (eblob is complete now)
    for (int t = tid; t < KS * RG; t += kThreads) {
      const int j = t / RG, i = t - j * RG, row = b + NB * i;
      if (row < I) {
        const float g = gres[(j * 2) * RG + i], u = gres[(j * 2 + 1) * RG + i];
        put_tagged(a.awords + (int64_t)j * I + row, __float_as_uint(g / (1.0f + __expf(-g)) * u), tag);
      }
    }
    // down rows of every slot, in flight while the activations arrive (not
    // earlier: they would share the memory system with the gate/up rows
    // every block is waiting for)
    issue_down();
    stamp0(li, 7);
    stamp(li, 8);

    // ------------------------------------------------------------ phase D
    // activations: one packed word of one slot per thread, staged with a
    // power-of-two scale per 16-byte chunk (the four threads of a chunk
    // agree on it with two lane shuffles), so staging needs no block-wide
    // maximum; the one block barrier below also settles a failed poll
    {
      const int nwa = I / PW;
      const int total = KS * nwa;
      bool got_all = true;
      for (int t0 = 0; t0 < total; t0 += kThreads) {
        const int t = t0 + tid;
        const bool ok = t < total;
        const int m = ok ? t / nwa : 0, w = ok ? t - m * nwa : 0;
        float v[PW];
        uint32_t raw[PW];
#pragma unroll
        for (int j = 0; j < PW; ++j) raw[j] = 0u;
        const uint64_t* src = a.awords + (int64_t)m * I + (int64_t)w * PW;
        const bool got = take_tagged<PW>(src, [](int j) { return j; }, ok ? (uint32_t)((1ull << PW) - 1) : 0u,
                                         tag, raw, abort_word, a.status);
        got_all = got_all && got;
        stamp0(li, 16);
        float lm = 0.0f;
#pragma unroll
        for (int j = 0; j < PW; ++j) {
          v[j] = __uint_as_float(raw[j]);
          lm = fmaxf(lm, fabsf(v[j]));
        }
        lm = fmaxf(lm, __shfl_xor(lm, 1, 64));
        lm = fmaxf(lm, __shfl_xor(lm, 2, 64));
        const float p = pow2_stage_factor(lm);
        float2 s = make_float2(0.0f, 0.0f);
        if (ok) s = stage_word<BITS>(v, p, ap + (int64_t)m * (I / 2), w, nchD);
        s = quad_sum(s);
        if (ok && (tid & 3) == 0)
          *reinterpret_cast<float4*>(as + kActSums * (m * nchD + (w >> 2))) = make_float4(s.x, s.y, 1.0f / p, 0.0f);
      }
      if (block_failed(got_all)) return;
      stamp0(li, 17);
    }
    stamp(li, 9);
    {
      // down rows of every slot and the combine, in registers: lane LPRD-1
      // of each row group ends with the row's h
      const int sub = lane % LPRD;
      const int i = wave * RPSD + lane / LPRD;
      const int row = b + NB * i;
      const bool ok = i < RD && row < H;
      float acc = ok ? hs[row] : 0.0f;
#pragma unroll
      for (int s = 0; s < STEPSD; ++s) {
        if (s >= KS) break;
        float part = 0.0f;
#pragma unroll
        for (int c = 0; c < CPLD; ++c) {
          const int cc = min(sub + LPRD * c, nchD - 1);
          const XChunk<BITS> x = load_xchunk<BITS>(ap + (int64_t)s * (I / 2), cc, nchD);
          const float4 xsm = *reinterpret_cast<const float4*>(as + kActSums * (s * nchD + cc));
          if (ok && sub + LPRD * c < nchD)
            part += chunk_affine(chunk_dot<BITS>(qd[s][c], x), sd[s][c], make_float2(xsm.x, xsm.y)) * xsm.z;
        }
        const float d = group_sum_dpp<LPRD>(part);
        acc = fmaf(s < K ? selw[s] : 1.0f, d, acc);   // slot order: routed, then shared
      }
      stamp0(li, 18);
      if (ok && sub == LPRD - 1) {
        if (a.h_trace) a.h_trace[(int64_t)li * H + row] = hs[row];
        if (li + 1 == L) a.h[row] = acc;   // complete when the launch ends
        else put_tagged(a.hwords + row, __float_as_uint(acc), tag);
      }
    }
    stamp(li, 10);
    if (li + 1 == L) break;
    // next layer: router rows, shared-expert gate/up rows, pointer-table row,
    // in flight while h arrives
    if (S > 0 && tid == 0) eblob[K] = shp[li + 1];   // at most one shared expert
    block_sync_lds();
    plan_router(li + 1);
    plan_gu(K, KS);
    issue_router();
    issue_gu();
    stamp0(li, 11);
  }
  if (a.clocks && b == 0) {   // stamps were kept in LDS so taking them adds no memory traffic
    block_sync_lds();
    for (int i = tid; i < L * kStackClockEvents; i += kThreads) a.clocks[i] = clk[i];
  }
}

__global__ void reset_barrier_kernel(uint32_t* bar) {
  for (int i = threadIdx.x; i < kBarWords; i += blockDim.x) bar[i] = 0u;
}

template <int BITS, int CPLR, int CPLG, int RPWG, int LPRD, int CPLD, int STEPSD, int HW>
hipError_t launch_t(const StackArgs& a, int nb, size_t lds, hipStream_t stream) {
  hipLaunchKernelGGL(reset_barrier_kernel, dim3(1), dim3(256), 0, stream, a.bar);
  StackArgs args = a;
  void* params[] = {&args};
  return hipLaunchCooperativeKernel(
      reinterpret_cast<const void*>(&stack_kernel<BITS, CPLR, CPLG, RPWG, LPRD, CPLD, STEPSD, HW>),
      dim3(nb), dim3(kThreads), params, (unsigned int)lds, stream);
}

int device_cus() {
  static int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return cus;
  }();
  return n;
}

// Does instantiation <BITS, CPLR, CPLG, RPWG, LPRD, CPLD, STEPSD, HW> cover
// this shape on nb blocks?
struct Geometry {
  int nb, rw, H, I, E, S, KS, bits;
  bool fits(int BITS, int CPLR, int CPLG, int RPWG, int LPRD, int CPLD, int STEPSD, int HW) const {
    if (bits != BITS) return false;
    // expert blobs are addressed with 32-bit byte offsets
    if ((int64_t)3 * H * I * BITS / 8 + (int64_t)3 * (H / 64) * I * 4 >= (int64_t{1} << 31)) return false;
    const int PC = 128 / BITS;
    if (rw > CPLR) return false;
    if (H / PC > 64 * CPLG) return false;
    const int RG = (I + nb - 1) / nb, RD = (H + nb - 1) / nb;
    if (KS * 2 * RG > kWaves * RPWG) return false;
    const int nchd = I / PC;
    if (nchd > LPRD * CPLD) return false;
    if (KS * (I * BITS / 32) > kThreads) return false;   // one activation word per thread
    if (KS > STEPSD) return false;                 // one down step per slot
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
  const int KS = a.K + a.S;
  if (a.K < 1 || KS > kMaxKS || a.L > kMaxLayers) return hipErrorNotSupported;
  const int rw_need = (a.E + nb - 1) / nb;
  int rw = 1;
  while (rw < rw_need) rw <<= 1;
  if (rw > kWaves) return hipErrorNotSupported;
  a.router_rows = rw;
  const int PC = 128 / a.bits;
  const int RG = (a.I + nb - 1) / nb, RD = (a.H + nb - 1) / nb;
  const size_t lds =
      (size_t)stack_lds_layout(a.H, a.I, a.E, a.S, KS, PC, RG, RD, a.clocks ? a.L * kStackClockEvents : 0).total;
  if (lds > 96 * 1024) return hipErrorNotSupported;
  const Geometry g{nb, rw, a.H, a.I, a.E, a.S, KS, a.bits};
  // hidden 4096, intermediate 1024, 512 experts on 256 CUs: 4-bit K+S <= 4,
  // 2-bit K+S <= 5; a small shape for tests; else the per-layer path.
  if (g.fits(4, 2, 2, 4, 32, 1, 4, 4)) return launch_t<4, 2, 2, 4, 32, 1, 4, 4>(a, nb, lds, stream);
  if (g.fits(2, 2, 1, 5, 32, 1, 5, 4)) return launch_t<2, 2, 1, 5, 32, 1, 5, 4>(a, nb, lds, stream);
  if (g.fits(4, 1, 1, 1, 64, 1, 3, 1)) return launch_t<4, 1, 1, 1, 64, 1, 3, 1>(a, nb, lds, stream);
  return hipErrorNotSupported;
}

}  // namespace moeq
