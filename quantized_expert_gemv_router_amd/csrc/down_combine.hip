// SwiGLU, down projection and weighted combine (Flash-MoE,
// fr.news.hada.io, "Shaders de calcul Metal": SwiGLU and MoE combine +
// residual + gate; "Deferred GPU Expert Compute": the combined output stays
// on the GPU for the next layer):
//   a   = silu(g) * u                         per (token, slot)
//   d_i = sum_g ( s[i,g] sum_{r in g} q[i,r] a_r + b[i,g] sum_{r in g} a_r )
//   out[t] = residual[t] + sum_{s<k} w[t,s] d_s + gamma[t] d_shared
// summed in slot order.  a is built from gate_up while it is staged into
// LDS as fp16 pairs (per-vector power-of-two rescale).
//
// Two launch shapes, same arithmetic per (token, slot, row):
//  - fused (every (token, slot) pair fits one workgroup's LDS, e.g. one
//    decode token): one workgroup per block of 16 output rows streams those
//    rows of every selected expert and sums them in registers, no atomics;
//  - grouped (multi-token batches): one workgroup per (expert item, block of
//    32 rows) writes per-slot outputs to the workspace with write-through
//    stores; the last workgroup to finish a row block (relaxed arrival
//    counter) sums them per token in slot order.
// Either way a token's output does not depend on what else is in the batch.
#include "grouping.hpp"
#include "moeq_internal.hpp"
#include "staging.hpp"

namespace moeq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kGroupedRows = 32;   // rows per workgroup, grouped shape
constexpr int kFusedRows = 16;     // rows per workgroup, fused shape
constexpr int kTokensPerStage = 4; // grouped shape
constexpr int kFusedPairs = 8;     // fused shape: max (token, slot) pairs

__device__ __forceinline__ float residual_at(const DownArgs& a, int64_t i) {
  return a.res_f32 ? static_cast<const float*>(a.residual)[i]
                   : __uint_as_float((uint32_t) static_cast<const uint16_t*>(a.residual)[i] << 16);
}

// Rows handled by one lane group: LPR lanes per row, RPS = 64/LPR rows per
// step, STEPS steps cover ROWS rows of a wave.
template <int BITS, int LPR, int CPL, int ROWS>
struct DownTile {
  static constexpr int PC = Pack<BITS>::kPerChunk;
  static constexpr int RPS = 64 / LPR;
  static constexpr int STEPS = (ROWS + RPS - 1) / RPS;
  u32x4 q[STEPS][CPL];
  uint32_t sbw[STEPS][CPL];

  __device__ __forceinline__ void load(const uint8_t* blob, int H, int I, int wrow0, int lane) {
    const int64_t qoff = 2 * (int64_t)H * I * BITS / 8;                                // down.q
    const int64_t row_bytes = (int64_t)I * BITS / 8;
    const uint32_t* sb = reinterpret_cast<const uint32_t*>(
        blob + 3 * (int64_t)H * I * BITS / 8 + 2 * (int64_t)H * I / 64 * 4);          // down.sb
    const int gpr = I / 64, nch = I / PC;
    const int sub = lane % LPR, rsub = lane / LPR;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const int rr = s * RPS + rsub, r = wrow0 + rr;
      const bool row_ok = rr < ROWS && r < H && blob != nullptr;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int cc = sub + LPR * c;
        if (row_ok && cc < nch) {
          q[s][c] = load_stream(reinterpret_cast<const u32x4*>(blob + qoff + r * row_bytes) + cc);
          sbw[s][c] = load_stream(sb + (int64_t)r * gpr + (cc * PC) / 64);
        } else {
          q[s][c] = u32x4{0u, 0u, 0u, 0u};
          sbw[s][c] = 0u;
        }
      }
    }
  }

  // d for step s against one staged vector; valid in lane LPR - 1 of the row group.
  __device__ __forceinline__ float dot(int s, const uint32_t* xp, const float* xs, float undo,
                                       int I, int lane) const {
    const int sub = lane % LPR, nch = I / PC;
    float part = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int cc = sub + LPR * c;
      if (cc < nch) part += chunk_affine(chunk_dot<BITS>(q[s][c], xp, cc, nch), sbw[s][c], xs + kChunkSums * cc);
    }
    return group_sum_dpp<LPR>(part) * undo;
  }
};

// ------------------------------------------------------------ grouped shape
template <int BITS, int LPR, int CPL, int WMAX>
__global__ __launch_bounds__(kThreads) void down_grouped_kernel(DownArgs a, int n_rb, int list_words) {
  extern __shared__ __align__(16) uint32_t smem[];
  __shared__ GroupLds g;
  __shared__ float red[2 * kTokensPerStage * kWaves];
  __shared__ float undo[kTokensPerStage];
  __shared__ int is_last;
  constexpr int ROWS = kGroupedRows / kWaves;
  using Tile = DownTile<BITS, LPR, CPL, ROWS>;
  const int item = blockIdx.x / n_rb, rb = blockIdx.x - item * n_rb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, I = a.I, KS = a.k + a.S;
  const int nch = I / Tile::PC;
  uint32_t* pairs = smem;
  float* xsum = reinterpret_cast<float*>(pairs + kTokensPerStage * (I / 2));
  uint32_t* list = reinterpret_cast<uint32_t*>(xsum + kTokensPerStage * kChunkSums * nch);
  int* ids = reinterpret_cast<int*>(list + list_words);
  const uint8_t** ptrs = reinterpret_cast<const uint8_t**>(ids + list_words);

  group_item(item, a.topk_idx, a.blobs, a.T, a.k, a.E, a.S, g, list, ids, ptrs, a.status);
  if (!g.in_range) return;   // no item for this workgroup: not counted
  const int n_items = g.n_distinct + a.S;
  if (g.expert >= 0) {
    const int wrow0 = rb * kGroupedRows + wave * ROWS;
    Tile tile;
    tile.load(g.blob, H, I, wrow0, lane);
    for (int m0 = 0; m0 < g.count; m0 += kTokensPerStage) {
      const int nv = min(kTokensPerStage, g.count - m0);
      auto loader = [&](int m, int64_t o, float* v) {
        const uint32_t e = list[m0 + m];
        const int t = (int)(e >> 8), slot = (int)(e & 255u);
        load_swiglu<Pack<BITS>::kPerWord>(a.gate_up + ((int64_t)t * KS + slot) * 2 * I, I, o, v);
      };
      stage_batch<BITS, WMAX, kTokensPerStage>(nv, I, loader, false, pairs, xsum, undo, red);
      const int sub = lane % LPR, rsub = lane / LPR;
#pragma unroll
      for (int s = 0; s < Tile::STEPS; ++s) {
        const int rr = s * Tile::RPS + rsub, r = wrow0 + rr;
        const bool row_ok = rr < ROWS && r < H;
        for (int m = 0; m < nv; ++m) {
          const float d = tile.dot(s, pairs + (int64_t)m * (I / 2), xsum + (int64_t)m * kChunkSums * nch, undo[m], I,
                                   lane);
          if (sub == LPR - 1 && row_ok) {
            const uint32_t e = list[m0 + m];
            const int t = (int)(e >> 8), slot = (int)(e & 255u);
            st_agent(a.dbuf + ((int64_t)t * KS + slot) * H + r, d);
          }
        }
      }
      __syncthreads();
    }
  }

  // arrival; the last of the row block's n_items workgroups combines
  drain_memory();
  __syncthreads();
  if (tid == 0) is_last = atomic_add_agent(a.rb_counters + rb, 1u) == (uint32_t)(n_items - 1);
  __syncthreads();
  if (!is_last) return;
  if (tid == 0) st_agent(a.rb_counters + rb, 0u);
  const int rows = min(kGroupedRows, H - rb * kGroupedRows);
  for (int idx = tid; idx < a.T * rows; idx += blockDim.x) {
    const int t = idx / rows, r = rb * kGroupedRows + (idx - t * rows);
    // all of this token's per-slot outputs are requested before the sum
    float dv[MOEQ_MAX_TOPK + 1], wv[MOEQ_MAX_TOPK + 1];
#pragma unroll
    for (int s = 0; s < MOEQ_MAX_TOPK + 1; ++s) {
      dv[s] = 0.0f;
      wv[s] = 0.0f;
      if (s < KS) {
        bool ok = true;
        if (s < a.k) {
          const int e = a.topk_idx[(int64_t)t * a.k + s];
          ok = e >= 0 && e < a.E;
          wv[s] = a.topk_w[(int64_t)t * a.k + s];
        } else {
          wv[s] = a.shared_w ? a.shared_w[t] : 1.0f;
        }
        if (ok) dv[s] = ld_agent(a.dbuf + ((int64_t)t * KS + s) * H + r);
        else wv[s] = 0.0f;
      }
    }
    float acc = residual_at(a, (int64_t)t * H + r);
#pragma unroll
    for (int s = 0; s < MOEQ_MAX_TOPK + 1; ++s)
      if (s < KS && wv[s] != 0.0f) acc = fmaf(wv[s], dv[s], acc);
    a.out[(int64_t)t * H + r] = acc;
  }
}

// -------------------------------------------------------------- fused shape
template <int BITS, int LPR, int CPL, int WMAX>
__global__ __launch_bounds__(kThreads) void down_fused_kernel(DownArgs a) {
  extern __shared__ __align__(16) uint32_t smem[];
  __shared__ float red[2 * kFusedPairs * kWaves];
  __shared__ float undo[kFusedPairs];
  __shared__ const uint8_t* blob_of[kFusedPairs];
  __shared__ float coef[kFusedPairs];
  constexpr int ROWS = kFusedRows / kWaves;
  using Tile = DownTile<BITS, LPR, CPL, ROWS>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, I = a.I, KS = a.k + a.S, NP = a.T * KS;
  const int nch = I / Tile::PC;
  uint32_t* pairs = smem;
  float* xsum = reinterpret_cast<float*>(pairs + kFusedPairs * (I / 2));

  if (tid < NP) {
    const int t = tid / KS, slot = tid - t * KS;
    const uint8_t* b = nullptr;
    float c = 0.0f;
    if (slot < a.k) {
      const int e = a.topk_idx[(int64_t)t * a.k + slot];
      if (e >= 0 && e < a.E) {
        b = static_cast<const uint8_t*>(a.blobs[e]);
        c = a.topk_w[(int64_t)t * a.k + slot];
      } else {
        set_status(a.status, kStatusBadExpert);
      }
    } else {
      b = static_cast<const uint8_t*>(a.blobs[a.E + (slot - a.k)]);
      c = a.shared_w ? a.shared_w[t] : 1.0f;
    }
    blob_of[tid] = b;
    coef[tid] = c;
  }
  __syncthreads();

  const int wrow0 = blockIdx.x * kFusedRows + wave * ROWS;
  Tile tile[kFusedPairs];
#pragma unroll
  for (int p = 0; p < kFusedPairs; ++p)
    if (p < NP) tile[p].load(blob_of[p], H, I, wrow0, lane);

  auto loader = [&](int m, int64_t o, float* v) {
    load_swiglu<Pack<BITS>::kPerWord>(a.gate_up + (int64_t)m * 2 * I, I, o, v);
  };
  stage_batch<BITS, WMAX, kFusedPairs>(NP, I, loader, false, pairs, xsum, undo, red);

  const int sub = lane % LPR, rsub = lane / LPR;
#pragma unroll
  for (int s = 0; s < Tile::STEPS; ++s) {
    const int rr = s * Tile::RPS + rsub, r = wrow0 + rr;
    const bool row_ok = rr < ROWS && r < H;
    float acc = 0.0f;
#pragma unroll
    for (int p = 0; p < kFusedPairs; ++p) {
      if (p < NP) {
        const int t = p / KS, slot = p - t * KS;
        if (slot == 0) acc = row_ok ? residual_at(a, (int64_t)t * H + r) : 0.0f;
        const float d = tile[p].dot(s, pairs + (int64_t)p * (I / 2), xsum + (int64_t)p * kChunkSums * nch, undo[p],
                                      I, lane);
        if (blob_of[p] != nullptr && coef[p] != 0.0f) acc = fmaf(coef[p], d, acc);
        if (slot == KS - 1 && sub == LPR - 1 && row_ok) a.out[(int64_t)t * H + r] = acc;
      }
    }
  }
}

template <int BITS, int LPR, int CPL, int WMAX>
hipError_t launch_t(const DownArgs& a, hipStream_t stream) {
  const int nch = a.I / Pack<BITS>::kPerChunk;
  const int NP = a.T * (a.k + a.S);
  using FusedTile = DownTile<BITS, LPR, CPL, kFusedRows / kWaves>;
  if (NP <= kFusedPairs && FusedTile::STEPS * CPL <= 2) {
    const int grid = (a.H + kFusedRows - 1) / kFusedRows;
    const size_t lds =
        sizeof(uint32_t) * ((size_t)kFusedPairs * (a.I / 2) + (size_t)kFusedPairs * kChunkSums * nch);
    hipLaunchKernelGGL((down_fused_kernel<BITS, LPR, CPL, WMAX>), dim3(grid), dim3(kThreads), lds,
                       stream, a);
    return hipGetLastError();
  }
  const int n_rb = (a.H + kGroupedRows - 1) / kGroupedRows;
  const int items = min(a.E, a.T * a.k) + a.S;
  const int list_words = (max(a.T * a.k, a.T) + 3) & ~3;
  const size_t lds = sizeof(uint32_t) * ((size_t)kTokensPerStage * (a.I / 2) +
                                         (size_t)kTokensPerStage * kChunkSums * nch +
                                         2 * (size_t)list_words) +
                     sizeof(void*) * (size_t)list_words;
  hipLaunchKernelGGL((down_grouped_kernel<BITS, LPR, CPL, WMAX>), dim3(items * n_rb), dim3(kThreads),
                     lds, stream, a, n_rb, list_words);
  return hipGetLastError();
}

template <int BITS, int LPR, int CPL>
hipError_t launch_w(const DownArgs& a, hipStream_t stream) {
  const int nwords = a.I * BITS / 32;
  const int wmax = (nwords + kThreads - 1) / kThreads;
  if (wmax <= 1) return launch_t<BITS, LPR, CPL, 1>(a, stream);
  if (wmax <= 2) return launch_t<BITS, LPR, CPL, 2>(a, stream);
  return launch_t<BITS, LPR, CPL, 4>(a, stream);
}

template <int BITS>
hipError_t launch_bits(const DownArgs& a, hipStream_t stream) {
  const int nch = a.I / Pack<BITS>::kPerChunk;
  if (nch <= 1) return launch_w<BITS, 1, 1>(a, stream);
  if (nch <= 2) return launch_w<BITS, 2, 1>(a, stream);
  if (nch <= 4) return launch_w<BITS, 4, 1>(a, stream);
  if (nch <= 8) return launch_w<BITS, 8, 1>(a, stream);
  if (nch <= 16) return launch_w<BITS, 16, 1>(a, stream);
  if (nch <= 32) return launch_w<BITS, 32, 1>(a, stream);
  if (nch <= 64) return launch_w<BITS, 64, 1>(a, stream);
  if (nch <= 128) return launch_w<BITS, 64, 2>(a, stream);
  return launch_w<BITS, 64, 4>(a, stream);
}

}  // namespace

int down_row_blocks(int H) { return (H + kGroupedRows - 1) / kGroupedRows; }

hipError_t launch_down_combine(const DownArgs& a, hipStream_t stream) {
  return a.bits == 4 ? launch_bits<4>(a, stream) : launch_bits<2>(a, stream);
}

}  // namespace moeq
