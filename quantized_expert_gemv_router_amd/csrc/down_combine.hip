// SwiGLU, down projection and weighted combine of 4-, 3- or 2-bit experts (Flash-MoE,
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
//  - grouped (multi-token batches): one workgroup per (chunk of 4 of the
//    expert's (token, slot) pairs, expert item, range of rows), so an
//    expert many tokens chose spreads over more workgroups.  Each stages
//    its activation vectors once and streams its down rows in tiles of
//    about 8 KB per wave, double-buffered in registers (range-checked
//    buffer loads; 4-bit rows dequantised once for all staged vectors),
//    writing per-slot rows to the workspace; a second kernel then sums
//    them per token in slot order onto the residual.
// Either way a token's output does not depend on what else is in the batch.
#include "grouping.hpp"
#include "moeq_internal.hpp"
#include "staging.hpp"

namespace moeq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
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
  uint2 qh[STEPS][CPL];   // 3-bit: the chunk's high-bit plane
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
        qh[s][c] = make_uint2(0u, 0u);
        if (row_ok && cc < nch) {
          q[s][c] = load_stream(reinterpret_cast<const u32x4*>(blob + qoff + r * row_bytes) + cc);
          if constexpr (BITS == 3) qh[s][c] = load_stream_u2(blob + qoff + r * row_bytes + I / 4 + 8 * cc);
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
      if (cc < nch)
        part += chunk_term<BITS>(chunk_dot_q<BITS>(q[s][c], qh[s][c], load_xchunk<BITS>(xp, cc, nch)), sbw[s][c],
                                 *reinterpret_cast<const float2*>(xs + kChunkSums * cc));
    }
    return group_sum_dpp<LPR>(part) * undo;
  }
};

// ------------------------------------------------------------ grouped shape
// 4-bit chunk dequantised once into its magic-exponent fp16 pairs (the
// operands chunk_dot forms, same order), then dotted with several staged
// chunks, so a row pays the dequant once for all of a workgroup's tokens.
struct DqChunk4 {
  uint32_t p[16];
};
__device__ __forceinline__ DqChunk4 dequant_chunk4(u32x4 q) {
  DqChunk4 d;
  const uint32_t mg = magic_pair();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = q[i], t = w >> 8;
    d.p[4 * i + 0] = (w & 0x000F000Fu) | mg;
    d.p[4 * i + 1] = (w & 0x00F000F0u) | mg;
    d.p[4 * i + 2] = (t & 0x000F000Fu) | mg;
    d.p[4 * i + 3] = (t & 0x00F000F0u) | mg;
  }
  return d;
}
__device__ __forceinline__ float dot_chunk4(const DqChunk4& d, const XChunk<4>& x) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = dot2(d.p[4 * i + 0], x.u[i].x, acc);
    acc = dot2(d.p[4 * i + 1], x.u[i].y, acc);
    acc = dot2(d.p[4 * i + 2], x.u[i].z, acc);
    acc = dot2(d.p[4 * i + 3], x.u[i].w, acc);
  }
  return acc;
}

// A tile of down rows: LPR lanes per row (lane sub = lane % LPR holds
// chunks sub + LPR * c), RPS = 64 / LPR rows per step, STEPS steps per wave,
// about 8 KB per wave.
template <int BITS, int LPR, int CPL>
struct DownRows {
  static constexpr int RPS = 64 / LPR;
  static constexpr int STEPS = 4 / CPL > 0 ? 4 / CPL : 1;
  static constexpr int RW = STEPS * RPS;          // rows per wave per tile
  static constexpr int TR = kWaves * RW;          // rows per tile
  u32x4 q[STEPS][CPL];
  uint2 qh[STEPS][CPL];   // 3-bit: the chunk's high-bit plane
  uint32_t sb[STEPS][CPL];
};

// Row of step s of tile j for this lane: r_lo + j * TR + wave * RW + s * RPS + lane / LPR.
// Rows at or past r_hi (and lanes past the last chunk) read at the end of
// the buffer's range: zeros, and no memory request.
template <int BITS, int LPR, int CPL>
__device__ __forceinline__ void issue_down_tile(DownRows<BITS, LPR, CPL>& t, rsrc_t rq, rsrc_t rs,
                                                uint32_t q_bytes, uint32_t s_bytes, int j, int r_lo, int r_hi,
                                                int row_bytes, int gpr, int nch, int wave, int lane_in) {
  using T = DownRows<BITS, LPR, CPL>;
  constexpr int PC = Pack<BITS>::kPerChunk;
  int lane;   // re-derived per tile: its offsets are not kept live across the loop
  asm volatile("v_mov_b32 %0, %1" : "=v"(lane) : "v"(lane_in));
  const int sub = lane % LPR, rsub = lane / LPR;
#pragma unroll
  for (int s = 0; s < T::STEPS; ++s) {
    const int r = r_lo + j * T::TR + wave * T::RW + s * T::RPS + rsub;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int cc = sub + LPR * c;
      const bool ok = r < r_hi && cc < nch;
      const uint32_t qo = ok ? (uint32_t)r * (uint32_t)row_bytes + 16u * (uint32_t)cc : q_bytes;
      const uint32_t so = ok ? 4u * ((uint32_t)r * (uint32_t)gpr + (uint32_t)(cc * PC / 64)) : s_bytes;
      t.q[s][c] = load_rsrc_b128(rq, qo);
      if constexpr (BITS == 3) {
        // the high-bit plane follows the low plane (2/3 of the row's bytes)
        const uint32_t ho = ok ? (uint32_t)r * (uint32_t)row_bytes + (uint32_t)(2 * row_bytes / 3) + 8u * (uint32_t)cc
                               : q_bytes;
        t.qh[s][c] = load_rsrc_b64(rq, ho);
      } else {
        t.qh[s][c] = make_uint2(0u, 0u);
      }
      t.sb[s][c] = load_rsrc_b32(rs, so);
    }
  }
  issue_fence();
}

// Tile j against the nv staged activation vectors (list entries m0..m0+nv):
// per-slot rows into dbuf.
template <int BITS, int LPR, int CPL, int MMAX>
__device__ __forceinline__ void apply_down_tile(const DownRows<BITS, LPR, CPL>& t, const DownArgs& a, int j,
                                                int r_lo, int r_hi, int nv, int m0, const uint32_t* pairs,
                                                const float* xsum, const float* undo, const uint32_t* list,
                                                int nch, int wave, int lane_in) {
  using T = DownRows<BITS, LPR, CPL>;
  const int H = a.H, I = a.I, KS = a.k + a.S;
  int lane;
  asm volatile("v_mov_b32 %0, %1" : "=v"(lane) : "v"(lane_in));
  const int sub = lane % LPR, rsub = lane / LPR;
  float part[T::STEPS][MMAX];
#pragma unroll
  for (int s = 0; s < T::STEPS; ++s)
#pragma unroll
    for (int m = 0; m < MMAX; ++m) part[s][m] = 0.0f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int cc = sub + LPR * c;
    if (cc < nch) {
      XChunk<BITS> xc[MMAX];
      float2 x2[MMAX];
#pragma unroll
      for (int m = 0; m < MMAX; ++m) {
        if (m < nv) {
          xc[m] = load_xchunk<BITS>(pairs + (int64_t)m * (I / 2), cc, nch);
          x2[m] = *reinterpret_cast<const float2*>(xsum + (int64_t)m * kChunkSums * nch + kChunkSums * cc);
        }
      }
#pragma unroll
      for (int s = 0; s < T::STEPS; ++s) {
        if constexpr (BITS == 4) {
          const DqChunk4 d = dequant_chunk4(t.q[s][c]);
#pragma unroll
          for (int m = 0; m < MMAX; ++m)
            if (m < nv) part[s][m] += chunk_affine(dot_chunk4(d, xc[m]), t.sb[s][c], x2[m]);
        } else {
#pragma unroll
          for (int m = 0; m < MMAX; ++m)
            if (m < nv) part[s][m] += chunk_term<BITS>(chunk_dot_q<BITS>(t.q[s][c], t.qh[s][c], xc[m]), t.sb[s][c], x2[m]);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MMAX; ++m) {
    if (m < nv) {
      const uint32_t e = list[m0 + m];
      const int tk = (int)(e >> 8), slot = (int)(e & 255u);
      const float u = undo[m];
      float* dst = a.dbuf + ((int64_t)tk * KS + slot) * H;
#pragma unroll
      for (int s = 0; s < T::STEPS; ++s) {
        const float v = group_sum_dpp<LPR>(part[s][m]) * u;
        const int r = r_lo + j * T::TR + wave * T::RW + s * T::RPS + rsub;
        if (sub == LPR - 1 && r < r_hi) dst[r] = v;
      }
    }
  }
}

// Grid, NS row ranges per unit: first the n_extra units that may hold a
// later chunk of an item's (token, slot) list (entries 4c.., c >= 1;
// group_extra finds which, the rest exit), then chunk 0 of the n_routed
// routed items and the S shared experts (items missing from this batch
// exit).  Writes d for every (token, slot, row) of its items into dbuf
// [T][k + S][H].
template <int BITS, int LPR, int CPL, int WMAX>
__global__ __launch_bounds__(kThreads) void down_batch_kernel(DownArgs a, int NS, int n_routed, int n_extra,
                                                                                       int list_words) {
  using T = DownRows<BITS, LPR, CPL>;
  extern __shared__ __align__(16) uint32_t smem[];
  __shared__ GroupLds g;
  __shared__ float red[2 * kTokensPerStage * kWaves];
  __shared__ float undo[kTokensPerStage];
  constexpr int MMAX = kTokensPerStage;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, I = a.I, KS = a.k + a.S;
  const int nch = I / Pack<BITS>::kPerChunk;
  uint32_t* pairs = smem;
  float* xsum = reinterpret_cast<float*>(pairs + kTokensPerStage * (I / 2));
  uint32_t* list = reinterpret_cast<uint32_t*>(xsum + kTokensPerStage * kChunkSums * nch);
  int* ids = reinterpret_cast<int*>(list + list_words);
  const uint8_t** ptrs = reinterpret_cast<const uint8_t**>(ids + list_words);

  uint32_t* hist = reinterpret_cast<uint32_t*>(ptrs + list_words);
  int split;
  if ((int)blockIdx.x < n_extra * NS) {   // later token chunks first: they run long
    const int u = blockIdx.x / NS;
    split = blockIdx.x - u * NS;
    group_extra<MMAX>(u, a.topk_idx, a.blobs, a.T, a.k, a.E, a.S, g, list, ids, ptrs, hist, a.status);
  } else {
    const int b = blockIdx.x - n_extra * NS;
    const int it = b / NS;
    split = b - it * NS;
    const int item = it < n_routed ? it : -1 - (it - n_routed);
    group_item(item, a.topk_idx, a.blobs, a.T, a.k, a.E, a.S, g, list, ids, ptrs, a.status);
  }
  if (g.expert < 0) return;
  const int m0 = g.chunk * MMAX;
  if (m0 >= g.count) return;
  const int nv = min(MMAX, g.count - m0);

  const int ntiles = (H + T::TR - 1) / T::TR;
  const int t_lo = (int)((int64_t)ntiles * split / NS), t_hi = (int)((int64_t)ntiles * (split + 1) / NS);
  if (t_lo >= t_hi) return;
  const int r_lo = t_lo * T::TR, r_hi = min(H, t_hi * T::TR);
  const int nt = t_hi - t_lo;

  const int row_bytes = I * BITS / 8;
  const int gpr = I / 64;
  const uint8_t* blob = g.blob;
  const uint32_t q_bytes = (uint32_t)H * (uint32_t)row_bytes, s_bytes = (uint32_t)H * (uint32_t)gpr * 4u;
  const rsrc_t rq = make_rsrc(blob + 2 * (int64_t)H * I * BITS / 8, q_bytes);                           // down.q
  const rsrc_t rs = make_rsrc(blob + 3 * (int64_t)H * I * BITS / 8 + 2 * (int64_t)H * I / 64 * 4, s_bytes);  // down.sb

  auto loader = [&](int m, int64_t o, float* v) {
    const uint32_t e = list[m0 + m];
    const int t = (int)(e >> 8), slot = (int)(e & 255u);
    load_swiglu<Pack<BITS>::kPerWord>(a.gate_up + ((int64_t)t * KS + slot) * 2 * I, I, o, v);
  };
  stage_batch<BITS, WMAX, MMAX>(nv, I, loader, false, pairs, xsum, undo, red);

  T ta, tb;
  issue_down_tile<BITS, LPR, CPL>(ta, rq, rs, q_bytes, s_bytes, 0, r_lo, r_hi, row_bytes, gpr, nch, wave, lane);
  for (int j = 0; j < nt; j += 2) {
    issue_down_tile<BITS, LPR, CPL>(tb, rq, rs, q_bytes, s_bytes, j + 1, r_lo, r_hi, row_bytes, gpr, nch, wave,
                                    lane);
    apply_down_tile<BITS, LPR, CPL, MMAX>(ta, a, j, r_lo, r_hi, nv, m0, pairs, xsum, undo, list, nch, wave, lane);
    issue_down_tile<BITS, LPR, CPL>(ta, rq, rs, q_bytes, s_bytes, j + 2, r_lo, r_hi, row_bytes, gpr, nch, wave,
                                    lane);
    if (j + 1 < nt)
      apply_down_tile<BITS, LPR, CPL, MMAX>(tb, a, j + 1, r_lo, r_hi, nv, m0, pairs, xsum, undo, list, nch, wave,
                                            lane);
  }
}

// out[t][r] = residual[t][r] + sum over slots, in slot order, of w * d.
// Slots whose routed id is out of range add nothing.  One thread per (t, r).
__global__ __launch_bounds__(kThreads) void combine_kernel(DownArgs a) {
  const int H = a.H, KS = a.k + a.S;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (int64_t)a.T * H) return;
  const int t = (int)(idx / H), r = (int)(idx - (int64_t)t * H);
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
      if (ok) dv[s] = a.dbuf[((int64_t)t * KS + s) * H + r];
      else wv[s] = 0.0f;
    }
  }
  float acc = residual_at(a, (int64_t)t * H + r);
#pragma unroll
  for (int s = 0; s < MOEQ_MAX_TOPK + 1; ++s)
    if (s < KS && wv[s] != 0.0f) acc = fmaf(wv[s], dv[s], acc);
  a.out[(int64_t)t * H + r] = acc;
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

int cu_count() {
  static int n = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return 256;
    return v;
  }();
  return n;
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
  const int n_routed = min(a.E, a.T * a.k);
  const int n_items = n_routed + a.S;
  const int list_words = (max(a.T * a.k, a.T) + 3) & ~3;
  const int ntiles = (a.H + DownRows<BITS, LPR, CPL>::TR - 1) / DownRows<BITS, LPR, CPL>::TR;
  // about eight workgroups per CU over the items' first token chunks
  const int NS = max(1, min((8 * cu_count() + n_items - 1) / max(n_items, 1), ntiles));
  const int NTC = (a.T + kTokensPerStage - 1) / kTokensPerStage;
  const int n_extra = a.T * a.k / kTokensPerStage + a.S * (NTC - 1);   // bound on later token chunks
  const int64_t grid = (int64_t)(n_extra + n_items) * NS;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const size_t lds = sizeof(uint32_t) * ((size_t)kTokensPerStage * (a.I / 2) +
                                         (size_t)kTokensPerStage * kChunkSums * nch +
                                         2 * (size_t)list_words + (size_t)a.E) +
                     sizeof(void*) * (size_t)list_words;
  hipLaunchKernelGGL((down_batch_kernel<BITS, LPR, CPL, WMAX>), dim3((unsigned)grid), dim3(kThreads), lds, stream,
                     a, NS, n_routed, n_extra, list_words);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t cgrid = ((int64_t)a.T * a.H + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)cgrid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int BITS, int LPR, int CPL>
hipError_t launch_w(const DownArgs& a, hipStream_t stream) {
  const int nwords = a.I / Pack<BITS>::kPerWord;   // staged words per activation vector
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

hipError_t launch_down_combine(const DownArgs& a, hipStream_t stream) {
  if (a.bits == 4) return launch_bits<4>(a, stream);
  if (a.bits == 3) return launch_bits<3>(a, stream);
  return launch_bits<2>(a, stream);
}

}  // namespace moeq
