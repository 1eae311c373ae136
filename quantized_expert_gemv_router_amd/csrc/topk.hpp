// Top-K selection over fp64 router logits by one wave, ties to the lower
// expert index (Flash-MoE, fr.news.hada.io, "Architecture du modèle": K of
// 512 experts per token), and the softmax weights of the selection.
#pragma once

#include <climits>

#include "moeq_device.hpp"

namespace moeq {

// (value desc, index asc) total order: does (va, ia) rank before (vb, ib)?
__device__ __forceinline__ bool ranks_before(double va, int ia, double vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// One wave: logits lg[0..E) in LDS (E <= 4096).  Writes sel[0..K) and
// selv[0..K) (LDS, by lane 0) in rank order.  Each round every lane finds
// its best untaken logit, then a butterfly over the wave picks the winner.
__device__ __forceinline__ void wave_topk(const double* lg, int E, int K, int* sel, double* selv) {
  const int lane = threadIdx.x & 63;
  uint64_t taken = 0;
  for (int r = 0; r < K; ++r) {
    double bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int m = 0, e = lane; e < E; ++m, e += 64) {
      const double v = lg[e];
      if (!((taken >> m) & 1) && ranks_before(v, e, bv, bi)) { bv = v; bi = e; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double ov = shfl_xor_f64(bv, o);
      const int oi = __shfl_xor(bi, o, 64);
      if (ranks_before(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if ((bi & 63) == lane) taken |= 1ull << (bi >> 6);
    if (lane == 0) { sel[r] = bi; selv[r] = bv; }
  }
  __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------- key form
// Register-resident selection.  A logit becomes a signed 64-bit key whose
// integer order is the numeric order of the logit (-0 is folded into +0 so
// the two tie, as they do when compared as numbers); kNoKey sorts below every
// key of a real logit and marks empty or taken slots.
constexpr int kTopkNone = 0x7FFFFFFF;
constexpr int64_t kNoKey = (int64_t)0x8000000000000000ull;

__device__ __forceinline__ int64_t order_key(double v) {
  if (v == 0.0) v = 0.0;
  const int64_t b = __double_as_longlong(v);
  return b >= 0 ? b : (b ^ 0x7FFFFFFFFFFFFFFFll);
}

// Wave maxima of 32-bit words; each step is one DPP-modified max (the lane
// move is folded into the max), the identity fills rows a broadcast skips.
__device__ __forceinline__ int wave_max_i32(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, kDppQuadXor1, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, kDppQuadXor2, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, kDppHalfMirror, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, kDppMirror, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, kDppBcast15, 0xA, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, kDppBcast31, 0xC, 0xF, false));
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadXor1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadXor2, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppHalfMirror, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppMirror, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppBcast15, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppBcast31, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Wave maximum of 64-bit keys: the high words first (signed), then the low
// words (unsigned) of the lanes holding the top high word, skipped when a
// single lane holds it.
__device__ __forceinline__ int64_t wave_max_key(int64_t key) {
  const int hi = (int)(key >> 32);
  const uint32_t lo = (uint32_t)key;
  const int mh = wave_max_i32(hi);
  const uint64_t mask = __ballot(hi == mh);
  uint32_t ml;
  if ((mask & (mask - 1)) == 0) ml = (uint32_t)__builtin_amdgcn_readlane((int)lo, __builtin_ctzll(mask));
  else ml = wave_max_u32(hi == mh ? lo : 0u);
  return (int64_t)(((uint64_t)(uint32_t)mh << 32) | ml);
}

__device__ __forceinline__ int wave_min_int(int m) {
  m = min(m, dpp_move<kDppQuadXor1>(m, m));
  m = min(m, dpp_move<kDppQuadXor2>(m, m));
  m = min(m, dpp_move<kDppHalfMirror>(m, m));
  m = min(m, dpp_move<kDppMirror>(m, m));
  m = min(m, dpp_move<kDppBcast15, 0xA>(m, m));
  m = min(m, dpp_move<kDppBcast31, 0xC>(m, m));
  return __builtin_amdgcn_readlane(m, 63);
}

// A lane's best slot: highest key, then lowest index.  ORDERED says the slot
// order is the index order, so ties on the key keep the lower slot and the
// indices need not be compared.  Pairwise tree of selects over the slots.
template <int M, bool ORDERED>
__device__ __forceinline__ void lane_best(const int64_t (&k)[M], const int (&id)[M], int64_t& bk, int& bi) {
  int64_t tk[M];
  int ti[M];
#pragma unroll
  for (int i = 0; i < M; ++i) { tk[i] = k[i]; ti[i] = id[i]; }
#pragma unroll
  for (int w = 1; w < M; w *= 2) {
#pragma unroll
    for (int i = 0; i + w < M; i += 2 * w) {
      const bool right = ORDERED ? tk[i + w] > tk[i]
                                 : (tk[i + w] > tk[i] || (tk[i + w] == tk[i] && ti[i + w] < ti[i]));
      tk[i] = right ? tk[i + w] : tk[i];
      ti[i] = right ? ti[i + w] : ti[i];
    }
  }
  bk = tk[0];
  bi = ti[0];
}

// One wave: the K best of the elements held in k/id (lane's slots, kNoKey
// for empty ones), in rank order.  Round r publishes (key, index) through
// emit(r, key, index) on lane 0; index is kTopkNone once nothing is left.
// Each round is a DPP max over the lanes' best keys; lanes that tie on it
// settle on the lowest index; the winner's slot is then emptied.
template <int M, bool ORDERED, typename Emit>
__device__ __forceinline__ void wave_select(int64_t (&k)[M], const int (&id)[M], int K, Emit emit) {
  const int lane = threadIdx.x & 63;
  for (int r = 0; r < K; ++r) {
    int64_t lk;
    int li;
    lane_best<M, ORDERED>(k, id, lk, li);
    const int64_t m = wave_max_key(lk);
    int win = kTopkNone;
    if (m != kNoKey) {
      const uint64_t mask = __ballot(lk == m);
      win = (mask & (mask - 1)) == 0 ? __builtin_amdgcn_readlane(li, __builtin_ctzll(mask))
                                     : wave_min_int(lk == m ? li : kTopkNone);
#pragma unroll
      for (int i = 0; i < M; ++i) k[i] = id[i] == win ? kNoKey : k[i];
    }
    if (lane == 0) emit(r, m, win);
  }
}

// One wave: top-K of lg[0..E) (LDS, E <= 64*M), ties to the lower index.
// sel/selv (LDS) receive the indices and logits in rank order.
template <int M>
__device__ __forceinline__ void wave_topk_keys(const double* lg, int E, int K, int* sel, double* selv) {
  const int lane = threadIdx.x & 63;
  int64_t k[M];
  int id[M];
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const int e = lane + 64 * i;
    k[i] = e < E ? order_key(lg[e]) : kNoKey;
    id[i] = e < E ? e : kTopkNone;
  }
  wave_select<M, true>(k, id, K, [&](int r, int64_t, int win) {
    sel[r] = win;
    selv[r] = win != kTopkNone ? lg[win] : -INFINITY;
  });
  __builtin_amdgcn_wave_barrier();
}

// All NW waves of a block: top-K (K <= 64*MC/NW) of lg[0..E) (LDS, E <= 64*NW*M).
// Wave w selects the K best of its elements w*64 + lane + 64*NW*i into
// ck/ci[w*K + r]; wave 0 then selects the K best of those NW*K candidates
// (MC per lane).  Same result as one wave over all E.  Ends with a block
// barrier.
template <int NW, int M, int MC>
__device__ __forceinline__ void block_topk_keys(const double* lg, int E, int K, int64_t* ck, int* ci,
                                                int* sel, double* selv) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  {
    int64_t k[M];
    int id[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const int e = w * 64 + lane + 64 * NW * i;
      k[i] = e < E ? order_key(lg[e]) : kNoKey;
      id[i] = e < E ? e : kTopkNone;
    }
    wave_select<M, true>(k, id, K, [&](int r, int64_t key, int win) {
      ck[w * K + r] = key;
      ci[w * K + r] = win;
    });
  }
  __syncthreads();
  if (w == 0) {
    int64_t k[MC];
    int id[MC];
#pragma unroll
    for (int i = 0; i < MC; ++i) {
      const int c = lane + 64 * i;
      const bool ok = c < NW * K && ci[c] != kTopkNone;
      k[i] = ok ? ck[c] : kNoKey;
      id[i] = ok ? ci[c] : kTopkNone;
    }
    wave_select<MC, false>(k, id, K, [&](int r, int64_t, int win) {
      sel[r] = win;
      selv[r] = win != kTopkNone ? lg[win] : -INFINITY;
    });
  }
  __syncthreads();
}

// All NW waves, one logit per thread (E <= 64*NW), K <= 2*NW: top-K by a
// threshold.  Each wave publishes its P = ceil(K/NW) largest keys; tau, the
// K-th largest of those NW*P samples, is at most the K-th largest key of all
// E, so every element of the true top-K has a key >= tau, and at least K
// elements do.  Those candidates are compacted into LDS and ranked by
// (key desc, index asc) in wave 0.  Returns false (nothing written, block
// uniform) when more than 64 candidates pass, e.g. under massive ties; the
// caller then runs block_topk_keys.  Scratch: wk [2*NW], ck/ci [64], cnt,
// tau.  Ends with a block barrier.
template <int NW>
__device__ __forceinline__ bool block_topk_sample(const double* lg, int E, int K, int64_t* wk, int64_t* ck,
                                                  int* ci, int* cnt, int64_t* tau, int* sel, double* selv) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int P = (K + NW - 1) / NW;
  const int64_t key = tid < E ? order_key(lg[tid]) : kNoKey;
  const int64_t m1 = wave_max_key(key);
  int64_t m2 = kNoKey;
  if (P > 1) {   // second largest: drop one lane holding the maximum
    const uint64_t mask = __ballot(key == m1);
    m2 = wave_max_key(lane == __builtin_ctzll(mask) ? kNoKey : key);
  }
  if (lane == 0) {
    wk[w * P] = m1;
    if (P > 1) wk[w * P + 1] = m2;
  }
  if (tid == 0) *cnt = 0;
  __syncthreads();
  if (tid < NW * P) {   // the sample of rank K-1 (ties by sample position)
    const int64_t v = wk[tid];
    int r = 0;
    for (int s = 0; s < NW * P; ++s) {
      const int64_t o = wk[s];
      r += (o > v || (o == v && s < tid)) ? 1 : 0;
    }
    if (r == K - 1) *tau = v;
  }
  __syncthreads();
  if (tid < E && key >= *tau) {
    const int slot = atomicAdd(cnt, 1);
    if (slot < 64) {
      ck[slot] = key;
      ci[slot] = tid;
    }
  }
  __syncthreads();
  const int C = *cnt;
  if (C > 64) return false;
  if (tid < C) {
    const int64_t v = ck[tid];
    const int vi = ci[tid];
    int r = 0;
    for (int c = 0; c < C; ++c) {
      const int64_t o = ck[c];
      r += (o > v || (o == v && ci[c] < vi)) ? 1 : 0;
    }
    if (r < K) {
      sel[r] = vi;
      selv[r] = lg[vi];
    }
  }
  __syncthreads();
  return true;
}

// One wave, K <= 64: softmax weights over the K selected logits (fp64,
// rounded to fp32), one exponential per lane.  Returns lane's weight.
__device__ __forceinline__ float wave_softmax_selected(const double* selv, int K) {
  const int lane = threadIdx.x & 63;
  const double m = selv[0];   // the top-ranked logit is the maximum
  const double e = lane < K ? exp(selv[lane] - m) : 0.0;
  const double z = wave_sum_f64_dpp(e);
  return lane < K ? (float)(e / z) : 0.0f;
}

// One wave: softmax weights of the selection (fp64, rounded to fp32):
// over the K selected logits, or (no_renorm) the full softmax over all E
// logits read at the selected experts.  Returns the weight of lane's slot.
__device__ __forceinline__ float wave_softmax_weight(const double* lg, int E, int K,
                                                     const double* selv, bool no_renorm) {
  const int lane = threadIdx.x & 63;
  const double m = selv[0];   // the top-ranked logit is the maximum
  double z = 0.0;
  if (no_renorm) {
    double part = 0.0;
    for (int e = lane; e < E; e += 64) part += exp(lg[e] - m);
    z = wave_sum_f64(part);
  } else {
    for (int r = 0; r < K; ++r) z += exp(selv[r] - m);
  }
  return lane < K ? (float)(exp(selv[lane] - m) / z) : 0.0f;
}

}  // namespace moeq
