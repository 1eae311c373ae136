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

// One wave: the K best of M keys per lane (element index lane + 64 i, so a
// lane's slots are in index order; kNoKey marks an empty slot), in rank
// order, through emit(r, index) on lane 0 (kTopkNone once nothing is left).
// Same result as wave_select, with fewer instructions per round: a round
// takes the wave maximum of the keys' high words (a monotone map of the
// key, 32-bit DPP steps); when one element alone holds it, that element's
// key is strictly the largest and wins.  A tie on the high word is settled
// on the full keys of the tied elements, then on the lower index.
template <int M, typename Emit>
__device__ __forceinline__ void wave_select_hi(const int64_t (&k)[M], int K, Emit emit) {
  const int lane = threadIdx.x & 63;
  int h[M];
  uint32_t alive = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const bool real = k[i] != kNoKey;
    h[i] = real ? (int)(k[i] >> 32) : INT_MIN;
    alive |= real ? (1u << i) : 0u;
  }
  for (int r = 0; r < K; ++r) {
    int lm = h[0];
#pragma unroll
    for (int i = 1; i < M; ++i) lm = max(lm, h[i]);
    const int mh = wave_max_i32(lm);
    uint32_t mk = 0;   // alive slots of this lane holding the maximum
#pragma unroll
    for (int i = 0; i < M; ++i) mk |= (h[i] == mh) ? (1u << i) : 0u;
    mk &= alive;
    const uint64_t B = __ballot(mk != 0);
    int win = kTopkNone;
    if (B != 0) {
      const int l0 = (int)__builtin_ctzll(B);
      const uint32_t m0 = (uint32_t)__builtin_amdgcn_readlane((int)mk, l0);
      if ((B & (B - 1)) == 0 && (m0 & (m0 - 1)) == 0) {
        win = l0 + 64 * (int)__builtin_ctz(m0);
      } else {
        int64_t lk = kNoKey;
        int li = kTopkNone;
#pragma unroll
        for (int i = 0; i < M; ++i)
          if (((mk >> i) & 1u) && (li == kTopkNone || k[i] > lk)) { lk = k[i]; li = lane + 64 * i; }
        const int64_t m = wave_max_key(lk);
        const uint64_t mask = __ballot(li != kTopkNone && lk == m);
        win = (mask & (mask - 1)) == 0 ? __builtin_amdgcn_readlane(li, __builtin_ctzll(mask))
                                       : wave_min_int(li != kTopkNone && lk == m ? li : kTopkNone);
      }
      const uint32_t wm = lane == (win & 63) ? (1u << (win >> 6)) : 0u;
#pragma unroll
      for (int i = 0; i < M; ++i) h[i] = ((wm >> i) & 1u) ? INT_MIN : h[i];
      alive &= ~wm;
    }
    if (lane == 0) emit(r, win);
  }
}

// ------------------------------------------------------ selection network
// One wave, K <= 4, eight logits per lane (element lane + 64 i): the top
// elements found by one pass of sorted four-lists through the wave instead
// of K rounds of wave maxima.  Each element becomes a 32-bit key:
// the high word of its order key with the three lowest bits replaced by
// 7 - i (its slot), so a key names its element within the lane.  A lane
// sorts its eight keys into its four best; six DPP steps then merge lists
// pairwise (the top four of two sorted lists: the bitonic elementwise
// maximum of one list against the other reversed, then two half-cleaner
// stages), and lane 63 ends with the wave's four best keys.  When their
// 29-bit prefixes (the truncated order keys) are strictly decreasing, the
// order of the K best and the boundary to the (K+1)-th are fixed by the
// prefixes alone, so the keys give the exact selection.  At K = 4 the lists
// hold no fifth key; the boundary is shown instead by a count: exactly four
// elements have a prefix at or above the fourth's.  Otherwise (near-ties
// within 2^-17 relative, or ties) it returns false and the caller selects
// on the full keys.  On success lane r < K receives the
// element of rank r in `win` (wave-uniform per rank through readlane).
__device__ __forceinline__ int net_key(double v, int slot) {
  v = v + 0.0;   // -0 becomes +0: the two tie, as numbers do
  const int hb = (int)((uint64_t)__double_as_longlong(v) >> 32);
  const int hk = hb ^ ((hb >> 31) & 0x7FFFFFFF);
  return (hk & ~7) | (7 - slot);
}

// top four of the sorted (descending) lists a and b, sorted
__device__ __forceinline__ void net_merge4(int (&a)[4], const int (&b)[4]) {
  const int c0 = max(a[0], b[3]), c1 = max(a[1], b[2]), c2 = max(a[2], b[1]), c3 = max(a[3], b[0]);
  const int d0 = max(c0, c2), d2 = min(c0, c2), d1 = max(c1, c3), d3 = min(c1, c3);
  a[0] = max(d0, d1);
  a[1] = min(d0, d1);
  a[2] = max(d2, d3);
  a[3] = min(d2, d3);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void net_step(int (&a)[4]) {
  int b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = __builtin_amdgcn_update_dpp(INT_MIN, a[i], CTRL, ROW_MASK, 0xF, false);
  net_merge4(a, b);
}

// lg: the E (<= 512) logits in LDS, lg[e] for e < E; K <= 4.  Returns true
// with lane r < K holding the rank-r element in win; false when the
// prefixes do not separate the top K from the rest.
__device__ __forceinline__ bool wave_topk_net(const double* lg, int E, int K, int& win) {
  const int lane = threadIdx.x & 63;
  // every read in range (clamped), so the eight are issued together
  double lv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) lv[i] = lg[min(lane + 64 * i, E - 1)];
  int k[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int kk = net_key(lv[i], i);   // computed in every lane: a select, no branch
    k[i] = lane + 64 * i < E ? kk : INT_MIN;
  }
  // the lane's four best, sorted
  int a[4] = {max(k[0], k[1]), min(k[0], k[1]), INT_MIN, INT_MIN};
  int b[4] = {max(k[2], k[3]), min(k[2], k[3]), INT_MIN, INT_MIN};
  int c[4] = {max(k[4], k[5]), min(k[4], k[5]), INT_MIN, INT_MIN};
  int d[4] = {max(k[6], k[7]), min(k[6], k[7]), INT_MIN, INT_MIN};
  net_merge4(a, b);
  net_merge4(c, d);
  net_merge4(a, c);
  int loc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) loc[i] = a[i];
  net_step<kDppQuadXor1, 0xF>(a);
  net_step<kDppQuadXor2, 0xF>(a);
  net_step<kDppHalfMirror, 0xF>(a);
  net_step<kDppMirror, 0xF>(a);
  net_step<kDppBcast15, 0xA>(a);
  net_step<kDppBcast31, 0xC>(a);
  int t[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) t[i] = __builtin_amdgcn_readlane(a[i], 63);
  // prefixes strictly decreasing over the min(K + 1, 4) best (INT_MIN past E)
  bool ok = true;
#pragma unroll
  for (int i = 0; i < 3; ++i)
    if (i < K) ok = ok && t[i] != INT_MIN && (t[i] >> 3) > (t[i + 1] >> 3);
  if (K == 4) {   // no fifth key: no element but the four may reach the fourth's prefix
    const int p3 = t[3] >> 3;
    int n = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) n += __popcll(__ballot((k[i] >> 3) >= p3));
    ok = ok && t[3] != INT_MIN && n == 4;
  }
  if (!ok) return false;
  win = kTopkNone;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (r >= K) break;
    const bool mine = loc[0] == t[r] || loc[1] == t[r] || loc[2] == t[r] || loc[3] == t[r];
    const int owner = (int)__builtin_ctzll(__ballot(mine));
    if (lane == r) win = owner + 64 * (7 - (t[r] & 7));
  }
  return true;
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

// Threshold top-K over NW waves, one key per thread (E <= 64*NW, K <= 2*NW),
// in three steps separated by block barriers, after which EVERY wave holds
// the selection (no barrier is needed between the selection and its use).
// The threshold works on the keys' high words h = key >> 32 (a monotone
// map, so ties only add candidates): each wave publishes its P =
// ceil(K/NW) largest h; tau, the K-th largest of those NW*P samples, is at
// most the high word of the K-th largest key, so every element of the true
// top-K has h >= tau, and at least K elements do.  Those candidates are
// compacted per wave and ranked on their full keys (key desc, index asc).
//
// Step 1 (each wave, then a block barrier): samples into wk[w*P ..].
template <int NW>
__device__ __forceinline__ void topk_samples(int64_t key, int K, int* wk) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int P = (K + NW - 1) / NW;
  const int h = (int)(key >> 32);
  const int m1 = wave_max_i32(h);
  int m2 = INT_MIN;
  if (P > 1) {   // second largest: drop one lane holding the maximum
    const uint64_t mask = __ballot(h == m1);
    m2 = wave_max_i32(lane == __builtin_ctzll(mask) ? INT_MIN : h);
  }
  if (lane == 0) {
    wk[w * P] = m1;
    if (P > 1) wk[w * P + 1] = m2;
  }
}

// Step 2 (every wave, then a block barrier): tau from the samples (each
// wave computes it), then this wave's candidates (h >= tau; element index
// e) into ck/ci[w*64 ..] and their number into cnt[w].
template <int NW>
__device__ __forceinline__ void topk_candidates(int64_t key, int e, int K, const int* wk, int64_t* ck,
                                                int* ci, int* cnt) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int NS = NW * ((K + NW - 1) / NW);
  // the sample of rank K-1 (ties by sample position): lane s < NS ranks
  // sample s by counting
  const int v = lane < NS ? wk[lane] : INT_MIN;
  int r = 0;
#pragma unroll
  for (int s = 0; s < 2 * NW; ++s) {
    const int o = __builtin_amdgcn_readlane(v, s);
    r += (s < NS && (o > v || (o == v && s < lane))) ? 1 : 0;
  }
  const uint64_t at = __ballot(lane < NS && r == K - 1);
  const int tau = __builtin_amdgcn_readlane(v, __builtin_ctzll(at));
  const bool pass = key != kNoKey && (int)(key >> 32) >= tau;
  const uint64_t mask = __ballot(pass);
  if (pass) {
    const int pos = __builtin_popcountll(mask & ((1ull << lane) - 1ull));
    ck[w * 64 + pos] = key;
    ci[w * 64 + pos] = e;
  }
  if (lane == 0) cnt[w] = __builtin_popcountll(mask);
}

// Step 3 (every wave): the K best candidates in rank order through
// emit(r, index) on the lane holding rank r.  Returns false (the same in
// every wave) when more than 64 candidates passed; the caller then falls
// back to block_topk_keys.
template <int NW, typename Emit>
__device__ __forceinline__ bool topk_select(int K, const int64_t* ck, const int* ci, const int* cnt, Emit emit) {
  const int lane = threadIdx.x & 63;
  int pre[NW + 1];
  pre[0] = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) pre[w + 1] = pre[w] + __builtin_amdgcn_readfirstlane(cnt[w]);
  const int C = pre[NW];
  if (C > 64) return false;
  int64_t k = kNoKey;
  int id = kTopkNone;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (lane >= pre[w] && lane < pre[w + 1]) {
      k = ck[w * 64 + lane - pre[w]];
      id = ci[w * 64 + lane - pre[w]];
    }
  }
  // rank by counting over the C candidates (few: about K)
  int r = 0;
  for (int c = 0; c < C; ++c) {
    const int64_t o = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(k >> 32), c) << 32) |
                                (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k, c));
    const int oi = __builtin_amdgcn_readlane(id, c);
    r += (o > k || (o == k && oi < id)) ? 1 : 0;
  }
  if (lane < C && r < K) emit(r, id);
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
