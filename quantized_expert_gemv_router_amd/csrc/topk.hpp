// Top-K selection over fp64 router logits by one wave, ties to the lower
// expert index (Flash-MoE, fr.news.hada.io, "Architecture du modèle": K of
// 512 experts per token), and the softmax weights of the selection.
#pragma once

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

// One wave, DPP lane moves: same selection as wave_topk.  Each lane holds
// its best untaken logit; six DPP steps fold the (value, index) pairs so
// lane 63 holds the winner, which readlane makes uniform.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ void argmax_step(double& v, int& i) {
  const double ov = dpp_move_f64<CTRL, ROW_MASK>(v, v);
  const int oi = dpp_move<CTRL, ROW_MASK>(i, i);
  if (ranks_before(ov, oi, v, i)) { v = ov; i = oi; }
}

__device__ __forceinline__ void wave_topk_dpp(const double* lg, int E, int K, int* sel, double* selv) {
  const int lane = threadIdx.x & 63;
  uint64_t taken = 0;
  for (int r = 0; r < K; ++r) {
    double bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int m = 0, e = lane; e < E; ++m, e += 64) {
      const double v = lg[e];
      if (!((taken >> m) & 1) && ranks_before(v, e, bv, bi)) { bv = v; bi = e; }
    }
    argmax_step<kDppQuadXor1>(bv, bi);
    argmax_step<kDppQuadXor2>(bv, bi);
    argmax_step<kDppHalfMirror>(bv, bi);
    argmax_step<kDppMirror>(bv, bi);
    argmax_step<kDppBcast15, 0xA>(bv, bi);
    argmax_step<kDppBcast31, 0xC>(bv, bi);
    bi = __builtin_amdgcn_readlane(bi, 63);
    bv = readlane_f64(bv, 63);
    if ((bi & 63) == lane) taken |= 1ull << (bi >> 6);
    if (lane == 0) { sel[r] = bi; selv[r] = bv; }
  }
  __builtin_amdgcn_wave_barrier();
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
