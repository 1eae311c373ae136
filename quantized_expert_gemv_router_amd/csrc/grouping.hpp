// Per-workgroup expert grouping for decode batches.
//
// Each workgroup of the expert kernels owns one (expert, row block) work
// item.  Items are numbered by the distinct routed experts of the batch in
// ascending id order, then the shared experts.  Every workgroup rebuilds
// the grouping from topk_idx in LDS (a bitmap of selected experts, a
// popcount scan to find its own expert, and a ballot compaction of the
// (token, slot) pairs routed to it, in pair order), so no separate sort
// launch is needed and the result is the same in every workgroup.
#pragma once

#include "moeq.h"
#include "moeq_device.hpp"

namespace moeq {

constexpr int kBitmapWords = MOEQ_MAX_EXPERTS / 32;   // 128

struct GroupLds {
  uint32_t bitmap[kBitmapWords];
  int expert;       // routed id, or E + s for shared expert s, or -1 (no work)
  int count;        // (token, slot) pairs in `list`
  int n_distinct;
};

// list entries: token << 8 | slot.  `list` must hold T*k (routed) or T
// (shared) entries.  Returns nothing; results in g / list.  Whole block.
__device__ __forceinline__ void group_item(int item, const int32_t* __restrict__ topk_idx,
                                           int T, int k, int E, int S, GroupLds& g,
                                           uint32_t* __restrict__ list,
                                           int32_t* status) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int P = T * k;
  for (int i = tid; i < kBitmapWords; i += blockDim.x) g.bitmap[i] = 0u;
  __syncthreads();
  for (int p = tid; p < P; p += blockDim.x) {
    int e = topk_idx[p];
    if (e >= 0 && e < E) atomicOr(&g.bitmap[e >> 5], 1u << (e & 31));
    else set_status(status, kStatusBadExpert);
  }
  __syncthreads();
  if (tid < 64) {
    // lane l owns bitmap words 2l and 2l+1
    uint32_t w0 = g.bitmap[2 * lane], w1 = g.bitmap[2 * lane + 1];
    int c = __popc(w0) + __popc(w1);
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    int excl = incl - c;
    int total = __shfl(incl, 63, 64);
    if (lane == 0) { g.n_distinct = total; g.expert = -1; g.count = 0; }
    __builtin_amdgcn_wave_barrier();
    if (item < total) {
      if (item >= excl && item < incl) {
        int r = item - excl;
        uint32_t w = w0;
        int base = 64 * lane;
        if (r >= __popc(w0)) { r -= __popc(w0); w = w1; base += 32; }
        for (int i = 0; i < r; ++i) w &= w - 1;   // drop the r lowest set bits
        g.expert = base + __builtin_ctz(w);
      }
    } else if (item < total + S) {
      if (lane == 0) g.expert = E + (item - total);
    }
  }
  __syncthreads();
  const int e = g.expert;
  if (tid < 64 && e >= 0) {
    if (e < E) {
      int cnt = 0;
      for (int base = 0; base < P; base += 64) {
        int p = base + lane;
        bool hit = p < P && topk_idx[p] == e;
        uint64_t m = __ballot(hit);
        if (hit) {
          int pos = cnt + __popcll(m & ((1ull << lane) - 1ull));
          int t = p / k;
          list[pos] = ((uint32_t)t << 8) | (uint32_t)(p - t * k);
        }
        cnt += __popcll(m);
      }
      if (lane == 0) g.count = cnt;
    } else {
      const int slot = k + (e - E);
      for (int t = lane; t < T; t += 64) list[t] = ((uint32_t)t << 8) | (uint32_t)slot;
      if (lane == 0) g.count = T;
    }
  }
  __syncthreads();
}

}  // namespace moeq
