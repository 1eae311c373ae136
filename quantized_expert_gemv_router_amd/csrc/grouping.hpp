// Per-workgroup expert grouping for decode batches.
//
// Each workgroup of the expert kernels owns one (expert item, row block)
// work item.  Items are numbered by the distinct routed experts of the
// batch in ascending id order, then the shared experts.  Every workgroup
// rebuilds the grouping from topk_idx in LDS (a bitmap of selected experts,
// a popcount scan to find its own expert, and a ballot compaction of the
// (token, slot) pairs routed to it, in pair order), so no separate sort
// launch is needed and the result is the same in every workgroup.  The
// blob pointer of every selected expert is fetched in the same pass as the
// ids, so the expert's weights can be requested as soon as it is known.
#pragma once

#include "moeq.h"
#include "moeq_device.hpp"

namespace moeq {

constexpr int kBitmapWords = MOEQ_MAX_EXPERTS / 32;   // 128

struct GroupLds {
  uint32_t bitmap[kBitmapWords];
  const uint8_t* blob;   // weights of this item's expert (null: no work)
  const uint8_t* shared_blob;
  int expert;            // routed id, or E + s for shared expert s, or -1 (no work)
  int count;             // (token, slot) pairs in `list`
  int n_distinct;
  int in_range;          // item < n_distinct + S (the item exists in this batch)
  int chunk;             // token chunk of the item this workgroup takes (group_extra)
};

// Wave 0: the (token, slot) list of item expert e (routed id, or E + s for
// shared expert s) into list, in pair order; returns its length and sets
// blob.  ids/ptrs hold the routed ids and their blobs (from the scan).
__device__ __forceinline__ int collect_item(int e, int lane, int T, int k, int E, int P,
                                            const void* const* __restrict__ blobs, const GroupLds& g,
                                            uint32_t* __restrict__ list, const int* __restrict__ ids,
                                            const uint8_t* const* __restrict__ ptrs, const uint8_t*& blob) {
  int cnt = 0;
  blob = nullptr;
  if (e >= 0 && e < E) {
    for (int base = 0; base < P; base += 64) {
      const int p = base + lane;
      const bool hit = p < P && ids[p] == e;
      const uint64_t m = __ballot(hit);
      if (hit) {
        const int pos = cnt + __popcll(m & ((1ull << lane) - 1ull));
        const int t = p / k;
        list[pos] = ((uint32_t)t << 8) | (uint32_t)(p - t * k);
        if (pos == 0) blob = ptrs[p];
      }
      cnt += __popcll(m);
    }
    const uint64_t hb = __ballot(blob != nullptr);
    if (hb) blob = reinterpret_cast<const uint8_t*>(
                __shfl((long long)(uintptr_t)blob, (int)__builtin_ctzll(hb), 64));
  } else if (e >= E) {
    const int slot = k + (e - E);
    for (int t = lane; t < T; t += 64) list[t] = ((uint32_t)t << 8) | (uint32_t)slot;
    cnt = T;
    blob = (e == E) ? g.shared_blob : static_cast<const uint8_t*>(blobs[e]);
  }
  return cnt;
}

// LDS scratch the caller provides: list [max(T*k, T)] u32, ids [T*k] int,
// ptrs [T*k] pointers.  list entries: token << 8 | slot.  A negative item
// -1 - s names shared expert s directly.  Whole block.
__device__ __forceinline__ void group_item(int item, const int32_t* __restrict__ topk_idx,
                                           const void* const* __restrict__ blobs, int T, int k,
                                           int E, int S, GroupLds& g, uint32_t* __restrict__ list,
                                           int* __restrict__ ids, const uint8_t** __restrict__ ptrs,
                                           int32_t* status) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int P = T * k;
  for (int i = tid; i < kBitmapWords; i += blockDim.x) g.bitmap[i] = 0u;
  if (tid == 0) g.shared_blob = S > 0 ? static_cast<const uint8_t*>(blobs[E]) : nullptr;
  __syncthreads();
  for (int p = tid; p < P; p += blockDim.x) {
    const int e = topk_idx[p];
    const bool ok = e >= 0 && e < E;
    ids[p] = ok ? e : -1;
    ptrs[p] = ok ? static_cast<const uint8_t*>(blobs[e]) : nullptr;
    if (ok) atomicOr(&g.bitmap[e >> 5], 1u << (e & 31));
    else set_status(status, kStatusBadExpert);
  }
  __syncthreads();
  if (tid < 64) {
    // lane l owns bitmap words 2l and 2l+1
    const uint32_t w0 = g.bitmap[2 * lane], w1 = g.bitmap[2 * lane + 1];
    const int c = __popc(w0) + __popc(w1);
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    const int excl = incl - c;
    const int total = __shfl(incl, 63, 64);
    int e = -1;
    if (item < 0) {
      if (-1 - item < S) e = E + (-1 - item);
    } else if (item < total) {
      // the owner lane finds the item-th set bit; broadcast it
      int mine = -1;
      if (item >= excl && item < incl) {
        int r = item - excl;
        uint32_t w = w0;
        int base = 64 * lane;
        if (r >= __popc(w0)) { r -= __popc(w0); w = w1; base += 32; }
        for (int i = 0; i < r; ++i) w &= w - 1;   // drop the r lowest set bits
        mine = base + __builtin_ctz(w);
      }
      const uint64_t owner = __ballot(mine >= 0);
      e = __shfl(mine, (int)__builtin_ctzll(owner), 64);
    } else if (item < total + S) {
      e = E + (item - total);
    }
    const uint8_t* blob;
    const int cnt = collect_item(e, lane, T, k, E, P, blobs, g, list, ids, ptrs, blob);
    if (lane == 0) {
      g.n_distinct = total;
      g.in_range = item < 0 ? (-1 - item < S) : (item < total + S);
      g.expert = (blob != nullptr && cnt > 0) ? e : -1;
      g.blob = blob;
      g.count = cnt;
      g.chunk = 0;
    }
  }
  __syncthreads();
}

// One token: item i is slot i (the k routed slots, then the S shared
// experts).  A token's slots are separate outputs, so no grouping is
// needed; an out-of-range id is flagged and its item does nothing.  Whole
// block.
__device__ __forceinline__ void group_single(int item, const int32_t* __restrict__ topk_idx,
                                             const void* const* __restrict__ blobs, int k, int E, int S,
                                             GroupLds& g, uint32_t* __restrict__ list, int32_t* status) {
  if (threadIdx.x == 0) {
    int e = -1;
    if (item < k) {
      const int id = topk_idx[item];
      if (id >= 0 && id < E) e = id;
      else set_status(status, kStatusBadExpert);
    } else if (item < k + S) {
      e = E + (item - k);
    }
    const uint8_t* blob = e >= 0 ? static_cast<const uint8_t*>(blobs[e]) : nullptr;
    g.expert = blob != nullptr ? e : -1;
    g.blob = blob;
    g.count = 1;
    g.chunk = 0;
    g.n_distinct = k;
    g.in_range = item < k + S;
    list[0] = (uint32_t)item;   // token 0, slot `item`
  }
  __syncthreads();
}

// Later token chunks.  An item with n (token, slot) pairs has ceil(n / C)
// chunks of C; chunks 1.. of all items, numbered in item order (routed
// experts by id, then the shared experts), are the batch's extra chunks,
// at most floor(T*k / C) + S * (ceil(T / C) - 1) of them.  Fills g and list
// as group_item does for the item holding extra chunk u, with g.chunk its
// chunk number (>= 1); g.expert = -1 past the last one.  hist: LDS [E] u32.
// Whole block.
template <int C>
__device__ __forceinline__ void group_extra(int u, const int32_t* __restrict__ topk_idx,
                                            const void* const* __restrict__ blobs, int T, int k, int E,
                                            int S, GroupLds& g, uint32_t* __restrict__ list,
                                            int* __restrict__ ids, const uint8_t** __restrict__ ptrs,
                                            uint32_t* __restrict__ hist, int32_t* status) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int P = T * k;
  for (int i = tid; i < E; i += blockDim.x) hist[i] = 0u;
  if (tid == 0) g.shared_blob = S > 0 ? static_cast<const uint8_t*>(blobs[E]) : nullptr;
  __syncthreads();
  for (int p = tid; p < P; p += blockDim.x) {
    const int e = topk_idx[p];
    const bool ok = e >= 0 && e < E;
    ids[p] = ok ? e : -1;
    ptrs[p] = ok ? static_cast<const uint8_t*>(blobs[e]) : nullptr;
    if (ok) atomicAdd(&hist[e], 1u);
    else set_status(status, kStatusBadExpert);
  }
  __syncthreads();
  if (tid < 64) {
    // lane l owns experts [l * per, (l + 1) * per)
    const int per = (E + 63) / 64;
    const int lo = lane * per, hi = min(E, lo + per);
    int c = 0;
    for (int e = lo; e < hi; ++e) c += hist[e] > 0 ? (int)((hist[e] - 1) / C) : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    const int excl = incl - c;
    const int total = __shfl(incl, 63, 64);
    int e = -1, chunk = 0;
    if (u < total) {
      int mine = -1, mc = 0;
      if (u >= excl && u < incl) {
        int r = u - excl;
        for (int x = lo; x < hi; ++x) {
          const int n = hist[x] > 0 ? (int)((hist[x] - 1) / C) : 0;
          if (r < n) { mine = x; mc = 1 + r; break; }
          r -= n;
        }
      }
      const uint64_t owner = __ballot(mine >= 0);
      const int ol = (int)__builtin_ctzll(owner);
      e = __shfl(mine, ol, 64);
      chunk = __shfl(mc, ol, 64);
    } else {
      const int per_s = (T + C - 1) / C - 1;
      const int v = u - total;
      if (per_s > 0 && v / per_s < S) {
        e = E + v / per_s;
        chunk = 1 + v % per_s;
      }
    }
    const uint8_t* blob;
    const int cnt = collect_item(e, lane, T, k, E, P, blobs, g, list, ids, ptrs, blob);
    if (lane == 0) {
      g.in_range = e >= 0;
      g.expert = (blob != nullptr && cnt > chunk * C) ? e : -1;
      g.blob = blob;
      g.count = cnt;
      g.chunk = chunk;
    }
  }
  __syncthreads();
}

}  // namespace moeq
