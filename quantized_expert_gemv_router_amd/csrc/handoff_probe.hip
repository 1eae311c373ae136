// Diagnostic: latency of the cross-workgroup hand-offs the persistent
// decode kernel is built from, measured on the device it runs on.
//
// One workgroup of 512 threads per CU, all co-resident (cooperative
// launch).  After a start barrier, `rounds` rounds of one pattern run back
// to back and workgroup 0 reports the wall-clock ticks (100 MHz) they took:
//   0  tagged all-gather: every workgroup publishes W tagged 64-bit words
//      (payload | round << 32) and polls all NB * W words until each
//      carries the round's tag (the words are their own flags);
//   1  flag + payload: every workgroup writes W payload words, waits for
//      them to complete, then publishes one tagged flag word; readers poll
//      the NB flags, then read the NB * W payload words once;
//   2  ping-pong: workgroups 0 and `peer` bounce one tagged word, so a
//      round is two one-way hand-offs;
//   3  counter barrier: every workgroup adds 1 to one counter and polls it
//      until it reaches (round + 1) * NB;
//   4  gather + broadcast: every workgroup publishes W tagged words; only
//      workgroup 0 polls them, then it publishes the round's tag in
//      `peer` copies of a go word (one per 4 KiB); every other workgroup
//      polls its copy (workgroup id mod copies);
//   5  as 4, then every workgroup also reads all NB * W words once (they
//      are complete when the go word is seen): completion detected by one
//      poller, data fetched once;
//   6  tagged all-gather as 0 with pipelined polls: every polled word has
//      `peer` (2 or 4) loads in flight, issued a back-off apart, so a word
//      is seen a fraction of a load's round trip after it lands;
//   7  fixed-point reduction: every workgroup adds (1 << 55) + (b mod 256)
//      to each of NB * W 64-bit accumulators with agent-scope atomics and
//      polls them until each count field (bits 55-63) reads NB; the sums
//      are checked.  The accumulators are triple-buffered by round mod 3:
//      after its poll of round r a workgroup clears its own W words of the
//      buffer of round r - 1 and drains, before its adds of round r + 1,
//      and every add of round r + 2 to that buffer follows a poll that saw
//      those round r + 1 adds, so no clear can race with a later add.
// In mode 0 writer j's words start at word j * stride (stride >= W),
// so a larger stride spreads the polled words over more memory channels.
// Every workgroup records the XCD id it runs on (hardware register XCC_ID).
// Words are double-buffered by round parity: a workgroup writes round r + 2
// only after it has seen every workgroup's round r + 1 words, which each
// wrote after finishing its reads of round r.  Every wait is bounded; a
// wait that gives up sets the status word and an abort word and every
// workgroup leaves.
#include "moeq_device.hpp"
#include "moeq_internal.hpp"

namespace moeq {
namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeMaxPer = 16;        // polled words per thread (NB * W <= 8192)
constexpr int kProbeSpin = 1 << 20;

struct ProbeArgs {
  uint64_t* words;      // [2][NB][W]
  uint64_t* flags;      // [2][NB]
  uint32_t* ctl;        // [0] start counter, [1] barrier counter, [2] abort, [3] mismatches
  uint32_t* xmap;       // [NB] XCD id + 1 of each workgroup
  uint64_t* local;      // [2][copies][512] go words (modes 4, 5)
  int W, stride, rounds, mode, sleep, peer;
  int64_t* out;         // [0] ticks of the rounds (workgroup 0)
  int32_t* status;
};

__device__ __forceinline__ void probe_sleep(int s) {
  switch (s) {
    case 0: break;
    case 1: __builtin_amdgcn_s_sleep(1); break;
    case 2: __builtin_amdgcn_s_sleep(2); break;
    default: __builtin_amdgcn_s_sleep(4); break;
  }
}

// Spin until *p (a 64-bit tagged word) carries `tag`; false on give-up.
__device__ bool wait_tag(const uint64_t* p, uint32_t tag, uint32_t* abort, int32_t* status, int s) {
  for (int spins = 0;; ++spins) {
    if ((uint32_t)(ld_agent(p) >> 32) == tag) return true;
    if ((spins & 63) == 63 && ld_agent(abort) != 0u) return false;
    if (spins > kProbeSpin) {
      set_status(status, kStatusTimeout);
      st_agent(abort, 1u);
      return false;
    }
    probe_sleep(s);
  }
}

__device__ __forceinline__ uint32_t xcc_id() {
  return __builtin_amdgcn_s_getreg((20) | (0 << 6) | (15 << 11));   // HW_REG_XCC_ID, bits [15:0]
}

// Polls n words base[tid + i * 512] until each carries `tag` (ld: the
// load); the words land in got[i].
template <class Ld>
__device__ bool poll_all(const uint64_t* base, int n, uint32_t tag, uint32_t* abort, int32_t* status, int s,
                         Ld ld, uint64_t (&got)[kProbeMaxPer]) {
  const int tid = threadIdx.x;
  uint32_t pending = 0;
#pragma unroll
  for (int i = 0; i < kProbeMaxPer; ++i) {
    got[i] = 0ull;
    if (tid + i * kProbeThreads < n) pending |= 1u << i;
  }
  for (int spins = 0; pending != 0; ++spins) {
    uint64_t v[kProbeMaxPer];
#pragma unroll
    for (int i = 0; i < kProbeMaxPer; ++i) v[i] = ((pending >> i) & 1) ? ld(base + tid + i * kProbeThreads) : 0ull;
#pragma unroll
    for (int i = 0; i < kProbeMaxPer; ++i)
      if (((pending >> i) & 1) && (uint32_t)(v[i] >> 32) == tag) {
        got[i] = v[i];
        pending &= ~(1u << i);
      }
    if (pending == 0) break;
    if ((spins & 63) == 63 && ld_agent(abort) != 0u) return false;
    if (spins > kProbeSpin) { set_status(status, kStatusTimeout); st_agent(abort, 1u); return false; }
    probe_sleep(s);
  }
  return true;
}

// Polls n accumulators base[tid + i * 512] until each count field (bits
// 55-63) reads `count`; the words land in got[i].
__device__ bool poll_count(const uint64_t* base, int n, uint32_t count, uint32_t* abort, int32_t* status, int s,
                           uint64_t (&got)[kProbeMaxPer]) {
  const int tid = threadIdx.x;
  uint32_t pending = 0;
#pragma unroll
  for (int i = 0; i < kProbeMaxPer; ++i) {
    got[i] = 0ull;
    if (tid + i * kProbeThreads < n) pending |= 1u << i;
  }
  for (int spins = 0; pending != 0; ++spins) {
    uint64_t v[kProbeMaxPer];
#pragma unroll
    for (int i = 0; i < kProbeMaxPer; ++i) v[i] = ((pending >> i) & 1) ? ld_agent(base + tid + i * kProbeThreads) : 0ull;
#pragma unroll
    for (int i = 0; i < kProbeMaxPer; ++i)
      if (((pending >> i) & 1) && (uint32_t)(v[i] >> 55) == count) {
        got[i] = v[i];
        pending &= ~(1u << i);
      }
    if (pending == 0) break;
    if ((spins & 63) == 63 && ld_agent(abort) != 0u) return false;
    if (spins > kProbeSpin) { set_status(status, kStatusTimeout); st_agent(abort, 1u); return false; }
    probe_sleep(s);
  }
  return true;
}

// Pipelined poll: D loads of each of this thread's (up to 4) words in
// flight at once; a returned load that lacks the tag is re-issued at once.
template <int D>
__device__ bool poll_pipelined(const uint64_t* base, int n, uint32_t tag, uint32_t* abort, int32_t* status,
                               int s) {
  constexpr int P = 4;
  const int tid = threadIdx.x;
  const uint64_t* p[P];
  uint32_t pending = 0;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int w = tid + i * kProbeThreads;
    p[i] = base + (w < n ? w : 0);
    if (w < n) pending |= 1u << i;
  }
  uint64_t v[D][P];
#pragma unroll
  for (int d = 0; d < D; ++d) {
#pragma unroll
    for (int i = 0; i < P; ++i) v[d][i] = ((pending >> i) & 1) ? ld_agent(p[i]) : 0ull;
    probe_sleep(s);
  }
  for (int spins = 0;; ++spins) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
#pragma unroll
      for (int i = 0; i < P; ++i)
        if (((pending >> i) & 1) && (uint32_t)(v[d][i] >> 32) == tag) pending &= ~(1u << i);
      if (pending == 0) return true;
#pragma unroll
      for (int i = 0; i < P; ++i) v[d][i] = ((pending >> i) & 1) ? ld_agent(p[i]) : 0ull;
      probe_sleep(s);
    }
    if ((spins & 15) == 15 && ld_agent(abort) != 0u) return false;
    if (spins > kProbeSpin / D) { set_status(status, kStatusTimeout); st_agent(abort, 1u); return false; }
  }
}

__global__ __launch_bounds__(kProbeThreads) void probe_kernel(ProbeArgs a) {
  const int NB = gridDim.x, b = blockIdx.x, tid = threadIdx.x;
  const int W = a.W, NW = NB * W, SW = a.stride;
  uint32_t* abort = a.ctl + 2;
  __shared__ int fail;
  if (tid == 0) fail = 0;
  if (tid == 0) st_agent(a.xmap + b, xcc_id() + 1u);
  drain_memory();
  // start barrier: every workgroup is running before the clock starts
  if (tid == 0) {
    atomic_add_agent(a.ctl, 1u);
    for (int spins = 0; ld_agent(a.ctl) < (uint32_t)NB; ++spins) {
      if (spins > kProbeSpin) { set_status(a.status, kStatusTimeout); st_agent(abort, 1u); fail = 1; break; }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  if (fail) return;
  const int64_t t0 = (int64_t)wall_clock64();
  for (int r = 0; r < a.rounds; ++r) {
    const uint32_t tag = (uint32_t)r + 1u;
    const int par = r & 1;
    bool ok = true;
    uint64_t got[kProbeMaxPer];
    if (a.mode == 0 && SW == W) {
      uint64_t* buf = a.words + (int64_t)par * NW;
      if (tid < W) st_agent(buf + (int64_t)b * W + tid, ((uint64_t)tag << 32) | (uint32_t)(b * W + tid));
      ok = poll_all(buf, NW, tag, abort, a.status, a.sleep, [](const uint64_t* p) { return ld_agent(p); }, got);
    } else if (a.mode == 0) {   // strided: word i of writer j at j * SW + i
      uint64_t* buf = a.words + (int64_t)par * NB * SW;
      if (tid < W) st_agent(buf + (int64_t)b * SW + tid, ((uint64_t)tag << 32) | (uint32_t)(b * W + tid));
      ok = poll_all(buf, NW, tag, abort, a.status, a.sleep,
                    [&](const uint64_t* p) {
                      const int i = (int)(p - buf);
                      return ld_agent(buf + (int64_t)(i / W) * SW + i % W);
                    }, got);
    } else if (a.mode == 6) {
      uint64_t* buf = a.words + (int64_t)par * NW;
      if (tid < W) st_agent(buf + (int64_t)b * W + tid, ((uint64_t)tag << 32) | (uint32_t)(b * W + tid));
      ok = a.peer >= 4 ? poll_pipelined<4>(buf, NW, tag, abort, a.status, a.sleep)
                       : poll_pipelined<2>(buf, NW, tag, abort, a.status, a.sleep);
    } else if (a.mode == 4 || a.mode == 5) {
      uint64_t* buf = a.words + (int64_t)par * NW;
      uint64_t* go = a.local + (int64_t)par * a.peer * 512;      // copies 4 KiB apart
      if (tid < W) st_agent(buf + (int64_t)b * W + tid, ((uint64_t)tag << 32) | (uint32_t)(b * W + tid));
      if (b == 0) {
        ok = poll_all(buf, NW, tag, abort, a.status, a.sleep, [](const uint64_t* p) { return ld_agent(p); }, got);
        if (!ok) fail = 1;
        block_sync_lds();
        if (!fail && tid < a.peer) st_agent(go + (int64_t)tid * 512, (uint64_t)tag << 32);
      } else if (tid == 0) {
        ok = wait_tag(go + (int64_t)(b % a.peer) * 512, tag, abort, a.status, a.sleep);
        if (!ok) fail = 1;
      }
      block_sync_lds();
      if (fail) return;
      if (a.mode == 5) {
        uint32_t bad = 0;
#pragma unroll
        for (int i = 0; i < kProbeMaxPer; ++i)
          if (tid + i * kProbeThreads < NW) got[i] = ld_agent(buf + tid + i * kProbeThreads);
#pragma unroll
        for (int i = 0; i < kProbeMaxPer; ++i)
          if (tid + i * kProbeThreads < NW && (uint32_t)(got[i] >> 32) != tag) ++bad;
        if (bad) atomic_add_agent(a.ctl + 3, bad);
      }
    } else if (a.mode == 1) {
      uint64_t* buf = a.words + (int64_t)par * NW;
      if (tid < W) st_agent(buf + (int64_t)b * W + tid, ((uint64_t)tag << 32) | (uint32_t)(b * W + tid));
      drain_memory();
      __syncthreads();
      if (tid == 0) st_agent(a.flags + par * NB + b, (uint64_t)tag << 32);
      for (int j = tid; j < NB; j += kProbeThreads)
        ok = ok && wait_tag(a.flags + par * NB + j, tag, abort, a.status, a.sleep);
      if (!ok) fail = 1;
      block_sync_lds();
      if (fail) return;
      uint32_t bad = 0;
      for (int i = tid; i < NW; i += kProbeThreads)
        if ((uint32_t)(ld_agent(buf + i) >> 32) != tag) ++bad;
      if (bad) atomic_add_agent(a.ctl + 3, bad);
    } else if (a.mode == 7) {
      uint64_t* buf = a.words + (int64_t)(r % 3) * NW;
      const uint64_t add = (1ull << 55) + (uint64_t)(b & 0xFF);
      for (int i = tid; i < NW; i += kProbeThreads)
        __hip_atomic_fetch_add(buf + i, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ok = poll_count(buf, NW, (uint32_t)NB, abort, a.status, a.sleep, got);
      if (ok) {
        uint64_t want = 0;   // sum over the workgroups of b mod 256
        for (int j = 0; j < NB; ++j) want += (uint64_t)(j & 0xFF);
        uint32_t bad = 0;
#pragma unroll
        for (int i = 0; i < kProbeMaxPer; ++i)
          if (tid + i * kProbeThreads < NW && (got[i] & ((1ull << 55) - 1)) != want) ++bad;
        if (bad) atomic_add_agent(a.ctl + 3, bad);
        if (tid < W) st_agent(a.words + (int64_t)((r + 2) % 3) * NW + (int64_t)b * W + tid, (uint64_t)0);
        drain_memory();
      }
    } else if (a.mode == 2) {
      if (tid == 0 && (b == 0 || b == a.peer) && a.peer != 0) {
        uint64_t* ping = a.flags;          // written by workgroup 0
        uint64_t* pong = a.flags + 1;      // written by the peer
        if (b == 0) {
          st_agent(ping, (uint64_t)tag << 32);
          ok = wait_tag(pong, tag, abort, a.status, a.sleep);
        } else {
          ok = wait_tag(ping, tag, abort, a.status, a.sleep);
          if (ok) st_agent(pong, (uint64_t)tag << 32);
        }
      }
    } else {
      if (tid == 0) {
        atomic_add_agent(a.ctl + 1, 1u);
        const uint32_t target = (uint32_t)(r + 1) * (uint32_t)NB;
        for (int spins = 0; ld_agent(a.ctl + 1) < target; ++spins) {
          if ((spins & 63) == 63 && ld_agent(abort) != 0u) { ok = false; break; }
          if (spins > kProbeSpin) { set_status(a.status, kStatusTimeout); st_agent(abort, 1u); ok = false; break; }
          probe_sleep(a.sleep);
        }
      }
    }
    if (!ok) fail = 1;
    block_sync_lds();
    if (fail) return;
  }
  if (b == 0 && tid == 0) a.out[0] = (int64_t)wall_clock64() - t0;
}

}  // namespace

// [ctl 4 KiB][xmap 4 KiB][words 2*NB*stride][flags 2*NB][go words 2*64*4 KiB]
int64_t probe_scratch_bytes(int nb, int W, int stride) {
  return 8192 + align_up((int64_t)2 * nb * stride * 8) + align_up((int64_t)2 * nb * 8) + 2 * 64 * 4096;
}

hipError_t launch_probe(int mode, int W, int stride, int rounds, int sleep, int peer, void* scratch, int nb,
                        hipStream_t stream) {
  char* s = static_cast<char*>(scratch);
  ProbeArgs a{};
  a.ctl = reinterpret_cast<uint32_t*>(s);
  a.status = reinterpret_cast<int32_t*>(s + 64);
  a.out = reinterpret_cast<int64_t*>(s + 128);
  a.xmap = reinterpret_cast<uint32_t*>(s + 4096);
  a.words = reinterpret_cast<uint64_t*>(s + 8192);
  a.flags = reinterpret_cast<uint64_t*>(s + 8192 + align_up((int64_t)2 * nb * stride * 8));
  a.local = reinterpret_cast<uint64_t*>(s + 8192 + align_up((int64_t)2 * nb * stride * 8) +
                                        align_up((int64_t)2 * nb * 8));
  a.W = W; a.stride = stride; a.rounds = rounds; a.mode = mode; a.sleep = sleep; a.peer = peer;
  void* params[] = {&a};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&probe_kernel), dim3(nb),
                                    dim3(kProbeThreads), params, 0, stream);
}

int probe_max_words() { return kProbeMaxPer * kProbeThreads; }

}  // namespace moeq
