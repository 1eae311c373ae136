// Expert slot pool: a bounded device arena of expert slots filled from a
// pinned host copy of every (layer, expert) blob on router demand, with the
// least recently used slot evicted (openclawradar.com/fr, Flash-MoE
// write-up: experts cached in a fixed number of resident slots and loaded
// when the router asks for them; fr.news.hada.io, Flash-MoE, "SSD Expert
// Streaming": each expert is one contiguous 6.75 MiB read).
//
// The pool keeps the device pointer table [layer][E + S] that the expert
// kernels read (the moeq_experts view): an entry points at its slot while
// the expert is resident and is NULL otherwise.  The host copy of each
// (layer, expert) blob is any pinned allocation (a host table of pointers),
// so the experts need not sit in one contiguous host image.  Misses are
// spread over the caller's copy streams (round robin: several DMA transfers
// in flight at once); table edits run on the first of them.  The compute
// stream waits on an event of every copy stream used, so a kernel never
// reads a slot before its copy has landed.  A slot is only overwritten after
// the last layer that used it has been released: the copy stream of the
// miss and the edit stream wait for that release's event.
#include <hip/hip_runtime.h>

#include <vector>

#include "moeq.h"
#include "moeq_internal.hpp"
#include "pool_core.hpp"

struct moeq_pool {
  moeq::PoolCore core;
  moeq_shape shape{};
  int64_t expert_bytes = 0, slot_bytes = 0;
  uint8_t* arena = nullptr;
  std::vector<const uint8_t*> host;     // [n_layers * (E + S)] pinned host blobs
  const void** table = nullptr;
  std::vector<hipStream_t> copy;        // copy streams; copy[0] also carries the table edits
  int next_stream = 0;                  // round-robin position for the next miss
  std::vector<hipEvent_t> released;     // [n_layers] recorded by moe_pool_release
  std::vector<char> released_valid;
  std::vector<hipEvent_t> ready;        // per copy stream: last work a compute stream must see
  std::vector<char> ready_valid;
  std::vector<char> prefetched;         // [n_slots] last filled by a prefetch (on copy stream 0)
  int64_t bytes_copied = 0;
};

struct moeq_poolsim {
  moeq::PoolCore core;
};

namespace moeq {
namespace {

constexpr int kEditBatch = 32;

struct TableEdits {
  int32_t n;
  int32_t idx[kEditBatch];
  const void* ptr[kEditBatch];
};

// Small pointer-table edits, passed by value so no host buffer has to
// outlive the launch.
__global__ void table_edit_kernel(const void** table, TableEdits e) {
  const int i = threadIdx.x;
  if (i < e.n) table[e.idx[i]] = e.ptr[i];
}

// Whole table: every entry NULL, or entry i -> arena + i * slot_bytes.
__global__ void table_fill_kernel(const void** table, int64_t n, const uint8_t* arena, int64_t slot_bytes,
                                  int identity) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    table[i] = identity ? static_cast<const void*>(arena + i * slot_bytes) : nullptr;
}

int fill_table(moeq_pool* p, int identity) {
  const int64_t n = (int64_t)p->core.n_layers * p->core.per_layer;
  const int blocks = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
  hipLaunchKernelGGL(table_fill_kernel, dim3(blocks), dim3(256), 0, p->copy[0], p->table, n, p->arena,
                     p->slot_bytes, identity);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOEQ_OK : hip_fail(e, "pool table fill launch");
}

int flush_edits(moeq_pool* p, TableEdits& ed) {
  if (ed.n == 0) return MOEQ_OK;
  hipLaunchKernelGGL(table_edit_kernel, dim3(1), dim3(kEditBatch), 0, p->copy[0], p->table, ed);
  ed.n = 0;
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOEQ_OK : hip_fail(e, "pool table edit launch");
}

int add_edit(moeq_pool* p, TableEdits& ed, int32_t idx, const void* ptr) {
  ed.idx[ed.n] = idx;
  ed.ptr[ed.n] = ptr;
  if (++ed.n == kEditBatch) return flush_edits(p, ed);
  return MOEQ_OK;
}

// The compute stream waits for everything queued so far on the copy streams
// marked in `used` (and on every stream that has ever carried work, whose
// last event is still recorded).
int publish(moeq_pool* p, hipStream_t compute, const std::vector<char>& used) {
  for (size_t i = 0; i < p->copy.size(); ++i) {
    if (used[i]) {
      hipError_t e = hipEventRecord(p->ready[i], p->copy[i]);
      if (e != hipSuccess) return hip_fail(e, "hipEventRecord (pool ready)");
      p->ready_valid[i] = 1;
    }
    if (p->ready_valid[i]) {
      hipError_t e = hipStreamWaitEvent(compute, p->ready[i], 0);
      if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent (pool ready)");
    }
  }
  return MOEQ_OK;
}

int check_pool(const moeq_pool* p) {
  if (!p) return fail(MOEQ_E_INVALID, "pool is NULL");
  return MOEQ_OK;
}

}  // namespace
}  // namespace moeq

using namespace moeq;

extern "C" {

int moe_pool_create(const moeq_shape* shape, int n_layers, void* arena, int64_t n_slots, int64_t slot_bytes,
                    const void* const* host_blobs, const void** table, void* const* copy_streams,
                    int n_copy_streams, moeq_pool** out) {
  if (int rc = check_shape(shape)) return rc;
  if (!out) return fail(MOEQ_E_INVALID, "out is NULL");
  *out = nullptr;
  if (n_layers <= 0) return fail(MOEQ_E_INVALID, "n_layers=%d must be positive", n_layers);
  if (n_slots <= 0) return fail(MOEQ_E_INVALID, "n_slots=%lld must be positive", (long long)n_slots);
  if (!arena || !host_blobs || !table) return fail(MOEQ_E_INVALID, "arena, host_blobs and table must be non-NULL");
  if (n_copy_streams < 1 || n_copy_streams > MOEQ_POOL_MAX_COPY_STREAMS || !copy_streams)
    return fail(MOEQ_E_INVALID, "n_copy_streams=%d outside [1, %d] or copy_streams NULL", n_copy_streams,
                MOEQ_POOL_MAX_COPY_STREAMS);
  const int64_t eb = moeq_expert_bytes(shape);
  if (slot_bytes < eb || slot_bytes % 256 != 0)
    return fail(MOEQ_E_INVALID, "slot_bytes=%lld must be a multiple of 256 and >= the expert size %lld",
                (long long)slot_bytes, (long long)eb);
  if (reinterpret_cast<uintptr_t>(arena) % 256 != 0) return fail(MOEQ_E_INVALID, "arena must be 256-byte aligned");
  const int64_t per = (int64_t)shape->n_experts + shape->n_shared;
  if ((int64_t)n_layers * per > INT32_MAX) return fail(MOEQ_E_UNSUPPORTED, "too many (layer, expert) entries");
  const int64_t entries = (int64_t)n_layers * per;

  // every host blob must be pinned (hipHostMalloc or a pinned tensor):
  // pageable memory would make every miss a synchronous staged copy.  Blobs
  // that share an allocation are checked once.
  const void* last_base = nullptr;
  size_t last_size = 0;
  for (int64_t i = 0; i < entries; ++i) {
    const void* h = host_blobs[i];
    if (!h) return fail(MOEQ_E_INVALID, "host blob %lld is NULL", (long long)i);
    const uintptr_t u = reinterpret_cast<uintptr_t>(h);
    if (last_base && u >= reinterpret_cast<uintptr_t>(last_base) &&
        u + (uintptr_t)eb <= reinterpret_cast<uintptr_t>(last_base) + last_size)
      continue;
    hipPointerAttribute_t attr{};
    hipError_t e = hipPointerGetAttributes(&attr, h);
    (void)hipGetLastError();
    if (e != hipSuccess || attr.type != hipMemoryTypeHost)
      return fail(MOEQ_E_INVALID, "host blob %lld is not pinned host memory (hipHostMalloc)", (long long)i);
    void* base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void*>(h)) == hipSuccess && base) {
      last_base = base;
      last_size = size;
    } else {
      (void)hipGetLastError();
      last_base = nullptr;
    }
  }

  moeq_pool* p = new moeq_pool;
  if (!p->core.init(n_layers, (int32_t)per, n_slots)) {
    delete p;
    return fail(MOEQ_E_INVALID, "pool sizes rejected");
  }
  p->shape = *shape;
  p->expert_bytes = eb;
  p->slot_bytes = slot_bytes;
  p->arena = static_cast<uint8_t*>(arena);
  p->host.assign(reinterpret_cast<const uint8_t* const*>(host_blobs),
                 reinterpret_cast<const uint8_t* const*>(host_blobs) + entries);
  p->table = table;
  for (int i = 0; i < n_copy_streams; ++i) p->copy.push_back(static_cast<hipStream_t>(copy_streams[i]));
  p->released.assign((size_t)n_layers, nullptr);
  p->released_valid.assign((size_t)n_layers, 0);
  p->ready.assign((size_t)n_copy_streams, nullptr);
  p->ready_valid.assign((size_t)n_copy_streams, 0);
  p->prefetched.assign((size_t)n_slots, 0);
  auto cleanup = [&]() {
    for (hipEvent_t ev : p->released)
      if (ev) (void)hipEventDestroy(ev);
    for (hipEvent_t ev : p->ready)
      if (ev) (void)hipEventDestroy(ev);
    delete p;
  };
  hipError_t e = hipSuccess;
  for (int l = 0; l < n_layers; ++l) {
    e = hipEventCreateWithFlags(&p->released[(size_t)l], hipEventDisableTiming);
    if (e != hipSuccess) {
      cleanup();
      return hip_fail(e, "hipEventCreateWithFlags");
    }
  }
  for (int i = 0; i < n_copy_streams; ++i) {
    e = hipEventCreateWithFlags(&p->ready[(size_t)i], hipEventDisableTiming);
    if (e != hipSuccess) {
      cleanup();
      return hip_fail(e, "hipEventCreateWithFlags");
    }
  }
  if (int rc = fill_table(p, 0)) {
    cleanup();
    return rc;
  }
  *out = p;
  return ok();
}

int moe_pool_make_resident(moeq_pool* p, void* stream) {
  if (int rc = check_pool(p)) return rc;
  if (!p->core.make_resident())
    return fail(MOEQ_E_UNSUPPORTED, "make_resident needs n_slots >= n_layers * (E + S) = %lld (have %lld)",
                (long long)p->core.n_layers * p->core.per_layer, (long long)p->core.n_slots);
  const int64_t entries = (int64_t)p->core.n_layers * p->core.per_layer;
  // identity placement: entry i in slot i, copies spread over the streams
  std::vector<char> used(p->copy.size(), 0);
  for (int64_t i = 0; i < entries; ++i) {
    const size_t c = (size_t)(i % (int64_t)p->copy.size());
    hipError_t e = hipMemcpyAsync(p->arena + i * p->slot_bytes, p->host[(size_t)i], (size_t)p->expert_bytes,
                                  hipMemcpyHostToDevice, p->copy[c]);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (make_resident)");
    used[c] = 1;
  }
  p->bytes_copied += entries * p->expert_bytes;
  if (int rc = fill_table(p, 1)) return rc;
  used[0] = 1;
  if (int rc = publish(p, static_cast<hipStream_t>(stream), used)) return rc;
  return ok();
}

int moe_pool_acquire(moeq_pool* p, int layer, const int32_t* ids, int n, void* compute_stream,
                     moeq_experts* view) {
  if (int rc = check_pool(p)) return rc;
  if (!view) return fail(MOEQ_E_INVALID, "view is NULL");
  if (n < 0 || (n > 0 && !ids)) return fail(MOEQ_E_INVALID, "ids must hold n >= 0 host int32 values");
  std::vector<PoolCore::Step> steps;
  const int rc = p->core.acquire(layer, ids, n, steps);
  if (rc == -1)
    return fail(MOEQ_E_INVALID, "layer %d outside [0, %d), an id outside [0, %d), or the layer not released",
                layer, p->core.n_layers, p->core.per_layer);
  if (rc == -2)
    return fail(MOEQ_E_POOL_EXHAUSTED, "layer %d needs more free slots than the %lld-slot pool has unpinned", layer,
                (long long)p->core.n_slots);
  hipStream_t compute = static_cast<hipStream_t>(compute_stream);
  const size_t ns = p->copy.size();
  // waited[s * n_layers + l]: copy stream s already waits for layer l's release
  std::vector<char> waited(ns * (size_t)p->core.n_layers, 0);
  std::vector<char> used(ns, 0);
  auto wait_release = [&](size_t s, int layer) -> int {
    if (layer < 0 || !p->released_valid[(size_t)layer] || waited[s * p->core.n_layers + layer]) return MOEQ_OK;
    const hipError_t e = hipStreamWaitEvent(p->copy[s], p->released[(size_t)layer], 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent (slot reuse)");
    waited[s * p->core.n_layers + layer] = 1;
    return MOEQ_OK;
  };
  TableEdits ed{};
  for (const PoolCore::Step& st : steps) {
    if (!st.miss) continue;
    // the slot's previous user must be done with it, on the copy stream of
    // this miss and on the edit stream (which clears the evicted entry)
    const size_t c = (size_t)p->next_stream;
    p->next_stream = (p->next_stream + 1) % (int)ns;
    if (int r = wait_release(c, st.prev_layer)) return r;
    if (int r = wait_release(0, st.prev_layer)) return r;
    // a slot last filled by a prefetch (copy stream 0) is overwritten only
    // after that copy
    if (p->prefetched[(size_t)st.slot] && c != 0 && p->ready_valid[0]) {
      const hipError_t e = hipStreamWaitEvent(p->copy[c], p->ready[0], 0);
      if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent (prefetched slot)");
    }
    p->prefetched[(size_t)st.slot] = 0;
    uint8_t* dst = p->arena + (int64_t)st.slot * p->slot_bytes;
    const hipError_t e = hipMemcpyAsync(dst, p->host[(size_t)st.entry], (size_t)p->expert_bytes,
                                        hipMemcpyHostToDevice, p->copy[c]);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (pool miss)");
    p->bytes_copied += p->expert_bytes;
    used[c] = 1;
    used[0] = 1;
    if (st.evicted >= 0)
      if (int r = add_edit(p, ed, st.evicted, nullptr)) return r;
    if (int r = add_edit(p, ed, st.entry, dst)) return r;
  }
  if (int r = flush_edits(p, ed)) return r;
  if (int r = publish(p, compute, used)) return r;
  view->blobs = p->table;
  view->n_layers = p->core.n_layers;
  return ok();
}

int moe_pool_prefetch(moeq_pool* p, int layer, const int32_t* ids, int n) {
  if (int rc = check_pool(p)) return rc;
  if (n < 0 || (n > 0 && !ids)) return fail(MOEQ_E_INVALID, "ids must hold n >= 0 host int32 values");
  std::vector<PoolCore::Step> steps;
  if (p->core.prefetch(layer, ids, n, steps) < 0)
    return fail(MOEQ_E_INVALID, "layer %d outside [0, %d) or an id outside [0, %d)", layer, p->core.n_layers,
                p->core.per_layer);
  if (steps.empty()) return ok();
  TableEdits ed{};
  std::vector<char> waited((size_t)p->core.n_layers, 0);
  for (const PoolCore::Step& st : steps) {
    // the slot's previous user must be done with it
    if (st.prev_layer >= 0 && p->released_valid[(size_t)st.prev_layer] && !waited[(size_t)st.prev_layer]) {
      const hipError_t e = hipStreamWaitEvent(p->copy[0], p->released[(size_t)st.prev_layer], 0);
      if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent (slot reuse)");
      waited[(size_t)st.prev_layer] = 1;
    }
    uint8_t* dst = p->arena + (int64_t)st.slot * p->slot_bytes;
    const hipError_t e = hipMemcpyAsync(dst, p->host[(size_t)st.entry], (size_t)p->expert_bytes,
                                        hipMemcpyHostToDevice, p->copy[0]);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (pool prefetch)");
    p->bytes_copied += p->expert_bytes;
    p->prefetched[(size_t)st.slot] = 1;
    if (st.evicted >= 0)
      if (int r = add_edit(p, ed, st.evicted, nullptr)) return r;
    if (int r = add_edit(p, ed, st.entry, dst)) return r;
  }
  if (int r = flush_edits(p, ed)) return r;
  // the next acquire's compute stream waits for these copies
  const hipError_t e = hipEventRecord(p->ready[0], p->copy[0]);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord (pool prefetch)");
  p->ready_valid[0] = 1;
  return ok();
}

int moe_pool_release(moeq_pool* p, int layer, void* compute_stream) {
  if (int rc = check_pool(p)) return rc;
  if (p->core.release(layer) < 0)
    return fail(MOEQ_E_INVALID, "layer %d outside [0, %d)", layer, p->core.n_layers);
  const hipError_t e = hipEventRecord(p->released[(size_t)layer], static_cast<hipStream_t>(compute_stream));
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord (pool release)");
  p->released_valid[(size_t)layer] = 1;
  return ok();
}

int moe_pool_stats(const moeq_pool* p, int64_t* out) {
  if (int rc = check_pool(p)) return rc;
  if (!out) return fail(MOEQ_E_INVALID, "out is NULL");
  out[0] = p->core.hits;
  out[1] = p->core.misses;
  out[2] = p->bytes_copied;
  out[3] = p->core.evictions;
  return ok();
}

void moe_pool_destroy(moeq_pool* p) {
  if (!p) return;
  for (hipStream_t c : p->copy) (void)hipStreamSynchronize(c);
  for (hipEvent_t ev : p->released)
    if (ev) (void)hipEventDestroy(ev);
  for (hipEvent_t ev : p->ready)
    if (ev) (void)hipEventDestroy(ev);
  delete p;
}

// ---------------------------------------------------- host-only bookkeeping

int moeq_poolsim_create(int n_layers, int per_layer, int64_t n_slots, moeq_poolsim** out) {
  if (!out) return fail(MOEQ_E_INVALID, "out is NULL");
  *out = nullptr;
  if (n_layers <= 0 || per_layer <= 0 || n_slots <= 0 || (int64_t)n_layers * per_layer > INT32_MAX)
    return fail(MOEQ_E_INVALID, "sizes must be positive (n_layers=%d per_layer=%d n_slots=%lld)", n_layers,
                per_layer, (long long)n_slots);
  moeq_poolsim* s = new moeq_poolsim;
  s->core.init(n_layers, per_layer, n_slots);
  *out = s;
  return ok();
}

int moeq_poolsim_make_resident(moeq_poolsim* s) {
  if (!s) return fail(MOEQ_E_INVALID, "pool is NULL");
  if (!s->core.make_resident()) return fail(MOEQ_E_UNSUPPORTED, "n_slots < n_layers * per_layer");
  return ok();
}

int moeq_poolsim_acquire(moeq_poolsim* s, int layer, const int32_t* ids, int n, int32_t* slots, int32_t* evicted,
                         int32_t* missed, int32_t* n_out) {
  if (!s) return fail(MOEQ_E_INVALID, "pool is NULL");
  if (n < 0 || (n > 0 && (!ids || !slots || !evicted || !missed)) || !n_out)
    return fail(MOEQ_E_INVALID, "ids/slots/evicted/missed must hold n entries, n_out non-NULL");
  std::vector<PoolCore::Step> steps;
  const int rc = s->core.acquire(layer, ids, n, steps);
  if (rc == -1) return fail(MOEQ_E_INVALID, "bad layer or id, or layer not released");
  if (rc == -2) return fail(MOEQ_E_POOL_EXHAUSTED, "not enough unpinned slots");
  for (size_t i = 0; i < steps.size(); ++i) {
    slots[i] = steps[i].slot;
    evicted[i] = steps[i].evicted;
    missed[i] = steps[i].miss ? 1 : 0;
  }
  *n_out = (int32_t)steps.size();
  return ok();
}

int moeq_poolsim_prefetch(moeq_poolsim* s, int layer, const int32_t* ids, int n, int32_t* slots,
                          int32_t* evicted, int32_t* n_out) {
  if (!s) return fail(MOEQ_E_INVALID, "pool is NULL");
  if (n < 0 || (n > 0 && (!ids || !slots || !evicted)) || !n_out)
    return fail(MOEQ_E_INVALID, "ids/slots/evicted must hold n entries, n_out non-NULL");
  std::vector<PoolCore::Step> steps;
  if (s->core.prefetch(layer, ids, n, steps) < 0) return fail(MOEQ_E_INVALID, "bad layer or id");
  for (size_t i = 0; i < steps.size(); ++i) {
    slots[i] = steps[i].slot;
    evicted[i] = steps[i].evicted;
  }
  *n_out = (int32_t)steps.size();
  return ok();
}

int moeq_poolsim_release(moeq_poolsim* s, int layer) {
  if (!s) return fail(MOEQ_E_INVALID, "pool is NULL");
  if (s->core.release(layer) < 0) return fail(MOEQ_E_INVALID, "layer %d out of range", layer);
  return ok();
}

int moeq_poolsim_stats(const moeq_poolsim* s, int64_t* out) {
  if (!s || !out) return fail(MOEQ_E_INVALID, "pool or out is NULL");
  out[0] = s->core.hits;
  out[1] = s->core.misses;
  out[2] = 0;
  out[3] = s->core.evictions;
  return ok();
}

void moeq_poolsim_destroy(moeq_poolsim* s) { delete s; }

}  // extern "C"
