// Host-side bookkeeping of the expert slot pool: which (layer, expert) sits
// in which device slot, which slots the layers in flight hold, and which
// slot a miss evicts.  No device calls; moe_pool_* drive the copies and the
// pointer-table updates from the plans made here, and moeq_poolsim_* expose
// the same object for host-only tests.
//
// The policy follows openclawradar.com/fr (Flash-MoE write-up, caching of
// experts): a bounded set of resident slots filled on router demand, the
// least recently used one evicted first.  A layer's slots stay pinned from
// its acquire until its release, so a running layer never loses an expert.
#pragma once

#include <cstdint>
#include <vector>

namespace moeq {

struct PoolCore {
  // What one acquire decided for one requested expert.
  struct Step {
    int32_t entry;    // layer * per_layer + expert
    int32_t slot;
    int32_t evicted;  // entry whose slot this miss took, or -1
    int32_t prev_layer;  // layer that acquired the slot before, or -1
    bool miss;
  };

  int32_t n_layers = 0, per_layer = 0;
  int64_t n_slots = 0;
  std::vector<int32_t> owner;               // [n_slots] entry or -1
  std::vector<int64_t> where;               // [n_layers * per_layer] slot or -1
  std::vector<uint64_t> last_tick;          // [n_slots] tick of the last acquire
  std::vector<int32_t> pins;                // [n_slots] layers holding the slot
  std::vector<int32_t> last_layer;          // [n_slots] layer of the last acquire, or -1
  std::vector<std::vector<int64_t>> held;   // [n_layers] slots pinned by the layer
  uint64_t tick = 0;
  int64_t hits = 0, misses = 0, evictions = 0, prefetches = 0;

  bool init(int32_t layers, int32_t per, int64_t slots) {
    if (layers <= 0 || per <= 0 || slots <= 0) return false;
    n_layers = layers;
    per_layer = per;
    n_slots = slots;
    owner.assign((size_t)slots, -1);
    where.assign((size_t)layers * per, -1);
    last_tick.assign((size_t)slots, 0);
    pins.assign((size_t)slots, 0);
    last_layer.assign((size_t)slots, -1);
    held.assign((size_t)layers, {});
    return true;
  }

  // Identity residency: entry i in slot i.  Needs n_slots >= entries.
  bool make_resident() {
    const int64_t entries = (int64_t)n_layers * per_layer;
    if (n_slots < entries) return false;
    for (int64_t s = 0; s < n_slots; ++s) {
      if (owner[(size_t)s] >= 0) where[(size_t)owner[(size_t)s]] = -1;
      owner[(size_t)s] = -1;
    }
    for (int64_t i = 0; i < entries; ++i) {
      owner[(size_t)i] = (int32_t)i;
      where[(size_t)i] = i;
    }
    return true;
  }

  // Plans an acquire of `ids` (duplicates count once) for `layer`.  Returns
  // 0 and fills `steps` in first-appearance order, -1 for a bad id or a
  // layer that already holds slots (released first), -2 when the misses
  // need more slots than are neither pinned nor requested here (nothing
  // changes then).
  int acquire(int32_t layer, const int32_t* ids, int n, std::vector<Step>& steps) {
    steps.clear();
    if (layer < 0 || layer >= n_layers || n < 0) return -1;
    if (!held[(size_t)layer].empty()) return -1;
    std::vector<int32_t> uniq;
    for (int i = 0; i < n; ++i) {
      const int32_t id = ids[i];
      if (id < 0 || id >= per_layer) return -1;
      bool seen = false;
      for (int32_t u : uniq) seen = seen || u == id;
      if (!seen) uniq.push_back(id);
    }
    // capacity: slots a miss may take are those neither pinned nor hit here
    std::vector<char> hit_here((size_t)n_slots, 0);
    int64_t need = 0;
    for (int32_t id : uniq) {
      const int64_t s = where[(size_t)layer * per_layer + id];
      if (s >= 0) hit_here[(size_t)s] = 1;
      else ++need;
    }
    int64_t avail = 0;
    for (int64_t s = 0; s < n_slots && avail < need; ++s)
      if (pins[(size_t)s] == 0 && !hit_here[(size_t)s]) ++avail;
    if (avail < need) return -2;

    ++tick;
    // hits are pinned first so that no miss of this call evicts them
    steps.resize(uniq.size());
    for (int pass = 0; pass < 2; ++pass) {
      for (size_t u = 0; u < uniq.size(); ++u) {
        const int32_t entry = layer * per_layer + uniq[u];
        int64_t s = where[(size_t)entry];
        if ((pass == 0) != (s >= 0)) continue;
        Step st{entry, -1, -1, -1, false};
        if (s >= 0) {
          ++hits;
        } else {
          s = victim();
          st.miss = true;
          ++misses;
          if (owner[(size_t)s] >= 0) {
            st.evicted = owner[(size_t)s];
            where[(size_t)owner[(size_t)s]] = -1;
            ++evictions;
          }
          owner[(size_t)s] = entry;
          where[(size_t)entry] = s;
        }
        st.slot = (int32_t)s;
        st.prev_layer = last_layer[(size_t)s];
        ++pins[(size_t)s];
        last_tick[(size_t)s] = tick;
        last_layer[(size_t)s] = layer;
        held[(size_t)layer].push_back(s);
        steps[u] = st;
      }
    }
    return 0;
  }

  // Plans a prefetch of `ids` for `layer`: each id not resident takes a
  // victim slot (empty first, else least recently used; never a pinned slot
  // or one this call already took) and is marked resident but not pinned;
  // resident ids are only touched (they become most recently used).  Stops
  // quietly when no slot is left.  Fills `steps` with the copies to make
  // (miss = true).  Returns 0, or -1 for a bad layer or id.
  int prefetch(int32_t layer, const int32_t* ids, int n, std::vector<Step>& steps) {
    steps.clear();
    if (layer < 0 || layer >= n_layers || n < 0) return -1;
    for (int i = 0; i < n; ++i)
      if (ids[i] < 0 || ids[i] >= per_layer) return -1;
    ++tick;
    std::vector<int64_t> taken;
    for (int i = 0; i < n; ++i) {
      const int32_t entry = layer * per_layer + ids[i];
      const int64_t s0 = where[(size_t)entry];
      if (s0 >= 0) {
        last_tick[(size_t)s0] = tick;
        continue;
      }
      const int64_t s = victim_excluding(taken);
      if (s < 0) break;
      Step st{entry, (int32_t)s, -1, last_layer[(size_t)s], true};
      if (owner[(size_t)s] >= 0) {
        st.evicted = owner[(size_t)s];
        where[(size_t)owner[(size_t)s]] = -1;
        ++evictions;
      }
      owner[(size_t)s] = entry;
      where[(size_t)entry] = s;
      last_tick[(size_t)s] = tick;
      ++prefetches;
      taken.push_back(s);
      steps.push_back(st);
    }
    return 0;
  }

  // Unpins the slots `layer` holds.  Returns how many.
  int64_t release(int32_t layer) {
    if (layer < 0 || layer >= n_layers) return -1;
    const int64_t n = (int64_t)held[(size_t)layer].size();
    for (int64_t s : held[(size_t)layer]) --pins[(size_t)s];
    held[(size_t)layer].clear();
    return n;
  }

 private:
  // As victim(), skipping the slots in `skip`; -1 if none is left.
  int64_t victim_excluding(const std::vector<int64_t>& skip) const {
    int64_t best = -1;
    for (int64_t s = 0; s < n_slots; ++s) {
      if (pins[(size_t)s] != 0) continue;
      bool skipped = false;
      for (int64_t k : skip) skipped = skipped || k == s;
      if (skipped) continue;
      if (owner[(size_t)s] < 0) return s;
      if (best < 0 || last_tick[(size_t)s] < last_tick[(size_t)best]) best = s;
    }
    return best;
  }

  // An empty slot if any (lowest index), else the unpinned slot acquired
  // longest ago (lowest index on equal ticks).  The caller checked that one
  // exists.
  int64_t victim() const {
    int64_t best = -1;
    for (int64_t s = 0; s < n_slots; ++s) {
      if (pins[(size_t)s] != 0) continue;
      if (owner[(size_t)s] < 0) return s;
      if (best < 0 || last_tick[(size_t)s] < last_tick[(size_t)best]) best = s;
    }
    return best;
  }
};

}  // namespace moeq
