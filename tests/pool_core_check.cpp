// Host-side check of the expert slot pool's placement policy (PoolCore),
// built by tests/test_pool_sim.py with AddressSanitizer and
// UndefinedBehaviorSanitizer.  Random acquire / prefetch / release streams
// over several pool sizes; after every step the structural invariants are
// checked against a separate, plainly written model of the same policy:
//   - every resident entry has exactly one slot and every slot one owner;
//   - acquired experts are resident and their slots pinned until release;
//   - a miss takes an empty slot if there is one, else the unpinned slot
//     used longest ago (ties to the lower index); pinned slots never move;
//   - hits + misses count the distinct ids of every acquire.
// Exit status 0 when every check holds; a message and status 1 otherwise.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "pool_core.hpp"

namespace {

struct Rng {
  uint64_t s;
  uint64_t next() {
    s += 0x9E3779B97F4A7C15ULL;
    uint64_t z = s;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
  }
  int below(int n) { return (int)(next() % (uint64_t)n); }
};

// The policy written out plainly: owner per slot, age per slot, pins.
struct Model {
  int n_layers, per;
  int64_t n_slots;
  std::vector<int32_t> owner;
  std::vector<uint64_t> age;
  std::vector<int> pins;
  std::vector<std::vector<int64_t>> held;
  uint64_t clock = 0;
  int64_t hits = 0, misses = 0;

  Model(int L, int P, int64_t S) : n_layers(L), per(P), n_slots(S), owner(S, -1), age(S, 0), pins(S, 0), held(L) {}

  int64_t find(int32_t entry) const {
    for (int64_t s = 0; s < n_slots; ++s)
      if (owner[s] == entry) return s;
    return -1;
  }
  int64_t victim(const std::vector<int64_t>& skip) const {
    for (int64_t s = 0; s < n_slots; ++s) {
      bool sk = false;
      for (int64_t k : skip) sk = sk || k == s;
      if (!sk && pins[s] == 0 && owner[s] < 0) return s;
    }
    int64_t best = -1;
    for (int64_t s = 0; s < n_slots; ++s) {
      bool sk = false;
      for (int64_t k : skip) sk = sk || k == s;
      if (sk || pins[s] != 0) continue;
      if (best < 0 || age[s] < age[best]) best = s;
    }
    return best;
  }
};

int fail(const char* what, int step) {
  std::fprintf(stderr, "pool_core_check: %s (step %d)\n", what, step);
  return 1;
}

int run(uint64_t seed, int L, int P, int64_t S, int steps) {
  moeq::PoolCore core;
  if (!core.init(L, P, S)) return fail("init", -1);
  Model m(L, P, S);
  Rng rng{seed};
  std::vector<moeq::PoolCore::Step> st;
  std::vector<char> active(L, 0);
  for (int step = 0; step < steps; ++step) {
    const int op = rng.below(10);
    const int layer = rng.below(L);
    if (op < 6) {   // acquire (if the layer is free), with duplicates
      if (active[layer]) continue;
      const int n = 1 + rng.below(std::min(P, 6));
      std::vector<int32_t> ids(n);
      for (auto& v : ids) v = rng.below(P);
      // model: distinct ids, first-appearance order
      std::vector<int32_t> uniq;
      for (int32_t v : ids) {
        bool seen = false;
        for (int32_t u : uniq) seen = seen || u == v;
        if (!seen) uniq.push_back(v);
      }
      int64_t need = 0, avail = 0;
      std::vector<char> hit(S, 0);
      for (int32_t u : uniq) {
        const int64_t s = m.find(layer * P + u);
        if (s >= 0) hit[s] = 1;
        else ++need;
      }
      for (int64_t s = 0; s < S; ++s)
        if (m.pins[s] == 0 && !hit[s]) ++avail;
      const int rc = core.acquire(layer, ids.data(), n, st);
      if (avail < need) {
        if (rc != -2) return fail("exhaustion not reported", step);
        continue;
      }
      if (rc != 0) return fail("acquire refused", step);
      ++m.clock;
      std::vector<int64_t> slot_of(uniq.size(), -1);
      for (size_t i = 0; i < uniq.size(); ++i) {   // hits first
        const int64_t s = m.find(layer * P + uniq[i]);
        if (s >= 0) {
          slot_of[i] = s;
          ++m.hits;
          ++m.pins[s];
          m.age[s] = m.clock;
          m.held[layer].push_back(s);
        }
      }
      for (size_t i = 0; i < uniq.size(); ++i) {   // then misses
        if (slot_of[i] >= 0) continue;
        const int64_t s = m.victim({});
        if (s < 0) return fail("model found no victim", step);
        m.owner[s] = layer * P + uniq[i];
        slot_of[i] = s;
        ++m.misses;
        ++m.pins[s];
        m.age[s] = m.clock;
        m.held[layer].push_back(s);
      }
      if (st.size() != uniq.size()) return fail("step count", step);
      for (size_t i = 0; i < uniq.size(); ++i) {
        if (st[i].entry != layer * P + uniq[i]) return fail("step order", step);
        if (st[i].slot != slot_of[i]) return fail("slot choice differs from the model", step);
      }
      active[layer] = 1;
    } else if (op < 8) {   // prefetch
      const int n = 1 + rng.below(std::min(P, 4));
      std::vector<int32_t> ids(n);
      for (auto& v : ids) v = rng.below(P);
      if (core.prefetch(layer, ids.data(), n, st) != 0) return fail("prefetch refused", step);
      ++m.clock;
      std::vector<int64_t> taken;
      size_t k = 0;
      for (int32_t v : ids) {
        const int64_t s0 = m.find(layer * P + v);
        if (s0 >= 0) {
          m.age[s0] = m.clock;
          continue;
        }
        const int64_t s = m.victim(taken);
        if (s < 0) break;
        m.owner[s] = layer * P + v;
        m.age[s] = m.clock;
        taken.push_back(s);
        if (k >= st.size() || st[k].slot != s || st[k].entry != layer * P + v)
          return fail("prefetch differs from the model", step);
        ++k;
      }
      if (k != st.size()) return fail("prefetch step count", step);
    } else {   // release
      if (!active[layer]) continue;
      const int64_t n = core.release(layer);
      if (n != (int64_t)m.held[layer].size()) return fail("release count", step);
      for (int64_t s : m.held[layer]) --m.pins[s];
      m.held[layer].clear();
      active[layer] = 0;
    }
    // invariants: the core's tables agree with the model
    for (int64_t s = 0; s < S; ++s) {
      if (core.owner[s] != m.owner[s]) return fail("owner table", step);
      if (core.pins[s] != m.pins[s]) return fail("pin counts", step);
      if (core.owner[s] >= 0 && core.where[core.owner[s]] != s) return fail("where/owner mismatch", step);
    }
    int64_t resident = 0;
    for (int64_t e = 0; e < (int64_t)L * P; ++e)
      if (core.where[e] >= 0) ++resident;
    int64_t owned = 0;
    for (int64_t s = 0; s < S; ++s) owned += core.owner[s] >= 0;
    if (resident != owned) return fail("an entry in two slots", step);
    if (core.hits != m.hits || core.misses != m.misses) return fail("hit/miss counts", step);
  }
  return 0;
}

}  // namespace

int main() {
  const int64_t sizes[][3] = {{2, 5, 3}, {3, 8, 6}, {4, 9, 16}, {6, 33, 24}, {2, 4, 8}};
  for (uint64_t seed = 1; seed <= 6; ++seed)
    for (const auto& z : sizes)
      if (int rc = run(seed * 7919, (int)z[0], (int)z[1], z[2], 4000)) return rc;
  std::printf("pool_core_check: ok\n");
  return 0;
}
