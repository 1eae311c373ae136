"""Host-side checks of the expert pool's placement and eviction policy
(moeq_poolsim_*, the same policy object moe_pool_* uses), and of the pool
entry points' argument validation.  No GPU needed.

The policy: a bounded set of slots filled on demand, least recently
acquired unpinned slot evicted first (openclawradar.com/fr, Flash-MoE
write-up on expert caching).  A small independent model of that policy is
written out below and driven with the same seeded request streams.
"""
import ctypes
import os
import random

import pytest

import quantized_expert_gemv_router_amd as q
from quantized_expert_gemv_router_amd import _binding as B


class LruModel:
    """Plain restatement of the policy: empty slots first (lowest index),
    else the unpinned slot whose last acquire is oldest (lowest index on
    ties); hits of a request are pinned before its misses are placed."""

    def __init__(self, layers, per, slots):
        self.per, self.n = per, slots
        self.owner = [None] * slots
        self.last = [0] * slots
        self.pins = [0] * slots
        self.held = {l: [] for l in range(layers)}
        self.tick = 0
        self.hits = self.misses = self.evictions = 0

    def where(self, entry):
        return self.owner.index(entry) if entry in self.owner else None

    def acquire(self, layer, ids):
        uniq = list(dict.fromkeys(ids))
        entries = [layer * self.per + i for i in uniq]
        need = sum(self.where(e) is None for e in entries)
        hit_slots = {self.where(e) for e in entries} - {None}
        free = [s for s in range(self.n) if self.pins[s] == 0 and s not in hit_slots]
        if len(free) < need:
            return None
        self.tick += 1
        out = {}
        for e in entries:                       # hits first
            s = self.where(e)
            if s is not None:
                self.hits += 1
                self.pins[s] += 1
                self.last[s] = self.tick
                self.held[layer].append(s)
                out[e] = (s, -1, False)
        for e in entries:
            if e in out:
                continue
            cands = [s for s in range(self.n) if self.pins[s] == 0]
            empty = [s for s in cands if self.owner[s] is None]
            s = empty[0] if empty else min(cands, key=lambda c: (self.last[c], c))
            ev = self.owner[s] if self.owner[s] is not None else -1
            if ev >= 0:
                self.evictions += 1
            self.misses += 1
            self.owner[s] = e
            self.pins[s] += 1
            self.last[s] = self.tick
            self.held[layer].append(s)
            out[e] = (s, ev, True)
        return [out[e] for e in entries]

    def release(self, layer):
        for s in self.held[layer]:
            self.pins[s] -= 1
        self.held[layer] = []


@pytest.mark.parametrize("seed,layers,per,slots,k", [(0, 4, 9, 6, 3), (1, 6, 17, 20, 4), (2, 3, 513, 40, 11),
                                                     (3, 8, 5, 5, 2)])
def test_policy_matches_model(seed, layers, per, slots, k):
    rng = random.Random(seed)
    sim, ref = q.PoolSim(layers, per, slots), LruModel(layers, per, slots)
    active = []
    for _ in range(400):
        idle = [l for l in range(layers) if l not in active]
        if active and (not idle or rng.random() < 0.45):
            l = active.pop(rng.randrange(len(active)))
            sim.release(l)
            ref.release(l)
            continue
        l = rng.choice(idle)
        ids = [rng.randrange(per) for _ in range(k)] + [per - 1]   # last id plays the shared expert
        want = ref.acquire(l, ids)
        if want is None:
            with pytest.raises(q.MoeqError) as ei:
                sim.acquire(l, ids)
            assert ei.value.code == B.E_POOL_EXHAUSTED
            continue
        assert sim.acquire(l, ids) == want
        active.append(l)
    st = sim.stats()
    assert (st["hits"], st["misses"], st["evictions"]) == (ref.hits, ref.misses, ref.evictions)


def test_duplicates_count_once_and_hit_after():
    sim = q.PoolSim(2, 8, 4)
    assert sim.acquire(0, [3, 3, 5, 3]) == [(0, -1, True), (1, -1, True)]
    sim.release(0)
    assert sim.acquire(0, [5, 3]) == [(1, -1, False), (0, -1, False)]
    assert sim.stats() == dict(hits=2, misses=2, bytes_copied=0, evictions=0)


def test_hit_later_in_request_is_not_evicted():
    sim = q.PoolSim(2, 4, 2)
    sim.acquire(0, [0])            # slot 0, older
    sim.release(0)
    sim.acquire(1, [1])            # slot 1, newer
    sim.release(1)
    # the miss (id 2) comes first in the request, but slot 0 holds id 0 which
    # this request hits: the miss must take slot 1
    assert sim.acquire(0, [2, 0]) == [(1, 1 * 4 + 1, True), (0, -1, False)]


def test_pinned_slots_survive_and_exhaustion_changes_nothing():
    sim = q.PoolSim(3, 6, 3)
    sim.acquire(0, [0, 1])
    with pytest.raises(q.MoeqError) as ei:
        sim.acquire(1, [0, 1])     # needs 2 new slots, only 1 unpinned
    assert ei.value.code == B.E_POOL_EXHAUSTED
    assert sim.stats()["misses"] == 2
    assert sim.acquire(1, [4]) == [(2, -1, True)]
    sim.release(1)
    sim.release(0)
    # LRU: slot 0 and 1 were acquired at tick 1, slot 2 at tick 2
    assert sim.acquire(2, [5, 4]) == [(0, 0 * 6 + 0, True), (1, 0 * 6 + 1, True)]


def test_acquire_twice_and_bad_ids_are_refused():
    sim = q.PoolSim(2, 4, 8)
    sim.acquire(0, [1])
    for layer, ids in ((0, [2]), (1, [4]), (1, [-1]), (2, [0])):
        with pytest.raises(q.MoeqError) as ei:
            sim.acquire(layer, ids)
        assert ei.value.code == B.E_INVALID


def test_make_resident_is_identity_and_all_hits():
    sim = q.PoolSim(3, 5, 15)
    sim.make_resident()
    for l in range(3):
        got = sim.acquire(l, [4, 0, 2])
        assert got == [(l * 5 + 4, -1, False), (l * 5 + 0, -1, False), (l * 5 + 2, -1, False)]
        sim.release(l)
    assert sim.stats()["misses"] == 0
    small = q.PoolSim(3, 5, 14)
    with pytest.raises(q.MoeqError) as ei:
        small.make_resident()
    assert ei.value.code == B.E_UNSUPPORTED


def test_pool_create_validates_before_touching_a_device():
    L = B.lib()
    shape = q.Shape(256, 128, 8, 1, 4, 64)
    h = ctypes.c_void_p()
    blobs = (ctypes.c_void_p * 18)(*[0x2000 + i * 55296 for i in range(18)])
    streams = (ctypes.c_void_p * 1)(None)
    args = dict(n_layers=2, arena=0x1000, n_slots=4, slot_bytes=55296, host=ctypes.cast(blobs, ctypes.c_void_p),
                table=0x3000, streams=ctypes.cast(streams, ctypes.c_void_p), n_streams=1)

    def create(**kw):
        a = dict(args, **kw)
        return L.moe_pool_create(ctypes.byref(shape), a["n_layers"], a["arena"], a["n_slots"],
                                 a["slot_bytes"], a["host"], a["table"], a["streams"], a["n_streams"],
                                 ctypes.byref(h))

    assert create(arena=None) == B.E_INVALID
    assert create(table=None) == B.E_INVALID
    assert create(host=None) == B.E_INVALID
    assert create(n_slots=0) == B.E_INVALID
    assert create(n_layers=0) == B.E_INVALID
    assert create(slot_bytes=55296 - 256) == B.E_INVALID     # below the expert size
    assert create(slot_bytes=55296 + 8) == B.E_INVALID       # not a multiple of 256
    assert create(n_streams=0) == B.E_INVALID                # at least one copy stream
    assert create(n_streams=9) == B.E_INVALID                # at most eight
    assert create(streams=None) == B.E_INVALID
    bad = q.Shape(256, 128, 8, 1, 5, 64)
    assert L.moe_pool_create(ctypes.byref(bad), 2, 0x1000, 4, 55296, args["host"], 0x3000, args["streams"], 1,
                             ctypes.byref(h)) == B.E_UNSUPPORTED
    assert h.value is None
    # the stats, release and acquire calls refuse a NULL pool
    out = (ctypes.c_int64 * 4)()
    assert L.moe_pool_stats(None, out) == B.E_INVALID
    assert L.moe_pool_release(None, 0, None) == B.E_INVALID
    L.moe_pool_destroy(None)


def test_prefetch_makes_a_later_acquire_hit_and_never_takes_pinned_slots():
    """Prefetched experts become resident unpinned (a later acquire of them is
    a hit); resident ones are only touched; a prefetch never evicts a slot a
    layer holds and stops quietly when no unpinned slot is left."""
    sim = q.PoolSim(2, 8, 6)
    assert [s for s, _ in sim.prefetch(0, [1, 2, 3])] == [0, 1, 2]
    got = sim.acquire(0, [1, 2, 4])
    assert [m for _, _, m in got] == [False, False, True]
    st = sim.stats()
    assert (st["hits"], st["misses"]) == (2, 1)
    # layer 0 pins slots 0, 1 (hits) and 3 (miss); three slots are unpinned
    plan = sim.prefetch(1, [0, 1, 2, 3, 4])
    assert len(plan) == 3 and {s for s, _ in plan} == {2, 4, 5}
    assert all(s not in (0, 1, 3) for s, _ in plan)
    # slot 2 held layer 0's prefetched expert 3, which is evicted
    assert (2, 0 * 8 + 3) in plan
    sim.release(0)
    # an id already resident is touched, not copied
    assert sim.prefetch(1, [0]) == []
    with pytest.raises(q.MoeqError):
        sim.prefetch(2, [0])
    with pytest.raises(q.MoeqError):
        sim.prefetch(0, [8])


def test_prefetch_touch_protects_from_eviction():
    """A resident expert named in a prefetch becomes most recently used, so
    the next miss evicts another slot."""
    sim = q.PoolSim(1, 8, 2)
    sim.acquire(0, [0])
    sim.release(0)
    sim.acquire(0, [1])
    sim.release(0)
    sim.prefetch(0, [0])            # touch expert 0: expert 1 is now the oldest
    got = sim.acquire(0, [2])
    assert got[0][1] == 1           # expert 1's slot was evicted


def test_pool_core_under_address_and_ub_sanitizers(tmp_path):
    """The pool's placement policy (pool_core.hpp), built for the host with
    AddressSanitizer and UndefinedBehaviorSanitizer, driven through random
    acquire / prefetch / release streams and checked step by step against a
    separately written model of the policy (tests/pool_core_check.cpp)."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    here = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(os.path.dirname(here), "quantized_expert_gemv_router_amd", "csrc")
    exe = str(tmp_path / "pool_core_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", csrc, os.path.join(here, "pool_core_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitize" in r.stderr:
        pytest.skip(f"sanitizer runtime unavailable: {r.stderr[:200]}")
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stderr[-2000:]
    assert "ok" in run.stdout
