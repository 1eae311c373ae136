"""GPU checks of the hand-off probe entry point (moeq_probe_handoff): every
pattern completes, reads no stale payload and, for the fixed-point
reduction, finds every accumulator's sum exact; argument errors are
reported before anything is launched."""
import pytest

import quantized_expert_gemv_router_amd as q
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

CASES = [
    # (mode, words per workgroup, stride, back-off, peer / copies / loads in flight)
    (0, 4, 4, 1, 1),     # tagged all-gather
    (0, 4, 64, 1, 1),    # strided writers
    (1, 4, 4, 1, 1),     # flag + payload
    (2, 1, 1, 1, 8),     # ping-pong with workgroup 8
    (3, 1, 1, 1, 1),     # counter barrier
    (4, 4, 4, 1, 8),     # gather to one + broadcast
    (5, 4, 4, 1, 8),     # ... + one read of the data
    (6, 4, 4, 1, 2),     # pipelined polls
    (7, 2, 4, 1, 1),     # fixed-point reduction, triple-buffered
]


@pytest.mark.parametrize("mode,w,stride,sleep,peer", CASES)
def test_probe_patterns_complete(mode, w, stride, sleep, peer):
    r = q.moeq_probe_handoff(mode, w, 40, sleep, peer, stride=stride)
    say(f"[probe] mode {mode} w={w} stride={stride}: {r['ticks'] * 0.01 / 40:.3f} us per round")
    assert r["ticks"] > 0
    assert r["stale"] == 0
    ids = r["xcc"]
    assert len(ids) > 0 and all(0 <= x < 64 for x in ids)


@pytest.mark.parametrize("mode,w,stride,peer", [
    (8, 1, 1, 1),        # no such pattern
    (7, 2, 2, 1),        # the reduction needs three buffers: stride >= 2 * words
    (0, 4, 2, 1),        # stride below the words per workgroup
    (2, 1, 1, 0),        # ping-pong with itself
])
def test_probe_rejects_bad_arguments(mode, w, stride, peer):
    with pytest.raises(q.MoeqError):
        q.moeq_probe_handoff(mode, w, 10, 1, peer, stride=stride)
