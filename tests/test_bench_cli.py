"""bench.py's command line, on the CPU: it measures one GPU and says so for
any other count before touching a device, and its workloads are listed."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = _bench("--gpus", n, "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "measures one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_workloads():
    r = _bench("--help")
    assert r.returncode == 0
    for w in ("stack60_decode", "decode_4bit", "decode_3bit", "decode_2bit", "batch16_top10", "stack60_prefill",
              "pool_decode"):
        assert w in r.stdout, w
