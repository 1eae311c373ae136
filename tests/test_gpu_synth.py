"""The device twin of the generator writes the same bytes as the host one."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import say, slot_stride

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "decode_4bit", "decode_2bit"])
def test_device_twin_matches_host(name):
    cfg = synth.CONFIGS[name]
    say(f"[synth twin] {name}")
    stride = slot_stride(cfg)
    first, count, layer = 5, 3, 2
    buf = torch.zeros(count * stride, dtype=torch.uint8, device="cuda")
    synth.device_fill_experts(cfg, layer, buf.data_ptr(), stride, first, count)
    torch.cuda.synchronize()
    dev = buf.cpu().numpy().reshape(count, stride)
    for i in range(count):
        host = synth.expert_blob(cfg, layer, first + i)
        assert np.array_equal(dev[i, :cfg.expert_bytes], host), (name, first + i)
