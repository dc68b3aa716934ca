"""The measurement probes run and leave their sink untouched on ordinary data
(the sink is written only when a result hits a fixed constant)."""
import pytest
import torch

import quantized_moe_q4_amd as mq
from gpu_util import banner

pytestmark = pytest.mark.gpu


def test_probe_read_and_mfma():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    mq.load_library()
    banner("probes: streaming read, int8 MFMA loop")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for n in (16, 4096 + 48, 1 << 22):   # one load, a ragged tail, many workgroups
        buf = torch.zeros(n, dtype=torch.uint8, device="cuda")
        assert mq.probe_read(buf, sink) == n
    assert mq.probe_mfma_i8(4, 8, sink) == 262144 * 4 * 4 * 8
    fsink = torch.zeros(1, dtype=torch.float32, device="cuda")
    assert mq.probe_w4a8_step(4, 8, fsink) == 131072 * 4 * 4 * 8
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    assert float(fsink.item()) == 0.0
