"""moe_q4_decode_static (no workspace argument: the library's static device
scratch) against moe_q4_decode with a caller workspace, through the C ABI:
bit-identical outputs on two calls in a row, the second with a smaller input
(the scratch keeps the first call's contents), and the size limit rejected
before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import quantized_moe_q4_amd as mq
import synth
from gpu_util import banner, experts_to_dev, np_of, to_dev

pytestmark = pytest.mark.gpu


def _inputs(seed, E, H, I, T, k):
    es = synth.expert_set(seed, 0, E, H, I)
    ex = experts_to_dev(es)
    xq, xd = mq.quantize_act(to_dev(synth.normal(seed, synth.x_tid(T), (T, H))))
    r = mq.route(to_dev(synth.normal(seed, synth.logits_tid(0, T), (T, E))), k)
    return ex, xq, xd, r


def test_decode_static_matches_decode_twice():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    mq.load_library()
    # first call: 40 tokens, 28 possible experts (expert-major down + combine, uses the o region); second: 3 tokens
    # of another layer shape (row-major down), smaller, over the first call's leftovers
    for seed, E, H, I, T, k, acc in ((91, 128, 2048, 512, 40, 8, False), (92, 16, 1024, 256, 3, 4, True)):
        banner(f"decode_static vs decode E={E} H={H} I={I} T={T} k={k} accumulate={acc}")
        ex, xq, xd, r = _inputs(seed, E, H, I, T, k)
        flags = mq.ACCUMULATE if acc else 0
        y0 = to_dev(synth.normal(seed, 77, (T, H)))
        y_ref, _ = mq.decode(ex, xq, xd, *r, flags=flags, y=y0.clone())
        y = mq.decode_static(ex, xq, xd, *r, flags=flags, y=y0.clone())
        torch.cuda.synchronize()
        np.testing.assert_array_equal(np_of(y), np_of(y_ref))


def test_decode_static_size_limit():
    mq.load_library()
    E, H, I, T, k = 16, 2048, 1024, 64, 16  # needs about 9.2 MB of workspace, above the 8 MiB scratch
    assert mq.workspace_size(T, E, k, H, I) > mq.STATIC_SCRATCH_BYTES
    ex, xq, xd, r = _inputs(93, E, H, I, T, k)
    y = torch.full((T, H), 3.0, dtype=torch.float32, device="cuda")
    with pytest.raises(mq.MoeQ4Error) as ei:
        mq.decode_static(ex, xq, xd, *r, y=y)
    assert ei.value.status == mq.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(y == 3.0).item()  # nothing was written
