"""GPU parity of the router projection (moe_q4_router_logits) against the oracle.

Bar (fp32, derived from the arithmetic): every logit within the recursive-summation bound
H * 2^-24 * sum_h |x_n[h] * w[h]| of the oracle's (an exact fp64 sum rounded once), plus one fp32 rounding;
with the pre-norm the bound is taken on the normalised row.  Routing from the GPU logits must pick the same
experts as routing from the oracle's logits on every token whose k-th and (k+1)-th largest logits are
further apart than twice that bound (elsewhere either choice is correct).
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_moe_q4_amd as mq
import synth
from gpu_util import banner, np_of, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    mq.load_library()
    yield
    torch.cuda.synchronize()


def _bound(x, wr, flags):
    xn = x.astype(np.float64)
    if flags & mq.QUANT_RMSNORM:
        xn = xn / np.sqrt((xn ** 2).mean(axis=1, keepdims=True) + 1e-6)
    H = x.shape[1]
    return H * 2.0 ** -24 * (np.abs(xn) @ np.abs(wr.astype(np.float64)).T)


def _check(x, wr, flags, k, got, rows=None):
    rows = np.arange(x.shape[0]) if rows is None else rows
    ref = oracle.router_logits(x[rows], wr, flags).astype(np.float64)
    bound = _bound(x[rows], wr, flags) + np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    err = np.abs(got[rows].astype(np.float64) - ref)
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3f}"
    # routing agreement away from near-ties at the k-th boundary
    srt = np.sort(ref, axis=1)[:, ::-1]
    clear = (srt[:, k - 1] - srt[:, k]) > 2 * bound.max(axis=1)
    ids_gpu = oracle.route(got[rows], k)[0]
    ids_ref = oracle.route(ref.astype(np.float32), k)[0]
    np.testing.assert_array_equal(ids_gpu[clear], ids_ref[clear])
    return int(clear.sum())


@pytest.mark.parametrize("T,H,E,flags", [
    (1, 2048, 128, 0),                      # decode
    (4, 2048, 128, 1),                      # decode batch, pre-norm
    (16, 512, 64, 0),                       # the largest batch of the one-wave-per-expert kernel
    (17, 1024, 96, 0),                      # tiled kernel: ragged token and expert tiles
    (100, 256, 300, 1),
    (947, 2048, 128, 1),                    # the 947-token prefill
    (40, 160, 70, 1),                       # H not a multiple of 64: 32-wide K chunks
    (600, 96, 40, 0),                       # 16 x 32 tiles with 32-wide K chunks
    (4096, 224, 256, 1),                    # 32 x 32 tiles with 32-wide K chunks
    (8192, 224, 256, 0),                    # 64 x 64 tiles with 32-wide K chunks
])
def test_router_logits(T, H, E, flags):
    banner(f"router logits T={T} H={H} E={E} flags={flags}")
    x = synth.normal(90 + T, synth.x_tid(T), (T, H))
    wr = synth.router_weights(90, 0, E, H)
    got = np_of(mq.router_logits(to_dev(x), to_dev(wr), flags=flags))
    torch.cuda.synchronize()
    _check(x, wr, flags, min(8, E - 1), got)


@pytest.mark.parametrize("T", [4096, 8192])
def test_router_logits_skewed_prefill_shape_sampled(T):
    """The 4096-token, 256-expert shape in the launch configuration the bench times (32 x 32 tiles, 128-wide
    K chunks), and twice the tokens (64 x 64 tiles, 64-wide chunks); the oracle on 64 rows."""
    H, E = 2048, 256
    banner(f"router logits T={T} H={H} E={E} (sampled rows)")
    x = synth.normal(95, synth.x_tid(T), (T, H))
    wr = synth.router_weights(95, 0, E, H)
    got = np_of(mq.router_logits(to_dev(x), to_dev(wr), flags=mq.QUANT_RMSNORM))
    torch.cuda.synchronize()
    rows = np.unique(np.linspace(0, T - 1, 64).astype(int))
    _check(x, wr, mq.QUANT_RMSNORM, 8, got, rows)


def test_router_logits_zero_rows_and_deterministic():
    banner("router logits: zero rows, empty batch, determinism")
    T, H, E = 40, 512, 64
    x = synth.normal(96, 1, (T, H))
    x[[0, 17, 39]] = 0.0
    wr = synth.router_weights(96, 0, E, H)
    xd, wd = to_dev(x), to_dev(wr)
    a = np_of(mq.router_logits(xd, wd, flags=mq.QUANT_RMSNORM))
    b = np_of(mq.router_logits(xd, wd, flags=mq.QUANT_RMSNORM))
    assert np.all(a[[0, 17, 39]] == 0.0)
    np.testing.assert_array_equal(a, b)
    out = torch.empty((0, E), dtype=torch.float32, device="cuda")
    mq.router_logits(torch.empty((0, H), dtype=torch.float32, device="cuda"), wd, out=out)
