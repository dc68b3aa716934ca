"""GPU parity of the batched one-launch layer stack (moe_q4_decode_stack_batch).

Bar: every layer's hidden state and h codes are bit-identical to the
three-call chain (quantize_act, route, decode per layer) that the oracle tests
pin, since both run the same arithmetic (with the pre-norm too: its fp64 sum of
squares is formed in quantize_act's order); with the pre-norm each layer is
also checked against the oracle given the GPU's own layer input: h codes within
the derived bound, the layer's contribution within 1e-3 x RMS conditioned on
the GPU's h (and reported unconditioned).  Plus repeated calls on one workspace
(the tags advance, the error word stays 0), odd shapes, and the 40-layer
workload at batch 16.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_moe_q4_amd as mq
import synth
from gpu_util import (assert_close_rms, banner, check_requant, depth_decode, experts_to_dev, np_of, report, to_dev,
                      to_pair_order)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    mq.load_library()
    yield
    torch.cuda.synchronize()


def _layers(seed, L, E, H, I, distinct=None):
    n = L if distinct is None else distinct
    sets = [synth.expert_set(seed, l, E, H, I) for l in range(n)]
    dev = [experts_to_dev(es) for es in sets]
    return [sets[l % n] for l in range(L)], [dev[l % n] for l in range(L)]


def _inputs(seed, L, T, E, H):
    h0 = synth.normal(seed, synth.x_tid(T), (T, H))
    lg = np.stack([synth.normal(seed, synth.logits_tid(l, T), (T, E)) for l in range(L)])
    return h0, lg


def _batch(layers, h0, lg, k, flags, ws=None):
    L, T = lg.shape[0], lg.shape[1]
    E, H, I = layers[0].E, layers[0].H, layers[0].I
    h = to_dev(h0)
    h_all = torch.empty((L, T, H), dtype=torch.float32, device="cuda")
    hq_all = torch.empty((L, T * k, I), dtype=torch.int8, device="cuda")
    hd_all = torch.empty((L, T * k, I // 32), dtype=torch.float32, device="cuda")
    h, ws = mq.decode_stack_batch(layers, h, to_dev(lg), k, flags=flags, h_all=h_all, hq_all=hq_all, hd_all=hd_all,
                                  ws=ws)
    torch.cuda.synchronize()
    return np_of(h), np_of(h_all), np_of(hq_all), np_of(hd_all), ws


def _three_call_chain(layers, h0, lg, k, flags):
    """quantize_act + route + decode per layer on the device; returns h after each layer, h codes/scales and the
    routing of each layer."""
    h = to_dev(h0)
    hs, hqs, hds, routes = [], [], [], []
    T = h0.shape[0]
    I = layers[0].I
    for l, ex in enumerate(layers):
        xq, xd = mq.quantize_act(h, flags=flags & mq.QUANT_RMSNORM)
        r = mq.route(to_dev(lg[l]), k)
        h, ws = mq.decode(ex, xq, xd, *r, flags=flags & mq.ACCUMULATE, y=h if flags & mq.ACCUMULATE else None)
        hq, hd = mq.workspace_views(ws, T, k, I)
        hs.append(np_of(h).copy())
        hqs.append(np_of(hq).copy())
        hds.append(np_of(hd).copy())
        routes.append([np_of(t) for t in r])
    torch.cuda.synchronize()
    return np.stack(hs), np.stack(hqs), np.stack(hds), routes


def _err_word(ws):
    return int(np_of(ws[mq.WS_ERROR_OFFSET:mq.WS_ERROR_OFFSET + 4].view(torch.int32))[0])


@pytest.mark.parametrize("E,H,I,T,k,L", [
    (128, 2048, 512, 16, 8, 3),
    (128, 2048, 512, 4, 8, 2),
    (128, 2048, 512, 1, 8, 2),
    (32, 2048, 512, 7, 6, 3),
    (8, 1024, 256, 5, 8, 2),      # every expert active, I = 256
    (64, 1024, 1024, 9, 3, 2),    # I = 1024 (two blocks per down lane)
    (300, 2048, 512, 16, 1, 2),   # k = 1, E > 256
])
def test_batch_equals_three_calls(E, H, I, T, k, L):
    """Residual stack without the pre-norm: bit-identical to the three-call chain, layer by layer."""
    banner(f"stack batch vs three calls E={E} H={H} I={I} T={T} k={k} L={L}")
    sets, layers = _layers(100 + E + T, L, E, H, I)
    h0, lg = _inputs(100 + T, L, T, E, H)
    flags = mq.ACCUMULATE
    h, h_all, hq_all, hd_all, ws = _batch(layers, h0, lg, k, flags)
    assert _err_word(ws) == 0
    hs_ref, hq_ref, hd_ref, _ = _three_call_chain(layers, h0, lg, k, flags)
    np.testing.assert_array_equal(hq_all, hq_ref, err_msg="h codes")
    np.testing.assert_array_equal(hd_all, hd_ref, err_msg="h scales")
    np.testing.assert_array_equal(h_all, hs_ref, err_msg="hidden state after each layer")
    np.testing.assert_array_equal(h, hs_ref[-1], err_msg="h_L")


@pytest.mark.parametrize("T,L", [(16, 3), (3, 2)])
def test_batch_rmsnorm_vs_oracle_per_layer(T, L):
    """Pre-norm residual stack: each layer against the oracle, given the GPU's layer input."""
    w4 = synth.WORKLOADS[4]
    E, H, I, k = w4.E, w4.H, w4.I, w4.k
    banner(f"stack batch rmsnorm vs oracle per layer T={T} L={L}")
    sets, layers = _layers(w4.seed, L, E, H, I)
    h0, lg = _inputs(w4.seed + T, L, T, E, H)
    flags = mq.QUANT_RMSNORM | mq.ACCUMULATE
    h, h_all, hq_all, hd_all, ws = _batch(layers, h0, lg, k, flags)
    assert _err_word(ws) == 0
    h_in = h0
    for l in range(L):
        xq_r, xd_r = oracle.q8_quantize(h_in, oracle.FLAG_RMSNORM)
        ids_r, w_r, off_r, sp_r = oracle.route(lg[l], k)
        hq_g = to_pair_order(hq_all[l], sp_r)
        hd_g = to_pair_order(hd_all[l], sp_r)
        y_ref, it = oracle.moe_layer(sets[l], xq_r, xd_r, ids_r, w_r, want_intermediates=True)
        rec = check_requant(hq_g, hd_g, it, np.arange(T * k), depth_decode(H), f"stack batch T={T} layer {l}")
        y_cond = oracle.moe_layer(sets[l], xq_r, xd_r, ids_r, w_r, hq_in=hq_g, hd_in=hd_g)
        contrib = h_all[l].astype(np.float64) - h_in.astype(np.float64)
        err_c, rms_c = assert_close_rms(contrib, y_cond, f"layer {l} contribution (conditioned on GPU h)")
        rms = float(np.sqrt(np.mean(y_ref.astype(np.float64) ** 2)))
        rec.update(tokens=T, y_cond_err_over_rms=err_c / rms_c,
                   y_uncond_err_over_rms=float(np.max(np.abs(contrib - y_ref))) / rms)
        report(rec)
        h_in = h_all[l]
    np.testing.assert_array_equal(h, h_all[-1])


@pytest.mark.parametrize("E,H,I,T,k,L", [
    (128, 2048, 512, 16, 8, 4),
    (128, 2048, 512, 3, 8, 3),
    (64, 1024, 1024, 9, 3, 2),    # H = 1024: one float4 per thread in quantize_act's sum
])
def test_batch_rmsnorm_equals_three_calls(E, H, I, T, k, L):
    """With the pre-norm: the whole chain bit-identical to the three-call chain, layer by layer (every layer's
    fp64 sum of squares in quantize_act's order)."""
    banner(f"stack batch rmsnorm vs three calls E={E} H={H} I={I} T={T} k={k} L={L}")
    sets, layers = _layers(131 + T, L, E, H, I)
    h0, lg = _inputs(131 + T, L, T, E, H)
    flags = mq.QUANT_RMSNORM | mq.ACCUMULATE
    h, h_all, hq_all, hd_all, ws = _batch(layers, h0, lg, k, flags)
    assert _err_word(ws) == 0
    hs_ref, hq_ref, hd_ref, _ = _three_call_chain(layers, h0, lg, k, flags)
    np.testing.assert_array_equal(hq_all, hq_ref, err_msg="h codes")
    np.testing.assert_array_equal(hd_all, hd_ref, err_msg="h scales")
    np.testing.assert_array_equal(h_all, hs_ref, err_msg="hidden state after each layer")
    np.testing.assert_array_equal(h, hs_ref[-1], err_msg="h_L")


def test_batch_repeated_calls_share_workspace():
    """Back-to-back calls on one workspace without host synchronisation, different inputs: each equals a
    call on a fresh workspace; the error word stays clear."""
    E, H, I, T, k, L = 64, 2048, 512, 6, 4, 3
    banner("stack batch repeated calls on one workspace")
    sets, layers = _layers(141, L, E, H, I)
    ws = mq.new_stack_batch_workspace(L, T, E, k, H, I)
    outs = []
    for rep in range(4):
        h0, lg = _inputs(141 + rep, L, T, E, H)
        h = to_dev(h0)
        mq.decode_stack_batch(layers, h, to_dev(lg), k, flags=mq.ACCUMULATE | mq.QUANT_RMSNORM, ws=ws)
        outs.append((h0, lg, h))
    torch.cuda.synchronize()
    assert _err_word(ws) == 0
    for h0, lg, h in outs:
        ref, *_ = _batch(layers, h0, lg, k, mq.ACCUMULATE | mq.QUANT_RMSNORM)
        np.testing.assert_array_equal(np_of(h), ref)


def test_batch_full_workload_40_layers_T16():
    """The 40-layer stack at batch 16 with the pre-norm residual, as bench.py times it.  Each layer against the
    three-call path run on the same layer input (the batched kernel's own h_l): identical h codes and hidden
    state, and the contribution within 1e-3 x RMS (reported)."""
    w4 = synth.WORKLOADS[4]
    E, H, I, k, L, T = w4.E, w4.H, w4.I, w4.k, w4.layers, 16
    banner(f"stack batch 40 layers T={T}")
    _, layers = _layers(w4.seed, L, E, H, I, distinct=6)
    h0, lg = _inputs(w4.seed, L, T, E, H)
    flags = mq.QUANT_RMSNORM | mq.ACCUMULATE
    h, h_all, hq_all, hd_all, ws = _batch(layers, h0, lg, k, flags)
    assert _err_word(ws) == 0
    assert np.all(np.isfinite(h_all))
    identical = 0
    for l in range(L):
        h_in = h0 if l == 0 else h_all[l - 1]
        hs_ref, hq_ref, hd_ref, _ = _three_call_chain([layers[l]], h_in, lg[l:l + 1], k, flags)
        contrib = h_all[l].astype(np.float64) - h_in.astype(np.float64)
        contrib_ref = hs_ref[0].astype(np.float64) - h_in.astype(np.float64)
        assert_close_rms(contrib, contrib_ref, f"layer {l} contribution vs three calls on the same input")
        identical += int(np.array_equal(h_all[l], hs_ref[0]) and np.array_equal(hq_all[l], hq_ref[0]))
    report({"what": "stack batch 40 layers T=16", "layers_bit_identical_to_three_calls": identical, "layers": L})
    assert identical == L, f"{L - identical} layers differ from the three-call path on the same input"
    np.testing.assert_array_equal(h, h_all[-1])
