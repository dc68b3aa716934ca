"""GPU parity of the one-launch decode (moe_q4_decode_fused).

Bar: bit-identical to the three-call path (quantize_act, route, decode) that
the oracle tests already pin, for every output (router outputs, hq/hd, y);
with the RMS pre-norm, whose fp64 row factor is summed in another order,
codes equal up to rounding-boundary cases and y within 1e-3 x RMS.  Plus the
oracle directly on the decode workload, repeated and graph-replayed calls (the
workspace's sync words must come back to zero every time) and an in-place
residual stack.
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


def _case(seed, E, H, I, T):
    es = synth.expert_set(seed, 0, E, H, I)
    x = synth.normal(seed, synth.x_tid(T), (T, H))
    lg = synth.normal(seed, synth.logits_tid(0, T), (T, E))
    return es, x, lg


def _three_calls(ex, x, lg, k, flags, y0=None):
    xq, xd = mq.quantize_act(x, flags=flags & mq.QUANT_RMSNORM)
    r = mq.route(lg, k)
    y = None if y0 is None else y0.clone()
    y, ws = mq.decode(ex, xq, xd, *r, flags=flags & mq.ACCUMULATE, y=y)
    return y, r, ws


def _ctl_words(ws):
    """(sum of the arrival and departure counters, error word) of a workspace's sync area."""
    words = np_of(ws[:mq.WS_ERROR_OFFSET + 4].view(torch.int32))
    return [int(words[:-1].sum()), int(words[-1])]


@pytest.mark.parametrize("E,H,I,T,k,flags", [
    (128, 2048, 512, 1, 8, 0),
    (128, 2048, 512, 4, 8, mq.ACCUMULATE),
    (128, 2048, 512, 8, 8, 0),
    (16, 256, 256, 3, 2, 0),
    (8, 512, 1024, 8, 8, mq.ACCUMULATE),   # T*k*I = 64 KB, the fused limit
    (300, 1024, 256, 2, 16, 0),            # E > 256: the 16-logits-per-lane router
    (5, 2048, 256, 2, 5, 0),
    (200, 2048, 512, 5, 3, 0),
    (6, 1024, 512, 4, 3, mq.ACCUMULATE),    # at most 8 experts, several pairs each: the quad down walk
    (128, 2048, 512, 1, 14, 0),            # tagged exchange with more items than resident gate/up workgroups
])
def test_fused_equals_three_calls(E, H, I, T, k, flags):
    banner(f"fused vs three calls E={E} H={H} I={I} T={T} k={k} flags={flags}")
    es, x, lg = _case(70 + E + T, E, H, I, T)
    ex = experts_to_dev(es)
    xd_, lgd = to_dev(x), to_dev(lg)
    y0 = to_dev(synth.normal(71, 5, (T, H))) if flags & mq.ACCUMULATE else None
    y_ref, r_ref, ws_ref = _three_calls(ex, xd_, lgd, k, flags, y0)
    ws = mq.new_workspace(T, E, k, H, I)
    y, r, ws = mq.decode_fused(ex, xd_, lgd, k, flags=flags, y=None if y0 is None else y0.clone(), ws=ws)
    torch.cuda.synchronize()
    for a, b, name in zip(r, r_ref, ("topk_ids", "topk_w", "offsets", "sorted")):
        np.testing.assert_array_equal(np_of(a), np_of(b), err_msg=name)
    hq, hd = mq.workspace_views(ws, T, k, I)
    hq_r, hd_r = mq.workspace_views(ws_ref, T, k, I)
    np.testing.assert_array_equal(np_of(hq), np_of(hq_r), err_msg="hq")
    np.testing.assert_array_equal(np_of(hd), np_of(hd_r), err_msg="hd")
    np.testing.assert_array_equal(np_of(y), np_of(y_ref), err_msg="y")
    assert _ctl_words(ws) == [0, 0]


def test_fused_oracle_workload1():
    w1 = synth.WORKLOADS[1]
    banner("fused decode workload 1 vs oracle (T=1, E=128, k=8)")
    es = synth.expert_set(w1.seed, 0, w1.E, w1.H, w1.I)
    x, lg = synth.activations(w1), synth.logits(w1)
    ex = experts_to_dev(es)
    y, (ids, w, off, sp), ws = mq.decode_fused(ex, to_dev(x), to_dev(lg), w1.k)
    torch.cuda.synchronize()
    xq_r, xd_r = oracle.q8_quantize(x)
    ids_r, w_r, off_r, sp_r = oracle.route(lg, w1.k)
    np.testing.assert_array_equal(np_of(ids), ids_r)
    np.testing.assert_array_equal(np_of(off), off_r)
    np.testing.assert_array_equal(np_of(sp), sp_r)
    y_ref, it = oracle.moe_layer(es, xq_r, xd_r, ids_r, w_r, want_intermediates=True)
    hq, hd = mq.workspace_views(ws, 1, w1.k, w1.I)
    hq_g, hd_g = to_pair_order(np_of(hq), np_of(sp)), to_pair_order(np_of(hd), np_of(sp))
    rec = check_requant(hq_g, hd_g, it, np.arange(w1.k), depth_decode(w1.H), "fused workload 1")
    y_cond = oracle.moe_layer(es, xq_r, xd_r, np_of(ids), np_of(w), hq_in=hq_g, hd_in=hd_g)
    err_c, rms_c = assert_close_rms(np_of(y), y_cond, "fused y (conditioned on GPU h)")
    err = float(np.max(np.abs(np_of(y).astype(np.float64) - y_ref)))
    rms = float(np.sqrt(np.mean(y_ref.astype(np.float64) ** 2)))
    rec.update(tokens=1, y_cond_err_over_rms=err_c / rms_c, y_uncond_err_over_rms=err / rms)
    report(rec)
    if rec["flips"] == 0:
        assert err <= 1e-3 * rms, f"fused y {err:.3e} > 1e-3 x RMS {rms:.3e}"


def test_fused_rmsnorm_close_to_three_calls():
    banner("fused rmsnorm vs three calls")
    E, H, I, T, k = 128, 2048, 512, 4, 8
    es, x, lg = _case(72, E, H, I, T)
    x *= np.float32(23.0)
    ex = experts_to_dev(es)
    flags = mq.QUANT_RMSNORM | mq.ACCUMULATE
    y0 = to_dev(synth.normal(72, 6, (T, H)))
    y_ref, r_ref, _ = _three_calls(ex, to_dev(x), to_dev(lg), k, flags, y0)
    y, r, ws = mq.decode_fused(ex, to_dev(x), to_dev(lg), k, flags=flags, y=y0.clone())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np_of(r[0]), np_of(r_ref[0]))
    assert_close_rms(np_of(y) - np_of(y0), np_of(y_ref) - np_of(y0), "fused rmsnorm: layer contribution")
    assert _ctl_words(ws) == [0, 0]


@pytest.mark.parametrize("batches", [(1,), (2,), (1, 2, 2, 1)], ids=["tagged", "counters", "mixed"])
def test_fused_back_to_back_calls(batches):
    """Many calls on one workspace without host synchronisation: each must find the sync area as the
    previous call left it.  T = 1 exchanges h through epoch-tagged words, T = 2 (k = 8, I = 512) through
    the arrival counters; the mixed sequence alternates the two on one workspace."""
    banner(f"fused back-to-back calls, batches {batches}")
    E, H, I, k = 128, 2048, 512, 8
    es = synth.expert_set(73, 0, E, H, I)
    ex = experts_to_dev(es)
    n = 24
    Ts = [batches[i % len(batches)] for i in range(n)]
    xs = [to_dev(synth.normal(73, 100 + i, (Ts[i], H))) for i in range(n)]
    lgs = [to_dev(synth.normal(73, 200 + i, (Ts[i], E))) for i in range(n)]
    ws = mq.new_workspace(max(Ts), E, k, H, I)
    ys = [mq.decode_fused(ex, xs[i], lgs[i], k, ws=ws)[0] for i in range(n)]
    torch.cuda.synchronize()
    assert _ctl_words(ws) == [0, 0]
    for i in (0, 1, 7, n - 1):
        y_ref, _, _ = _three_calls(ex, xs[i], lgs[i], k, 0)
        np.testing.assert_array_equal(np_of(ys[i]), np_of(y_ref), err_msg=f"call {i} (T={Ts[i]})")


@pytest.mark.parametrize("T", [1, 4], ids=["tagged", "counters-multi-item"])
def test_fused_graph_replays(T):
    """A captured graph of fused calls, replayed with eager work and synchronisations in between.  T = 4
    (464 gate/up items, more than the resident gate/up workgroups) takes several items per workgroup and the
    counter exchange."""
    banner(f"fused graph replays T={T}")
    E, H, I, k = 128, 2048, 512, 8
    es = synth.expert_set(74, 0, E, H, I)
    ex = experts_to_dev(es)
    n = 6
    xs = [to_dev(synth.normal(74, 300 + i, (T, H))) for i in range(n)]
    lgs = [to_dev(synth.normal(74, 400 + i, (T, E))) for i in range(n)]
    outs = [torch.empty((T, H), dtype=torch.float32, device="cuda") for _ in range(n)]
    ws = mq.new_workspace(T, E, k, H, I)
    eager = [np_of(_three_calls(ex, xs[i], lgs[i], k, 0)[0]) for i in range(n)]
    mq.decode_fused(ex, xs[0], lgs[0], k, y=outs[0], ws=ws)  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            mq.decode_fused(ex, xs[i], lgs[i], k, y=outs[i], ws=ws)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i in range(n):
            np.testing.assert_array_equal(np_of(outs[i]), eager[i], err_msg=f"replay {rep} call {i}")
        assert _ctl_words(ws) == [0, 0]
        _ = (xs[0] * 2).sum().item()  # unrelated eager work between replays


def test_fused_inplace_residual_stack():
    """y == x (residual stream updated in place) over several layers, against the three-call path."""
    banner("fused in-place residual stack")
    w4 = synth.WORKLOADS[4]
    H, I, E, k, T = w4.H, w4.I, w4.E, w4.k, 4
    h_f = to_dev(synth.normal(w4.seed, synth.x_tid(T), (T, H)))
    h_3 = h_f.clone()
    ws = mq.new_workspace(T, E, k, H, I)
    flags = mq.QUANT_RMSNORM | mq.ACCUMULATE
    for layer in range(3):
        ex = experts_to_dev(synth.expert_set(w4.seed, layer, E, H, I))
        lg = to_dev(synth.normal(w4.seed, synth.logits_tid(layer, T), (T, E)))
        h_in = np_of(h_f)
        mq.decode_fused(ex, h_f, lg, k, flags=flags, y=h_f, ws=ws)
        y3, _, _ = _three_calls(ex, to_dev(h_in), lg, k, flags, y0=to_dev(h_in))
        torch.cuda.synchronize()
        assert_close_rms(np_of(h_f) - h_in, np_of(y3) - h_in, f"in-place layer {layer}")
        h_3 = y3
    assert _ctl_words(ws) == [0, 0]
    assert np.all(np.isfinite(np_of(h_f)))
