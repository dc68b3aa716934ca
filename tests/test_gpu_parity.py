"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Bar: integers (Q8_0 codes of the activations, routing ids, offsets, the
pair permutation, per-block int32 dots) bit-exact; Q8_0 codes of h equal up to
rounding-boundary cases; fp32 outputs within 1e-3 x the oracle RMS (max abs).
Large workloads are checked on sampled tokens that the oracle computes one by
one.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_moe_q4_amd as mq
import synth
from gpu_util import (assert_close_rms, banner, check_requant, depth_decode, depth_prefill, experts_to_dev, np_of,
                      oracle_layer_all, report, to_dev, to_pair_order)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    mq.load_library()  # fails loudly if the HIP library is missing
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------------ quantize
@pytest.mark.parametrize("rows,cols,scale", [(1, 2048, 1.0), (3, 64, 1.0), (947, 2048, 1.0), (5, 512, 1e-3),
                                             (2, 2048, 1e4), (0, 2048, 1.0)])
def test_quantize_act_bitexact(rows, cols, scale):
    banner(f"quantize rows={rows} cols={cols} scale={scale}")
    x = synth.normal(31, 7, (rows, cols)) * np.float32(scale)
    if rows >= 3:
        x[1] = 0.0  # all-zero row: d = 0, q = 0
    xq_ref, xd_ref = oracle.q8_quantize(x)
    xq, xd = mq.quantize_act(to_dev(x))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np_of(xq), xq_ref)
    np.testing.assert_array_equal(np_of(xd), xd_ref)


def test_quantize_act_golden_ties():
    banner("quantize golden tie blocks")
    x = np.array([[127, 0.5, 1.5, 2.5, -2.5, -127, 3.5, -0.5, -1.5, 0.25, 0.75, -0.75, 126.5, -126.5, 4.5, 5.5]
                  + [0] * 16, [254, 3, 5, 7, -9, 1, -1] + [0] * 25], np.float32)
    xq_ref, xd_ref = oracle.q8_quantize(x)
    xq, xd = mq.quantize_act(to_dev(x))
    np.testing.assert_array_equal(np_of(xq), xq_ref)
    np.testing.assert_array_equal(np_of(xd), xd_ref)
    assert np_of(xd).tolist() == [[1.0], [2.0]]


def test_quantize_act_rmsnorm():
    banner("quantize rmsnorm")
    x = synth.normal(32, 7, (64, 2048)) * np.float32(37.0)
    xq_ref, xd_ref = oracle.q8_quantize(x, flags=oracle.FLAG_RMSNORM)
    xq, xd = mq.quantize_act(to_dev(x), flags=mq.QUANT_RMSNORM)
    xq, xd = np_of(xq), np_of(xd)
    np.testing.assert_allclose(xd, xd_ref, rtol=1e-6)
    # the fp64 row sums differ only in summation order: codes equal up to boundary cases
    diff = xq.astype(np.int32) - xq_ref.astype(np.int32)
    assert np.abs(diff).max() <= 1 and (diff != 0).sum() <= 4


# ------------------------------------------------------------------ route
@pytest.mark.parametrize("T,E,k", [(1, 128, 8), (4, 128, 8), (947, 128, 8), (37, 4, 2), (5, 16, 16), (9, 1000, 1),
                                   (0, 64, 4), (3, 1, 1)])
def test_route_bitexact(T, E, k):
    banner(f"route T={T} E={E} k={k}")
    lg = synth.normal(33, 9, (T, E))
    if T > 2:
        lg[1, :] = lg[1, 0]              # every logit equal: ties broken by expert id
        lg[2, E // 4:E // 2] = lg[2, 0]  # a tied block
    ids_r, w_r, off_r, sp_r = oracle.route(lg, k)
    ids, w, off, sp = (np_of(t) for t in mq.route(to_dev(lg), k))
    np.testing.assert_array_equal(ids, ids_r)
    np.testing.assert_array_equal(off, off_r)
    np.testing.assert_array_equal(sp, sp_r)
    if T:
        assert np.max(np.abs(w.astype(np.float64) - w_r)) <= 1e-6
        assert np.all(np.abs(w.astype(np.float64).sum(axis=1) - 1.0) <= 1e-6)


@pytest.mark.parametrize("T,E,k", [(1, 16, 4), (3, 16, 4), (80, 16, 4), (2, 300, 8)])
def test_route_signed_zero_ties(T, E, k):
    """-0.0 and +0.0 are equal logits: a tie at the k-th slot goes to the lower expert id, whichever zero it
    carries (both the one-workgroup router for small T and the two-kernel router for large T)."""
    banner(f"route signed-zero ties T={T} E={E} k={k}")
    lg = np.full((T, E), -1.0, np.float32)
    lg[:, 0:k - 1] = np.arange(k - 1, 0, -1, dtype=np.float32)[None, :]  # k-1 clear winners
    lg[:, k + 1] = np.float32(-0.0)  # lower id, negative zero
    lg[:, k + 3] = np.float32(0.0)   # higher id, positive zero
    lg[1::2, k + 1] = np.float32(0.0)  # odd rows: the signs swapped
    lg[1::2, k + 3] = np.float32(-0.0)
    ids_r, w_r, off_r, sp_r = oracle.route(lg, k)
    assert np.all(ids_r[:, k - 1] == k + 1)  # the oracle's reading: equal logits, lower id
    ids, w, off, sp = (np_of(t) for t in mq.route(to_dev(lg), k))
    np.testing.assert_array_equal(ids, ids_r)
    np.testing.assert_array_equal(off, off_r)
    np.testing.assert_array_equal(sp, sp_r)
    assert np.max(np.abs(w.astype(np.float64) - w_r)) <= 1e-6


def test_quantize_act_subnormal_scales():
    """Blocks whose amax is below 127 * 2^-126, so d = amax / 127 is subnormal (and the code clamp can fire):
    codes and scales bit-exact, on the row kernel and the short-row kernel."""
    banner("quantize subnormal block scales")
    rng = np.random.default_rng(5)
    tiny = np.float32(2.0 ** -126)
    for cols in (2048, 96):
        x = (rng.standard_normal((4, cols)) * tiny).astype(np.float32)
        x[1] *= np.float32(1e-3)           # subnormal inputs too
        x[2, :32] = tiny * np.float32(127.4)  # amax just above the normal threshold in one block
        x[2, 32:64] = np.float32(2.0 ** -149)  # one-ulp values: d rounds to 0 -> all codes 0
        x[3, 5] = np.float32(1e-39)        # a lone subnormal element
        xq_ref, xd_ref = oracle.q8_quantize(x)
        assert np.any((xd_ref > 0) & (xd_ref < tiny)), "the case must reach subnormal scales"
        xq, xd = mq.quantize_act(to_dev(x))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(np_of(xq), xq_ref, err_msg=f"codes, cols={cols}")
        np.testing.assert_array_equal(np_of(xd).view(np.uint32), xd_ref.view(np.uint32), err_msg=f"scales, cols={cols}")


def test_route_skewed_workload3():
    w3 = synth.WORKLOADS[3]
    banner("route workload 3 (T=4096, E=256, Zipf bias)")
    lg = synth.logits(w3)
    ids_r, w_r, off_r, sp_r = oracle.route(lg, w3.k)
    ids, w, off, sp = (np_of(t) for t in mq.route(to_dev(lg), w3.k))
    np.testing.assert_array_equal(ids, ids_r)
    np.testing.assert_array_equal(off, off_r)
    np.testing.assert_array_equal(sp, sp_r)
    assert np.max(np.abs(w.astype(np.float64) - w_r)) <= 1e-6


def test_route_deterministic():
    banner("route determinism")
    lg = to_dev(synth.normal(34, 9, (947, 128)))
    a = [np_of(t) for t in mq.route(lg, 8)]
    b = [np_of(t) for t in mq.route(lg, 8)]
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# ------------------------------------------------------------------ block dots and GEMV (decode walk)
@pytest.mark.parametrize("N,K,T,down", [(512, 2048, 1, False), (96, 2048, 3, False), (64, 256, 5, False),
                                        (2048, 512, 2, True), (40, 256, 3, True), (32, 1024, 16, True)])
def test_decode_block_dots_bitexact(N, K, T, down):
    banner(f"decode block dots N={N} K={K} T={T} down={down}")
    qs, _ = synth.q4_matrix(35, 0, 0, synth.MAT_DOWN if down else synth.MAT_GATE, N, K)
    x = synth.normal(35, 3, (T, K))
    xq, xd = oracle.q8_quantize(x)
    # extreme activations in one row to reach the int32 range ends
    if T > 1:
        xq[1, :32] = 127
    ref = oracle.block_dots(qs, xq)
    got = np_of(mq.debug_block_dots(to_dev(qs), to_dev(xq), down_walk=down))
    np.testing.assert_array_equal(got, ref)


def test_gemv_workload0():
    banner("gemv workload 0 (512 x 2048)")
    qs, d = synth.gemv_matrix()
    x = synth.activations(synth.WORKLOADS[0])
    xq, xd = oracle.q8_quantize(x)
    ref = oracle.gemv(qs, d, xq, xd)
    xq_g, xd_g = mq.quantize_act(to_dev(x))
    np.testing.assert_array_equal(np_of(xq_g), xq)
    y = np_of(mq.gemv(to_dev(qs), to_dev(d), xq_g, xd_g))
    assert_close_rms(y, ref, "gemv y")


@pytest.mark.parametrize("T", [1, 7, 64])
def test_gemv_multi_token(T):
    banner(f"gemv T={T}")
    qs, d = synth.q4_matrix(36, 0, 1, synth.MAT_UP, 200, 1024)
    x = synth.normal(36, 3, (T, 1024))
    xq, xd = oracle.q8_quantize(x)
    ref = oracle.gemv(qs, d, xq, xd)
    y = np_of(mq.gemv(to_dev(qs), to_dev(d), to_dev(xq), to_dev(xd)))
    assert_close_rms(y, ref, "gemv y")


# ------------------------------------------------------------------ whole layer
def _layer_case(seed, E, H, I, T, k, zipf=False, identical=False):
    es = synth.expert_set(seed, 0, E, H, I)
    if identical:
        for a in (es.gate_qs, es.up_qs, es.down_qs, es.gate_d, es.up_d, es.down_d):
            a[:] = a[0]
    x = synth.normal(seed, synth.x_tid(T), (T, H))
    lg = (synth.biased_logits(seed, synth.logits_tid(0, T), T, E, -2.2) if zipf
          else synth.normal(seed, synth.logits_tid(0, T), (T, E)))
    return es, x, lg


def _run_layer(path, es, x, lg, k, flags=0, y0=None, dev_experts=None):
    """Quantize, route and run one layer on the GPU through the C ABI."""
    ex = experts_to_dev(es) if dev_experts is None else dev_experts
    xq, xd = mq.quantize_act(to_dev(x))
    ids, w, off, sp = mq.route(to_dev(lg), k)
    y = None if y0 is None else to_dev(y0)
    fn = mq.decode if path == "decode" else mq.prefill
    y, ws = fn(ex, xq, xd, ids, w, off, sp, flags=flags, y=y)
    torch.cuda.synchronize()
    T = x.shape[0]
    hq, hd = mq.workspace_views(ws, T, k, es.I)
    return dict(y=np_of(y), xq=np_of(xq), xd=np_of(xd), ids=np_of(ids), w=np_of(w), off=np_of(off), sp=np_of(sp),
                hq=np_of(hq), hd=np_of(hd), ex=ex)


def _check_layer(g, es, x, lg, k, tokens=None, flags=0, y0=None, what="", path="decode"):
    """S1 (activation codes), S2 (routing), S4 (h codes within the derived bound) and S6 (y conditioned on the
    GPU's own h, asserted; y against the fully independent oracle, always computed and reported)."""
    xq_r, xd_r = oracle.q8_quantize(x)
    np.testing.assert_array_equal(g["xq"], xq_r, err_msg=f"{what}: activation codes")
    np.testing.assert_array_equal(g["xd"], xd_r, err_msg=f"{what}: activation scales")
    ids_r, w_r, off_r, sp_r = oracle.route(lg, k)
    np.testing.assert_array_equal(g["ids"], ids_r, err_msg=f"{what}: topk ids")
    np.testing.assert_array_equal(g["sp"], sp_r, err_msg=f"{what}: sorted pairs")
    np.testing.assert_array_equal(g["off"], off_r, err_msg=f"{what}: offsets")
    assert np.max(np.abs(g["w"].astype(np.float64) - w_r)) <= 1e-6, f"{what}: topk weights"
    T = x.shape[0]
    rows = np.arange(T) if tokens is None else np.asarray(tokens)
    pairs = (rows[:, None] * k + np.arange(k)[None, :]).ravel()
    # independent oracle (its own h re-quantisation)
    y_ref, it = oracle_layer_all(es, xq_r, xd_r, ids_r, w_r, tokens=tokens, flags=flags, y0=y0,
                                 want_intermediates=True)
    hq_g = to_pair_order(g["hq"], g["sp"])
    hd_g = to_pair_order(g["hd"], g["sp"])
    depth = depth_prefill(es.H) if path == "prefill" else depth_decode(es.H)
    rec = check_requant(hq_g[pairs], hd_g[pairs], it, pairs, depth, what)
    # conditioned on the GPU's own re-quantised h: the down projection and combine
    y_cond = oracle_layer_all(es, xq_r, xd_r, g["ids"], g["w"], tokens=tokens, flags=flags, y0=y0, hq_in=hq_g,
                              hd_in=hd_g)
    err_c, rms_c = assert_close_rms(g["y"][rows], y_cond[rows], f"{what}: y (conditioned on GPU h)")
    ref = y_ref[rows].astype(np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = float(np.max(np.abs(g["y"][rows].astype(np.float64) - ref))) if ref.size else 0.0
    rec.update(tokens=int(rows.size), y_cond_err_over_rms=err_c / rms_c if rms_c else 0.0,
               y_uncond_err_over_rms=err / rms if rms else 0.0)
    report(rec)
    if rec["flips"] == 0:  # with identical h codes the two comparisons are the same one
        assert err <= 1e-3 * rms or (rms == 0.0 and err == 0.0), f"{what}: y {err:.3e} > 1e-3 x RMS {rms:.3e}"
    return rec["flips"]


@pytest.mark.parametrize("path", ["decode", "prefill"])
@pytest.mark.parametrize("E,H,I,T,k", [(8, 256, 256, 3, 2), (4, 512, 512, 1, 4), (16, 1024, 1024, 17, 4),
                                       (6, 256, 512, 64, 6), (5, 2048, 256, 2, 5), (3, 256, 256, 5, 1),
                                       # more than 16 active experts at T <= 16, at H = 256, 512 and 1024
                                       (64, 256, 256, 16, 4), (32, 512, 256, 16, 2), (40, 1024, 512, 9, 4)])
def test_layer_small(path, E, H, I, T, k):
    banner(f"layer {path} E={E} H={H} I={I} T={T} k={k}")
    es, x, lg = _layer_case(40 + E + T, E, H, I, T, k)
    g = _run_layer(path, es, x, lg, k)
    _check_layer(g, es, x, lg, k, what=f"{path} small", path=path)


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_layer_accumulate_and_zero_token(path):
    banner(f"layer {path} accumulate")
    E, H, I, T, k = 8, 512, 512, 5, 3
    es, x, lg = _layer_case(50, E, H, I, T, k)
    x[2] = 0.0
    y0 = synth.normal(50, 99, (T, H))
    g = _run_layer(path, es, x, lg, k, flags=mq.ACCUMULATE, y0=y0)
    _check_layer(g, es, x, lg, k, flags=oracle.FLAG_ACCUMULATE, y0=y0, what=f"{path} accumulate", path=path)
    g0 = _run_layer(path, es, x, lg, k)
    assert np.all(g0["y"][2] == 0.0)


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_layer_identical_experts(path):
    banner(f"layer {path} identical experts")
    E, H, I, T, k = 16, 512, 256, 9, 8
    es, x, lg = _layer_case(51, E, H, I, T, k, identical=True)
    g = _run_layer(path, es, x, lg, k)
    _check_layer(g, es, x, lg, k, what=f"{path} identical", path=path)
    # equals one expert with k = 1 (weights sum to 1)
    g1 = _run_layer(path, es, x, lg, 1)
    assert_close_rms(g["y"], g1["y"], f"{path}: identical experts vs k=1", tol=1e-5)


def test_decode_workload1():
    w1 = synth.WORKLOADS[1]
    banner("decode workload 1 (T=1, E=128, k=8)")
    es = synth.expert_set(w1.seed, 0, w1.E, w1.H, w1.I)
    x, lg = synth.activations(w1), synth.logits(w1)
    g = _run_layer("decode", es, x, lg, w1.k)
    _check_layer(g, es, x, lg, w1.k, what="workload 1")


@pytest.mark.parametrize("T", [4, 16, 64])
def test_decode_batches(T):
    banner(f"decode batch T={T} (E=128, k=8)")
    es = synth.expert_set(60, 0, 128, 2048, 512)
    x = synth.normal(60, synth.x_tid(T), (T, 2048))
    lg = synth.normal(60, synth.logits_tid(0, T), (T, 128))
    g = _run_layer("decode", es, x, lg, 8)
    _check_layer(g, es, x, lg, 8, what=f"decode T={T}")


def test_decode_deterministic_and_prefill_agrees():
    banner("decode determinism; prefill vs decode")
    es = synth.expert_set(61, 0, 32, 2048, 512)
    x = synth.normal(61, 1, (16, 2048))
    lg = synth.normal(61, 2, (16, 32))
    a = _run_layer("decode", es, x, lg, 8)
    b = _run_layer("decode", es, x, lg, 8, dev_experts=a["ex"])
    np.testing.assert_array_equal(a["y"], b["y"])
    np.testing.assert_array_equal(a["hq"], b["hq"])
    p = _run_layer("prefill", es, x, lg, 8, dev_experts=a["ex"])
    assert_close_rms(p["y"], a["y"], "prefill vs decode y")


# rows per expert: about 20 (one m-tile), about 90 (three m-tiles of one 96-row tile) and about 150 (a full
# 96-row tile and a partial one of two m-tiles), so these short launches, which take their row tiles costliest
# first, hold tiles of every class of that order
@pytest.mark.parametrize("E,H,I,T,k", [(6, 512, 256, 40, 3), (4, 512, 256, 120, 3), (3, 256, 256, 150, 3)])
def test_prefill_block_dots_bitexact(E, H, I, T, k):
    banner(f"prefill MFMA block dots E={E} H={H} I={I} T={T} k={k}")
    es, x, lg = _layer_case(62 + T, E, H, I, T, k)
    ex = experts_to_dev(es)
    xq, xd = mq.quantize_act(to_dev(x))
    ids, w, off, sp = mq.route(to_dev(lg), k)
    ws = torch.empty(mq.workspace_size(T, E, k, H, I), dtype=torch.uint8, device="cuda")
    gu = np_of(mq.debug_prefill_dots(ex, xq, xd, off, sp, k, 0, ws))
    dn = np_of(mq.debug_prefill_dots(ex, xq, xd, off, sp, k, 1, ws))
    hq, _ = mq.workspace_views(ws, T, k, I)
    hq, xqn, spn, idn = np_of(hq), np_of(xq), np_of(sp), np_of(ids)
    offn = np_of(off)
    for e in range(E):
        rows = np.arange(offn[e], offn[e + 1])
        if rows.size == 0:
            continue
        toks = spn[rows] // k
        np.testing.assert_array_equal(gu[rows, 0], oracle.block_dots(es.gate_qs[e], xqn[toks]), err_msg=f"gate e={e}")
        np.testing.assert_array_equal(gu[rows, 1], oracle.block_dots(es.up_qs[e], xqn[toks]), err_msg=f"up e={e}")
        np.testing.assert_array_equal(dn[rows], oracle.block_dots(es.down_qs[e], hq[rows]), err_msg=f"down e={e}")
        assert np.all(idn.ravel()[spn[rows]] == e)


def test_prefill_workload2():
    """T=947, E=128, k=8: every token against the oracle (split over host threads)."""
    w2 = synth.WORKLOADS[2]
    banner("prefill workload 2 (T=947, E=128, k=8), all tokens")
    es = synth.expert_set(w2.seed, 0, w2.E, w2.H, w2.I)
    x, lg = synth.activations(w2), synth.logits(w2)
    g = _run_layer("prefill", es, x, lg, w2.k)
    _check_layer(g, es, x, lg, w2.k, what="workload 2 (all tokens)", path="prefill")


def test_prefill_workload3_skewed():
    """T=4096, E=256, k=8, Zipf-skewed: every token against the oracle (split over host threads)."""
    w3 = synth.WORKLOADS[3]
    banner("prefill workload 3 (T=4096, E=256, k=8, Zipf-skewed), all tokens")
    es = synth.expert_set(w3.seed, 0, w3.E, w3.H, w3.I)
    x, lg = synth.activations(w3), synth.logits(w3)
    g = _run_layer("prefill", es, x, lg, w3.k)
    _check_layer(g, es, x, lg, w3.k, what="workload 3 (all tokens)", path="prefill")


def test_prefill_deterministic():
    """The prefill combine sums each token's pairs in slot order: two runs give the same bits."""
    E, H, I, T, k = 64, 1024, 512, 300, 6
    banner(f"prefill run-to-run E={E} H={H} I={I} T={T} k={k}")
    es = synth.expert_set(97, 0, E, H, I)
    ex = experts_to_dev(es)
    x = to_dev(synth.normal(97, 1, (T, H)))
    lg = to_dev(synth.normal(97, 2, (T, E)))
    xq, xd = mq.quantize_act(x)
    r = mq.route(lg, k)
    y0 = to_dev(synth.normal(97, 3, (T, H)))
    ys = [mq.prefill(ex, xq, xd, *r, flags=mq.ACCUMULATE, y=y0.clone())[0] for _ in range(3)]
    torch.cuda.synchronize()
    for yy in ys[1:]:
        np.testing.assert_array_equal(np_of(yy), np_of(ys[0]))


@pytest.mark.parametrize("T", [1, 4, 16])
def test_stack40_per_layer(T):
    """40-layer stack, pre-norm + residual; each layer checked against the oracle given the GPU's layer input."""
    w4 = synth.WORKLOADS[4]
    banner(f"stack of 40 layers, T={T}")
    H, I, E, k = w4.H, w4.I, w4.E, w4.k
    h = to_dev(synth.normal(w4.seed, synth.x_tid(T), (T, H)))
    check_layers = {0, 1, 19, 39}
    for layer in range(w4.layers):
        es = synth.expert_set(w4.seed, layer, E, H, I)
        ex = experts_to_dev(es)
        lg_np = synth.normal(w4.seed, synth.logits_tid(layer, T), (T, E))
        h_in = np_of(h)
        xq, xd = mq.quantize_act(h, flags=mq.QUANT_RMSNORM)
        ids, w, off, sp = mq.route(to_dev(lg_np), k)
        h, ws = mq.decode(ex, xq, xd, ids, w, off, sp, flags=mq.ACCUMULATE, y=h)
        torch.cuda.synchronize()
        if layer in check_layers:
            xq_r, xd_r = oracle.q8_quantize(h_in, flags=oracle.FLAG_RMSNORM)
            diff = np_of(xq).astype(np.int32) - xq_r.astype(np.int32)
            assert np.abs(diff).max() <= 1 and (diff != 0).sum() <= 2
            hq, hd = mq.workspace_views(ws, T, k, I)
            y_cond = oracle.moe_layer(es, np_of(xq), np_of(xd), np_of(ids), np_of(w), flags=oracle.FLAG_ACCUMULATE,
                                      y=h_in.copy(), hq_in=to_pair_order(np_of(hq), np_of(sp)),
                                      hd_in=to_pair_order(np_of(hd), np_of(sp)))
            # compare the layer's contribution (y - residual), the quantity the layer computes
            assert_close_rms(np_of(h) - h_in, y_cond.astype(np.float64) - h_in, f"stack layer {layer} T={T}")
        del ex
    assert np.all(np.isfinite(np_of(h)))
