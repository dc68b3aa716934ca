"""CPU tests of the parity checker's derived bound (tests/gpu_util.check_requant).

An fp32 evaluation of the layer's h along another summation order (the shape
of what the GPU kernels do) must pass; a planted wrong code away from a
rounding boundary, or a wrong scale, must fail.  The GPU tests rely on this
checker, so it is pinned here without a GPU.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_requant, depth_decode, depth_prefill


def _fp32_h(es, xq, xd, ids, k, order_seed, chain):
    """h of every pair in fp32: block terms fl(d_w/16 * d_a) * 16 isum accumulated in a shuffled order, one
    rounding per step (chain=True: one sequential chain; False: 8 chains of 8 blocks and a tree of 8), then
    SwiGLU in fp32 and the Q8_0 requantisation of R2 in fp32."""
    rng = np.random.default_rng(order_seed)
    T = xq.shape[0]
    H, I = es.H, es.I
    nb = H // 32
    hs, hq, hd = [], [], []
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            out = []
            for W, D in ((es.gate_qs[e], es.gate_d[e]), (es.up_qs[e], es.up_d[e])):
                isum = oracle.block_dots(W, xq[t:t + 1])[0].astype(np.float32)  # [I][nb]
                dw = (D.view(np.float16).astype(np.float32) / np.float32(16.0))
                sc = (dw * xd[t][None, :]).astype(np.float32)
                terms = (np.float32(16.0) * isum) * sc  # exact product of the rounded scale, rounded once
                perm = rng.permutation(nb)
                if chain:
                    acc = np.zeros(I, np.float32)
                    for b in perm:
                        acc = (acc + terms[:, b]).astype(np.float32)
                else:
                    parts = []
                    for lane in range(8):
                        a = np.zeros(I, np.float32)
                        for b in perm[lane::8]:
                            a = (a + terms[:, b]).astype(np.float32)
                        parts.append(a)
                    while len(parts) > 1:
                        parts = [(parts[i] + parts[i + 1]).astype(np.float32) for i in range(0, len(parts), 2)]
                    acc = parts[0]
                out.append(acc)
            g, u = out
            h = (g / (np.float32(1.0) + np.exp(-g).astype(np.float32)) * u).astype(np.float32)
            q, d = oracle.q8_quantize(h[None, :])
            hs.append(h)
            hq.append(q[0])
            hd.append(d[0])
    return np.array(hs), np.array(hq), np.array(hd)


@pytest.mark.parametrize("chain", [True, False])
def test_fp32_reordered_evaluation_passes(chain):
    E, k, H, I, T = 6, 3, 2048, 64, 4
    es = synth.expert_set(81, 0, E, H, I)
    x = synth.normal(81, 1, (T, H))
    lg = synth.normal(81, 2, (T, E))
    ids, w, _, _ = oracle.route(lg, k)
    xq, xd = oracle.q8_quantize(x)
    _, it = oracle.moe_layer(es, xq, xd, ids, w, want_intermediates=True)
    depth = depth_prefill(H) if chain else depth_decode(H)
    for seed in range(3):
        _, hq, hd = _fp32_h(es, xq, xd, ids, k, seed, chain)
        rec = check_requant(hq, hd, it, np.arange(T * k), depth, "fp32 reordered")
        assert rec["window_max"] < 0.05


def test_planted_code_and_scale_errors_fail():
    E, k, H, I, T = 4, 2, 512, 64, 3
    es = synth.expert_set(82, 0, E, H, I)
    x = synth.normal(82, 1, (T, H))
    lg = synth.normal(82, 2, (T, E))
    ids, w, _, _ = oracle.route(lg, k)
    xq, xd = oracle.q8_quantize(x)
    _, it = oracle.moe_layer(es, xq, xd, ids, w, want_intermediates=True)
    pairs = np.arange(T * k)
    hq, hd = it["hq"].copy(), it["hd"].copy()
    check_requant(hq, hd, it, pairs, depth_decode(H), "identical")
    # a code moved by one where h/d is far from a half-integer
    r = it["h"].astype(np.float64) / np.repeat(it["hd"].astype(np.float64), 32, axis=1)
    far = np.argwhere(np.abs(np.abs(r - np.floor(r)) - 0.5) > 0.2)
    p, n = far[0]
    bad = hq.copy()
    bad[p, n] = np.int8(int(bad[p, n]) + (1 if bad[p, n] < 127 else -1))
    with pytest.raises(AssertionError, match="outside the derived window"):
        check_requant(bad, hd, it, pairs, depth_decode(H), "planted code")
    # a scale off by 1e-4 relative
    bad_d = hd.copy()
    bad_d[0, 0] *= np.float32(1.0001)
    with pytest.raises(AssertionError, match="scales differ"):
        check_requant(hq, bad_d, it, pairs, depth_decode(H), "planted scale")
