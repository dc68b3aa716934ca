"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Every check here compares the oracle with something it does not compute
itself: hand-derived fixtures (tests/golden), exhaustive integer brute force,
closed forms, library routines (numpy dense products, stable argsort, scipy's
softmax) and a pure-Python brute force of a whole tiny layer.  A plausible
slip anywhere in the oracle (a dropped term, a flipped sign, a wrong nibble
or slot index, a transposed operand) breaks at least one of them.
"""
import os

import numpy as np
import pytest
import scipy.special

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield [c.strip() for c in line.split("|")]


def _f16_value(bits: int) -> float:
    return float(np.array([bits], np.uint16).view(np.float16)[0])


def _np_dequant(qs: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Independent numpy reading of the Q4_0 layout (pinned by the golden blocks below)."""
    rows = qs.shape[0]
    blocks = qs.reshape(rows, -1, 16)
    lo = (blocks & 0x0F).astype(np.int64)
    hi = (blocks >> 4).astype(np.int64)
    q = np.concatenate([lo, hi], axis=2) - 8  # [rows][nb][32]
    scale = d.view(np.float16).astype(np.float64)[:, :, None]
    return (q * scale).reshape(rows, -1)


def _np_q8(x: np.ndarray):
    """numpy Q8_0 on fp32 data (pinned by the golden activation blocks below)."""
    x = x.astype(np.float32)
    b = x.reshape(x.shape[0], -1, 32)
    amax = np.abs(b).max(axis=2)
    d = (amax / np.float32(127)).astype(np.float32)
    safe = np.where(d == 0, np.float32(1), d)
    q = np.clip(np.rint(b / safe[:, :, None]), -127, 127)
    q = np.where(d[:, :, None] == 0, 0, q).astype(np.int8)
    return q.reshape(x.shape), d


# ----------------------------------------------------------------- Q4_0
def test_q4_golden_blocks():
    n = 0
    for name, dhex, bhex, vals in _rows("q4_0_hand_blocks.txt"):
        bits = int(dhex, 16)
        qs = np.frombuffer(bytes.fromhex(bhex), np.uint8).reshape(1, 16).copy()
        d = np.array([[bits]], np.uint16)
        expect = np.array([int(v) for v in vals.split()], np.float64) * _f16_value(bits)
        got = oracle.q4_dequant(qs, d)[0]
        np.testing.assert_array_equal(got, expect, err_msg=name)
        np.testing.assert_array_equal(_np_dequant(qs, d)[0], expect, err_msg=name)
        n += 1
    assert n == 5


def test_q4_endpoints_closed_form():
    # q = 0 -> -8d, q = 15 -> 7d, q = 8 -> 0 for every finite positive fp16 scale tried
    for bits in (0x0001, 0x03FF, 0x0400, 0x1E8C, 0x2148, 0x3C00, 0x7BFF):
        dval = _f16_value(bits)
        assert oracle.half_to_double(bits) == dval
        for byte, lo, hi in ((0x00, -8, -8), (0xFF, 7, 7), (0x88, 0, 0), (0x0F, 7, -8), (0xF0, -8, 7)):
            qs = np.full((1, 16), byte, np.uint8)
            w = oracle.q4_dequant(qs, np.array([[bits]], np.uint16))[0]
            assert np.all(w[:16] == lo * dval) and np.all(w[16:] == hi * dval)


def test_q4_random_matrix_vs_numpy_layout():
    qs, d = synth.q4_matrix(11, 0, 3, synth.MAT_DOWN, 64, 256)
    np.testing.assert_array_equal(oracle.q4_dequant(qs, d), _np_dequant(qs, d))


# ----------------------------------------------------------------- Q8_0
def test_q8_golden_blocks():
    n = 0
    for name, dstr, xs, qs in _rows("q8_0_hand_blocks.txt"):
        x = np.array([[float(v) for v in xs.split()]], np.float32)
        xq, xd = oracle.q8_quantize(x)
        assert xd[0, 0] == np.float32(float(dstr)), name
        np.testing.assert_array_equal(xq[0], np.array([int(v) for v in qs.split()], np.int8), err_msg=name)
        nq, nd = _np_q8(x)
        np.testing.assert_array_equal(nq, xq, err_msg=name)
        n += 1
    assert n == 5


def test_q8_power_of_two_scaling_invariance():
    x = synth.normal(5, 77, (16, 256))
    xq0, xd0 = oracle.q8_quantize(x)
    for e in (-20, -3, 1, 7, 30):
        s = np.float32(2.0 ** e)
        xq, xd = oracle.q8_quantize(x * s)
        np.testing.assert_array_equal(xq, xq0)
        np.testing.assert_array_equal(xd, xd0 * s)


def test_q8_properties_random():
    x = synth.normal(6, 78, (64, 2048)) * np.float32(3.0)
    xq, xd = oracle.q8_quantize(x)
    b = x.reshape(64, -1, 32).astype(np.float64)
    q = xq.reshape(64, -1, 32).astype(np.float64)
    d = xd.astype(np.float64)[:, :, None]
    # the element of largest magnitude maps to +-127, all codes in [-127, 127]
    assert np.all(np.abs(q).max(axis=2) == 127)
    assert xq.min() >= -127
    # round-to-nearest: |x - q d| <= d/2 up to the two fp32 divisions' rounding
    assert np.all(np.abs(b - q * d) <= d * (0.5 + 1e-6))
    nq, nd = _np_q8(x)
    np.testing.assert_array_equal(nq, xq)
    np.testing.assert_array_equal(nd, xd)


def test_q8_rmsnorm_closed_forms():
    # constant row c: mean(x^2) = c^2, so every element becomes c / sqrt(c^2 + 1e-6)
    c = np.float32(3.0)
    x = np.full((1, 64), c, np.float32)
    xq, xd = oracle.q8_quantize(x, flags=oracle.FLAG_RMSNORM)
    v = float(c) / np.sqrt(float(c) ** 2 + 1e-6)
    assert xd[0, 0] == np.float32(np.float32(v) / np.float32(127))
    assert np.all(xq == 127)
    # normalised random rows have mean square ~ 1 (checked through dequantised values)
    x = synth.normal(7, 79, (8, 2048)) * np.float32(50.0)
    xq, xd = oracle.q8_quantize(x, flags=oracle.FLAG_RMSNORM)
    deq = xq.reshape(8, -1, 32).astype(np.float64) * xd[:, :, None]
    ms = (deq.reshape(8, -1) ** 2).mean(axis=1)
    assert np.all(np.abs(ms - 1.0) < 2e-2)
    # the zero row stays zero
    xq, xd = oracle.q8_quantize(np.zeros((1, 32), np.float32), flags=oracle.FLAG_RMSNORM)
    assert np.all(xq == 0) and np.all(xd == 0)


# ----------------------------------------------------------------- block dots
def test_block_dot_exhaustive_single_terms():
    """All 16 x 255 (nibble, int8) pairs, each placed alone in a block at varying positions."""
    qs_rows, acts, expect = [], [], []
    for q in range(16):
        for a in range(-127, 128):
            pos = (q * 7 + a) % 32
            blk = np.full(16, 0x88, np.uint8)  # all weights zero (q = 8)
            i = pos % 16
            if pos < 16:
                blk[i] = (blk[i] & 0xF0) | q
            else:
                blk[i] = (blk[i] & 0x0F) | (q << 4)
            act = np.zeros(32, np.int8)
            act[pos] = a
            qs_rows.append(blk)
            acts.append(act)
            expect.append((q - 8) * a)
    qs = np.array(qs_rows, np.uint8)           # [4080][16]: one block per row
    xq = np.array(acts, np.int8)               # [4080][32]
    # evaluate row r against activation row r only: diagonal of the full product
    got = np.array([oracle.block_dots(qs[r:r + 1], xq[r:r + 1])[0, 0, 0] for r in range(len(expect))])
    np.testing.assert_array_equal(got, np.array(expect))


def test_block_dot_extremes():
    qs = np.zeros((1, 16), np.uint8)          # every q = 0 -> weight -8
    xq = np.full((1, 32), 127, np.int8)
    assert oracle.block_dots(qs, xq)[0, 0, 0] == -32512
    qs = np.full((1, 16), 0xFF, np.uint8)     # every q = 15 -> weight 7
    xq = np.full((1, 32), -127, np.int8)
    assert oracle.block_dots(qs, xq)[0, 0, 0] == -28448
    xq = np.full((1, 32), 127, np.int8)
    assert oracle.block_dots(qs, xq)[0, 0, 0] == 28448


def test_block_dot_random_identity():
    """sum (q-8) a == sum q a - 8 sum a, computed from raw nibbles by numpy."""
    qs, _ = synth.q4_matrix(12, 0, 1, synth.MAT_GATE, 48, 64)
    a = (synth.u64(12, 999, 5 * 64).astype(np.int64) % 255 - 127).astype(np.int8).reshape(5, 64)
    got = oracle.block_dots(qs, a)  # [5][48][2]
    blocks = qs.reshape(48, 2, 16)
    q = np.concatenate([blocks & 15, blocks >> 4], axis=2).astype(np.int64)  # [48][2][32]
    av = a.astype(np.int64).reshape(5, 2, 32)
    qa = np.einsum("rbi,tbi->trb", q, av)
    asum = av.sum(axis=2)[:, None, :]
    np.testing.assert_array_equal(got, qa - 8 * asum)


# ----------------------------------------------------------------- matvec
def test_gemv_vs_dense_dequantised_product():
    qs, d = synth.q4_matrix(13, 0, 0, synth.MAT_GATE, 96, 512)
    x = synth.normal(13, 5, (3, 512))
    xq, xd = oracle.q8_quantize(x)
    y = oracle.gemv(qs, d, xq, xd)
    W = _np_dequant(qs, d)
    X = (xq.reshape(3, -1, 32).astype(np.float64) * xd[:, :, None].astype(np.float64)).reshape(3, -1)
    ref = X @ W.T
    np.testing.assert_allclose(y, ref.astype(np.float32), rtol=0, atol=np.abs(ref).max() * 2e-7)


def test_gemv_workload0_shape_and_zero_vector():
    qs, d = synth.gemv_matrix()
    assert qs.shape == (512, 1024) and d.shape == (512, 64)
    xq = np.zeros((1, 2048), np.int8)
    xd = np.zeros((1, 64), np.float32)
    assert np.all(oracle.gemv(qs, d, xq, xd) == 0)


# ----------------------------------------------------------------- router
def test_route_ids_vs_stable_argsort_and_weights_vs_scipy():
    T, E, k = 37, 64, 8
    lg = synth.normal(14, 3, (T, E))
    lg[5, :] = lg[5, 0]                   # all-equal row: ties resolved by id
    lg[6, 10:20] = lg[6, 3]               # a tie block
    ids, w, off, sp = oracle.route(lg, k)
    ref_ids = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(ids, ref_ids)
    p = scipy.special.softmax(lg.astype(np.float64), axis=1)
    sel = np.take_along_axis(p, ref_ids, axis=1)
    ref_w = sel / sel.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(w, ref_w, rtol=2e-7, atol=0)
    assert np.all(np.abs(w.astype(np.float64).sum(axis=1) - 1.0) <= 1e-6)
    np.testing.assert_allclose(w[5], np.full(k, 1.0 / k, np.float32), rtol=1e-7)


def test_route_special_cases():
    lg = np.zeros((3, 16), np.float32)
    ids, w, off, sp = oracle.route(lg, 16)          # k = E, equal logits: every weight 1/E
    np.testing.assert_array_equal(ids, np.tile(np.arange(16), (3, 1)))
    assert np.all(w == np.float32(1.0 / 16))
    lg = synth.normal(15, 4, (9, 32))
    ids, w, off, sp = oracle.route(lg, 1)           # k = 1: the argmax with weight 1
    np.testing.assert_array_equal(ids[:, 0], lg.argmax(axis=1))
    assert np.all(w == 1.0)


def test_route_permutation_vs_library():
    for T, E, k, seed in ((947, 128, 8, 3), (50, 256, 8, 4), (5, 4, 2, 5), (0, 8, 2, 6)):
        lg = synth.normal(seed, 2, (T, E))
        ids, w, off, sp = oracle.route(lg, k)
        flat = ids.ravel()
        np.testing.assert_array_equal(sp, np.argsort(flat, kind="stable"))
        cnt = np.bincount(flat, minlength=E)
        np.testing.assert_array_equal(off, np.concatenate([[0], np.cumsum(cnt)]))
        assert off[E] == T * k
        # each pair exactly once, in its expert's range, and no token twice per expert
        assert sorted(sp.tolist()) == list(range(T * k))
        for e in range(E):
            seg = sp[off[e]:off[e + 1]]
            assert np.all(flat[seg] == e)
            assert len(set((seg // k).tolist())) == len(seg)


def test_route_zipf_bias_skews_load():
    w3 = synth.WORKLOADS[3]
    lg = synth.logits(w3)
    ids, w, off, sp = oracle.route(lg, w3.k)
    cnt = np.diff(off)
    assert cnt.sum() == w3.T * w3.k
    assert cnt.max() >= 0.9 * w3.T            # the head expert takes (almost) every token
    assert (cnt > 0).sum() < w3.E // 2        # most experts get nothing


# ----------------------------------------------------------------- whole layer
def _tiny_experts(seed, E, H, I, identical=False):
    es = synth.expert_set(seed, 0, E, H, I)
    if identical:
        for a in (es.gate_qs, es.up_qs, es.down_qs, es.gate_d, es.up_d, es.down_d):
            a[:] = a[0]
    return es


def _py_bruteforce_layer(es, x, logits, k):
    """Pure-Python loops over dequantised values (fp64)."""
    T, H = x.shape
    I = es.I
    xq, xd = _np_q8(x)
    Wg = [_np_dequant(es.gate_qs[e], es.gate_d[e]) for e in range(es.E)]
    Wu = [_np_dequant(es.up_qs[e], es.up_d[e]) for e in range(es.E)]
    Wd = [_np_dequant(es.down_qs[e], es.down_d[e]) for e in range(es.E)]
    y = np.zeros((T, H))
    for t in range(T):
        xv = [float(xq[t, i]) * float(xd[t, i // 32]) for i in range(H)]
        order = sorted(range(es.E), key=lambda e: (-float(logits[t, e]), e))[:k]
        m = max(float(v) for v in logits[t])
        ex = [np.exp(float(logits[t, e]) - m) for e in order]
        for j, e in enumerate(order):
            wt = float(np.float32(ex[j] / sum(ex)))
            h = np.zeros(I, np.float32)
            for n in range(I):
                g = sum(Wg[e][n, i] * xv[i] for i in range(H))
                u = sum(Wu[e][n, i] * xv[i] for i in range(H))
                h[n] = np.float32(g / (1.0 + np.exp(-g)) * u)
            hq, hd = _np_q8(h[None, :])
            hv = [float(hq[0, i]) * float(hd[0, i // 32]) for i in range(I)]
            for n in range(H):
                y[t, n] += wt * sum(Wd[e][n, i] * hv[i] for i in range(I))
    return y


def test_layer_tiny_bruteforce():
    E, k, H, I, T = 4, 2, 64, 32, 3
    es = _tiny_experts(21, E, H, I)
    x = synth.normal(21, 1, (T, H))
    lg = synth.normal(21, 2, (T, E))
    ids, w, off, sp = oracle.route(lg, k)
    xq, xd = oracle.q8_quantize(x)
    y = oracle.moe_layer(es, xq, xd, ids, w)
    ref = _py_bruteforce_layer(es, x, lg, k)
    np.testing.assert_allclose(y, ref, rtol=0, atol=np.abs(ref).max() * 1e-6)


def test_layer_identical_experts_is_dense_ffn():
    E, k, H, I, T = 8, 4, 256, 64, 6
    es = _tiny_experts(22, E, H, I, identical=True)
    x = synth.normal(22, 1, (T, H))
    lg = synth.normal(22, 2, (T, E))
    ids, w, off, sp = oracle.route(lg, k)
    xq, xd = oracle.q8_quantize(x)
    y = oracle.moe_layer(es, xq, xd, ids, w)
    # dense SwiGLU FFN with the (shared) W4A8 weights, numpy fp64
    X = (xq.reshape(T, -1, 32).astype(np.float64) * xd[:, :, None]).reshape(T, H)
    g = X @ _np_dequant(es.gate_qs[0], es.gate_d[0]).T
    u = X @ _np_dequant(es.up_qs[0], es.up_d[0]).T
    h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
    hq, hd = _np_q8(h)
    Hv = (hq.reshape(T, -1, 32).astype(np.float64) * hd[:, :, None]).reshape(T, I)
    ref = Hv @ _np_dequant(es.down_qs[0], es.down_d[0]).T
    # sum_j w_j = 1 up to fp32 rounding of the weights
    np.testing.assert_allclose(y, ref, rtol=0, atol=np.abs(ref).max() * 1e-5)


def test_layer_zero_token_and_accumulate_and_conditioning():
    E, k, H, I, T = 6, 3, 128, 64, 4
    es = _tiny_experts(23, E, H, I)
    x = synth.normal(23, 1, (T, H))
    x[2] = 0.0
    lg = synth.normal(23, 2, (T, E))
    ids, w, off, sp = oracle.route(lg, k)
    xq, xd = oracle.q8_quantize(x)
    y, it = oracle.moe_layer(es, xq, xd, ids, w, want_intermediates=True)
    assert np.all(y[2] == 0.0)
    # ACCUMULATE adds onto the incoming rows
    base = synth.normal(23, 9, (T, H))
    y2 = oracle.moe_layer(es, xq, xd, ids, w, flags=oracle.FLAG_ACCUMULATE, y=base.copy())
    np.testing.assert_allclose(y2, base.astype(np.float64) + y, rtol=0, atol=np.abs(y2).max() * 1e-6)
    # conditioning on its own re-quantised h reproduces y exactly
    y3 = oracle.moe_layer(es, xq, xd, ids, w, hq_in=it["hq"], hd_in=it["hd"])
    np.testing.assert_array_equal(y3, y)
    # g and u match the matvec of the routed expert; h = silu(g) u
    t, j = 1, 2
    e = ids[t, j]
    p = t * k + j
    gref = oracle.gemv(es.gate_qs[e], es.gate_d[e], xq[t:t + 1], xd[t:t + 1])[0]
    np.testing.assert_array_equal(it["g"][p], gref)
    # sampling a token subset matches the full computation on those rows
    ys = oracle.moe_layer(es, xq, xd, ids, w, tokens=[3, 0])
    np.testing.assert_array_equal(ys[[0, 3]], y[[0, 3]])
    assert np.all(ys[[1, 2]] == 0)


def test_layer_abs_sums_closed_forms():
    """sg/su (sum over blocks of |d_w d_a isum|, the magnitude sum that bounds fp32 rounding of g and u):
    a hand-built case with cancelling blocks, the same-sign case, the triangle inequality and sign symmetry."""
    E, k, H, I, T = 2, 1, 64, 32, 1
    es = _tiny_experts(24, E, H, I)
    # expert 0: gate rows all q = 9 (w = +d) in block 0 and q = 7 (w = -d) in block 1, d = 1.0 (fp16 0x3C00)
    es.gate_qs[0, :, :16] = 0x99
    es.gate_qs[0, :, 16:] = 0x77
    es.gate_d[0] = 0x3C00
    es.up_qs[0] = 0xFF  # every up weight q = 15: w = 7 d
    es.up_d[0] = 0x3C00
    x = np.full((T, H), 127.0, np.float32)  # amax 127 -> d_a = 1, every code 127
    xq, xd = oracle.q8_quantize(x)
    assert np.all(xq == 127) and np.all(xd == 1.0)
    ids = np.zeros((T, k), np.int32)
    w = np.ones((T, k), np.float32)
    _, it = oracle.moe_layer(es, xq, xd, ids, w, want_intermediates=True)
    # gate: +32*127 in block 0, -32*127 in block 1 -> g = 0, sum of magnitudes 8128
    assert np.all(it["g"][0] == 0.0) and np.all(it["sg"][0] == 8128.0)
    # up: both blocks 32 * 7 * 127 = 28448 -> u = S = 56896
    assert np.all(it["u"][0] == 56896.0) and np.all(it["su"][0] == 56896.0)
    # random experts: S >= |g| (fp32 g within half an ulp of the fp64 sum), S(-x) = S(x), g(-x) = -g(x)
    es = _tiny_experts(25, 4, 256, 64)
    x = synth.normal(25, 1, (3, 256))
    lg = synth.normal(25, 2, (3, 4))
    ids, w, _, _ = oracle.route(lg, 2)
    xq, xd = oracle.q8_quantize(x)
    _, a = oracle.moe_layer(es, xq, xd, ids, w, want_intermediates=True)
    _, b = oracle.moe_layer(es, (-xq).astype(np.int8), xd, ids, w, want_intermediates=True)
    for g, sabs in ((a["g"], a["sg"]), (a["u"], a["su"])):
        assert np.all(sabs >= np.abs(g.astype(np.float64)) * (1 - 2.0 ** -23))
        assert np.all(sabs > 0)
    np.testing.assert_array_equal(b["sg"], a["sg"])
    np.testing.assert_array_equal(b["su"], a["su"])
    np.testing.assert_array_equal(b["g"], -a["g"])
    # one block per row: the magnitude sum is |g| itself
    es1 = _tiny_experts(26, 2, 32, 32)
    x1 = synth.normal(26, 1, (2, 32))
    xq1, xd1 = oracle.q8_quantize(x1)
    ids1 = np.array([[0], [1]], np.int32)
    _, c = oracle.moe_layer(es1, xq1, xd1, ids1, np.ones((2, 1), np.float32), want_intermediates=True)
    np.testing.assert_array_equal(c["sg"].astype(np.float32), np.abs(c["g"]))


# ------------------------------------------------------------------ router projection (R10)
def test_router_one_hot_rows_select_inputs():
    """W_r = [I | 0] (E <= H): every logit is an input element, exactly."""
    T, H, E = 4, 96, 40
    x = synth.normal(81, 1, (T, H))
    wr = np.zeros((E, H), np.float32)
    wr[np.arange(E), np.arange(E)] = 1.0
    np.testing.assert_array_equal(oracle.router_logits(x, wr), x[:, :E])
    x[2] = 0.0  # a zero row gives zero logits, with the pre-norm too (its factor is finite)
    assert np.all(oracle.router_logits(x, wr, oracle.FLAG_RMSNORM)[2] == 0.0)


def test_router_vs_numpy_float64_matmul():
    """Reduces to a dense fp64 matmul rounded once to fp32 (numpy's summation order differs: <= 1 ulp)."""
    T, H, E = 6, 160, 11
    x = synth.normal(82, 1, (T, H))
    wr = synth.router_weights(82, 0, E, H)
    got = oracle.router_logits(x, wr).astype(np.float64)
    ref = (x.astype(np.float64) @ wr.astype(np.float64).T).astype(np.float32).astype(np.float64)
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - ref) <= ulp)


def test_router_rmsnorm_properties():
    """With the pre-norm and W_r = I, the logits are the normalised row: mean square 1 (up to eps 1e-6) and
    invariant to scaling the row by a power of two."""
    T, H = 3, 128
    x = synth.normal(83, 1, (T, H)) * np.float32(7.0)
    eye = np.eye(H, dtype=np.float32)
    xn = oracle.router_logits(x, eye, oracle.FLAG_RMSNORM).astype(np.float64)
    ms = (xn ** 2).mean(axis=1)
    np.testing.assert_allclose(ms, 1.0, rtol=1e-6)
    wr = synth.router_weights(83, 0, 9, H)
    a = oracle.router_logits(x, wr, oracle.FLAG_RMSNORM)
    b = oracle.router_logits(x * np.float32(8.0), wr, oracle.FLAG_RMSNORM)
    np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-7)
    # without the pre-norm the logits scale with the input instead
    np.testing.assert_array_equal(oracle.router_logits(x * np.float32(8.0), wr), oracle.router_logits(x, wr) * 8)


# ------------------------------------------------------------------ W4A16 expert FFN (R11)
def test_round_to_half_vs_numpy_float16():
    """fp16 rounding (nearest, ties to even) against numpy's float16 conversion: random values over the whole
    range, exact ties, subnormals and the overflow threshold."""
    rng = np.random.default_rng(5)
    vals = list(rng.standard_normal(2000) * 10.0 ** rng.integers(-9, 5, 2000))
    vals += [0.5 + 2 ** -11, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 2049.0, 2051.0, -2051.0,  # ties
             2 ** -24, 2 ** -25, 3 * 2 ** -26, 2 ** -14 - 2 ** -25, 1e-9,                  # subnormals, underflow
             65504.0, 65519.99, 65520.0, -65520.0, 1e6, 0.0, -0.0]                        # overflow threshold
    for v in vals:
        with np.errstate(over="ignore"):  # the overflow cases round to infinity on purpose
            ref = float(np.float64(v).astype(np.float16))
        got = oracle.round_to_half(v)
        assert got == ref or (np.isinf(got) and np.isinf(ref) and np.sign(got) == np.sign(ref)), (v, got, ref)


def _np_layer_a16(es, x, ids, w, exact):
    """numpy W4A16 layer: dequantised weights, x and h rounded through numpy float16 (weights too) unless exact."""
    T, H = x.shape
    k = ids.shape[1]
    r16 = (lambda a: a) if exact else (lambda a: a.astype(np.float16).astype(np.float64))
    y = np.zeros((T, H))
    for t in range(T):
        xv = r16(x[t].astype(np.float64))
        for j in range(k):
            e = ids[t, j]
            g = r16(_np_dequant(es.gate_qs[e], es.gate_d[e])) @ xv
            u = r16(_np_dequant(es.up_qs[e], es.up_d[e])) @ xv
            h = r16(g / (1.0 + np.exp(-g)) * u)
            y[t] += float(w[t, j]) * (r16(_np_dequant(es.down_qs[e], es.down_d[e])) @ h)
    return y.astype(np.float32)


@pytest.mark.parametrize("flags", [0, 4])
def test_layer_a16_tiny_vs_numpy(flags):
    E, k, H, I, T = 4, 2, 64, 32, 3
    es = _tiny_experts(22, E, H, I)
    x = synth.normal(22, 1, (T, H)) * np.float32(3.0)
    ids, w, _, _ = oracle.route(synth.normal(22, 2, (T, E)), k)
    y = oracle.moe_layer_a16(es, x, ids, w, flags=flags)
    ref = _np_layer_a16(es, x, ids, w, exact=flags == oracle.FLAG_EXACT_ACT)
    np.testing.assert_allclose(y, ref, rtol=0, atol=np.abs(ref).max() * 1e-6)
    # a zero row gives zero output; ACCUMULATE adds
    x[1] = 0.0
    y0 = oracle.moe_layer_a16(es, x, ids, w, flags=flags)
    assert np.all(y0[1] == 0.0)
    base = synth.normal(22, 3, (T, 64))
    ya = oracle.moe_layer_a16(es, x, ids, w, flags=flags | oracle.FLAG_ACCUMULATE, y=base.copy())
    np.testing.assert_allclose(ya, base + y0, rtol=2e-7, atol=1e-6)


def test_layer_a16_exact_equals_w4a8_on_lossless_inputs():
    """Inputs whose every 32-block is lossless in Q8_0 (amax = 127 * 2^-5, so d = 2^-5 and x / d is an integer)
    and in fp16: the W4A8 layer's h and the exact-activation W4A16 layer's h are the same numbers."""
    E, k, H, I, T = 4, 2, 64, 32, 3
    es = _tiny_experts(23, E, H, I)
    rng = np.random.default_rng(23)
    q = rng.integers(-127, 128, (T, H))
    q[:, ::32] = 127                                     # every block reaches amax = 127 * 2^-5
    x = (q * 2.0 ** -5).astype(np.float32)
    ids, w, _, _ = oracle.route(synth.normal(23, 2, (T, E)), k)
    xq, xd = oracle.q8_quantize(x)
    assert np.all(xd == np.float32(2.0 ** -5)) and np.array_equal(xq.astype(np.int64), q)
    _, inter = oracle.moe_layer(es, xq, xd, ids, w, want_intermediates=True)
    _, h16 = oracle.moe_layer_a16(es, x, ids, w, flags=oracle.FLAG_EXACT_ACT, want_h=True)
    np.testing.assert_array_equal(h16, inter["h"])
