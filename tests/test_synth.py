"""The seeded input generator: reproducible, sliceable, with the stated distributions."""
import numpy as np

import synth


def test_splitmix64_reference_values():
    # SplitMix64 seeded with state 0 yields these published first outputs; the stream
    # key of (seed, tid) is an arbitrary state, so check the finaliser through a
    # stream whose key we can reproduce in pure Python.
    M = (1 << 64) - 1

    def mix(z):
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M
        return z ^ (z >> 31)

    state = 0
    outs = []
    for _ in range(3):
        state = (state + 0x9E3779B97F4A7C15) & M
        outs.append(mix(state))
    assert outs == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    seed, tid = 9, 1234
    key = mix((seed * 0x9E3779B97F4A7C15 + mix((tid + 0x632BE59BD9B4E019) & M)) & M)
    expect = [mix((key + (i + 1) * 0x9E3779B97F4A7C15) & M) for i in range(5)]
    assert synth.u64(seed, tid, 5).tolist() == expect


def test_slices_are_consistent():
    full = synth.normal(3, 17, (1000,))
    np.testing.assert_array_equal(synth.normal(3, 17, (301,), start=99), full[99:400])
    nb = synth.nibble_bytes(3, 18, 1000)
    for s, n in ((0, 1000), (3, 2), (3, 10), (5, 500), (8, 16), (999, 1)):
        np.testing.assert_array_equal(synth.nibble_bytes(3, 18, n, start=s), nb[s:s + n])
    sc = synth.scales_f16(3, 19, 100)
    np.testing.assert_array_equal(synth.scales_f16(3, 19, 50, start=25), sc[25:75])


def test_distributions():
    z = synth.normal(1, 2, (200000,)).astype(np.float64)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1.0) < 0.01
    nb = synth.nibble_bytes(1, 3, 200000)
    nib = np.concatenate([nb & 15, nb >> 4])
    cnt = np.bincount(nib, minlength=16) / nib.size
    assert np.all(np.abs(cnt - 1 / 16) < 0.003)
    d = synth.scales_f16(1, 4, 100000).view(np.float16).astype(np.float64)
    assert d.min() >= 0.002 - 1e-6 and d.max() <= 0.02 + 1e-5
    assert abs(d.mean() - 0.011) < 0.0002


def test_fp16_rounding_is_nearest_even():
    u = synth.uniform(1, 4, 5000)
    exact = synth.SCALE_LO + (synth.SCALE_HI - synth.SCALE_LO) * u
    got = synth.scales_f16(1, 4, 5000).view(np.float16)
    np.testing.assert_array_equal(got, exact.astype(np.float16))  # numpy casts with RNE


def test_workload_shapes_and_bias():
    es = synth.expert_set(2, 0, 2, 2048, 512)
    assert es.gate_qs.shape == (2, 512, 1024) and es.down_qs.shape == (2, 2048, 256)
    assert es.nbytes == 2 * 1769472
    w3 = synth.WORKLOADS[3]
    lg = synth.logits(w3, T=4)
    z = synth.normal(w3.seed, synth.logits_tid(0, 4), (4, w3.E)).astype(np.float64)
    bias = -2.2 * np.log(np.arange(1, w3.E + 1))
    np.testing.assert_allclose(lg, (z + bias).astype(np.float32), rtol=1e-6, atol=1e-6)
