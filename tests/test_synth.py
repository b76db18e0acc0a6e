"""The seeded input generator (shared by both sides, holds no method arithmetic)."""
import math

import numpy as np

from test_token_chunk_amd import synth


def test_splitmix64_published_sequence():
    # first outputs of SplitMix64 seeded with 1234567 (the commonly published
    # test vector of the reference implementation)
    assert [synth.splitmix64_at(1234567, i) for i in range(5)] == [
        6457827717110365317, 3203168211198807973, 9817491932198370423, 4593380528125082431,
        16408922859458223821]


def test_normal_moments_and_bf16_rounding():
    z = synth.normal(0, 3, (400000,), std=0.02)
    assert abs(z.mean()) < 1e-4 and abs(z.std() - 0.02) < 2e-4
    zb = synth.normal(0, 3, (400000,), std=0.02, bf16=True)
    bits = zb.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)  # bf16-representable
    assert np.max(np.abs(zb - z)) <= np.max(np.abs(z)) * 2 ** -8  # RNE: within half a bf16 ulp


def test_tokens_uniform_and_zipf():
    u = synth.tokens(2, 50000, 512, "uniform")
    assert u.min() >= 0 and u.max() < 512 and not np.array_equal(u[0], u[1])
    z = synth.tokens(1, 300000, 32000, "zipf")[0]
    assert z.min() >= 0 and z.max() < 32000
    p = np.bincount(z, minlength=32000) / z.size
    H = 1.1
    ranks = np.arange(1, 32001, dtype=np.float64)
    q = ranks ** -H
    q /= q.sum()
    assert abs(p[0] - q[0]) < 3e-3 and abs(p[1] - q[1]) < 3e-3
    ent = -(q * np.log(q)).sum()
    assert abs(ent - 6.28) < 0.01 and ent < math.log(32000)


def test_streams_are_reproducible():
    a = synth.weights(synth.Shape(2, 16, 2, 24, 11), bf16=True)
    b = synth.weights(synth.Shape(2, 16, 2, 24, 11), bf16=True)
    assert all(np.array_equal(x, y) for x, y in zip(a["w_up"], b["w_up"]))
    assert not np.array_equal(a["wq"][0], a["wk"][0])
