"""CPU checks of the seeded input generator (inputs/)."""
import numpy as np

import inputs


def test_splitmix64_published_vector():
    # SplitMix64 seeded with 1234567: the first five outputs published with
    # Vigna's reference splitmix64.c test harness.
    got = [int(v) for v in inputs.splitmix64(np.uint64(1234567), np.arange(5))]
    assert got == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                   4593380528125082431, 16408922859458223821]


def test_blob_is_deterministic_and_keyed():
    a = inputs.gen_blob(3, 17)
    b = inputs.gen_blob(3, 17)
    c = inputs.gen_blob(3, 18)
    d = inputs.gen_blob(4, 17)
    assert a.size == inputs.blob_bytes() == 1382400
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c) and not np.array_equal(a, d)


def test_blob_fields_follow_the_law():
    blob = inputs.gen_blob(0, 123).reshape(-1, 18)
    d = blob[:, 0:2].copy().view("<f2").astype(np.float64).ravel()
    assert d.min() >= 1e-4 * (1 - 2 ** -10) and d.max() < 0.05
    # mean of |N(0, 0.01)| + 1e-4 is 0.01 * sqrt(2 / pi) + 1e-4
    assert abs(d.mean() - (0.01 * np.sqrt(2 / np.pi) + 1e-4)) < 2e-4
    codes = np.unpackbits(blob[:, 2:].ravel(), bitorder="little").reshape(-1, 2)
    c = codes[:, 0] + 2 * codes[:, 1]
    freq = np.bincount(c, minlength=4) / c.size
    assert np.all(np.abs(freq - 0.25) < 0.002)


def test_scale_table_is_monotone_half_normal():
    t = inputs.scale_table().view(np.float16).astype(np.float64)
    assert t.size == 65536 and np.all(np.diff(t) >= 0)
    assert abs(t[32768] - (0.01 * 0.6744897501960817 + 1e-4)) < 2e-5  # median of |N(0,1)|


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], dtype=np.float32)
    bits = inputs.f32_to_bf16_bits(vals)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert list(back) == [1.0, 1.0, 1.0 + 4 * 2 ** -8, -2.5, 1.0]


def test_streams_are_seeded_and_independent():
    a, b = inputs.Streams(1), inputs.Streams(1)
    xa, xb = inputs.draw_x(a.x, 4), inputs.draw_x(b.x, 4)
    assert np.array_equal(xa, xb) and xa.dtype == np.float32 and xa.shape == (4, 2560)
    r = inputs.draw_router(a.router)
    assert r.shape == (512, 2560) and r.dtype == np.uint16
    rv = (r.astype(np.uint32) << 16).view(np.float32)
    assert abs(rv.std() - 0.02) < 2e-4
    bias = inputs.draw_zipf_bias(a.bias)
    assert np.isclose(np.sort(bias)[-1], 0.0) and np.isclose(bias.min(), -1.1 * np.log(512))
