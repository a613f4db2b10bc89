"""The seeded input generator (CPU only)."""
import math

import numpy as np

import gen


def test_splitmix64_published_stream():
    # SplitMix64 (Steele, Lea & Flood 2014) seeded with 0: its well-known first outputs.
    # Our stream (seed 0, tensor 0) is exactly that stream, since mix(0) = 0.
    w = gen.words(0, 0, 0, 3)
    assert [int(x) for x in w] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_index_addressable_and_deterministic():
    a = gen.normal_f32(5, 1, (10000,))
    b = gen.normal_f32(5, 1, (3000,), offset=7000, nthreads=3)
    assert np.array_equal(a[7000:], b)
    assert np.array_equal(a, gen.normal_f32(5, 1, (10000,), nthreads=1))
    assert not np.array_equal(a, gen.normal_f32(5, 2, (10000,)))
    assert not np.array_equal(a, gen.normal_f32(6, 1, (10000,)))


def test_box_muller_from_words():
    # element 2p and 2p+1 come from words 2p, 2p+1 by the Box-Muller pair
    w = gen.words(3, 2, 0, 8)
    z = gen.normal_f32(3, 2, (8,))
    for p in range(4):
        u1 = ((int(w[2 * p]) >> 11) + 0.5) * 2.0 ** -53
        u2 = (int(w[2 * p + 1]) >> 11) * 2.0 ** -53
        r = math.sqrt(-2.0 * math.log(u1))
        assert z[2 * p] == np.float32(r * math.cos(2 * math.pi * u2))
        assert z[2 * p + 1] == np.float32(r * math.sin(2 * math.pi * u2))


def test_moments():
    x = gen.normal_f32(1, 0, (1 << 20,)).astype(np.float64)
    assert abs(x.mean()) < 5e-3
    assert abs(x.var() - 1.0) < 5e-3
    assert abs((x ** 3).mean()) < 2e-2
    assert abs((x ** 4).mean() - 3.0) < 3e-2


def test_scale_then_round():
    f = gen.normal_f32(4, 0, (4096,), scale=3.0)
    assert np.array_equal(f, gen.normal_f32(4, 0, (4096,)) * np.float32(3.0))
    b = gen.normal_bf16(4, 0, (4096,), scale=3.0)
    assert np.array_equal(b, gen.f32_to_bf16(f))


def test_bf16_round_to_nearest_even():
    def bits(v):
        return int(np.array([v], dtype=np.float32).view(np.uint32)[0])

    def f(b):
        return float(np.array([b], dtype=np.uint32).view(np.float32)[0])

    assert gen.bf16_rne_scalar(1.0) == 0x3F80
    # exactly halfway between 0x3F80 and 0x3F81: ties to even (down)
    assert gen.bf16_rne_scalar(f(0x3F808000)) == 0x3F80
    # halfway between 0x3F81 and 0x3F82: ties to even (up)
    assert gen.bf16_rne_scalar(f(0x3F818000)) == 0x3F82
    assert gen.bf16_rne_scalar(f(0x3F808001)) == 0x3F81
    assert gen.bf16_rne_scalar(f(0x3F807FFF)) == 0x3F80
    # largest finite float rounds to +inf; largest bf16 stays
    assert gen.bf16_rne_scalar(f(0x7F7FFFFF)) == 0x7F80
    assert gen.bf16_rne_scalar(f(0x7F7F0000)) == 0x7F7F
    # subnormals and signed zero
    assert gen.bf16_rne_scalar(f(0x00018000)) == 0x0002
    assert gen.bf16_rne_scalar(-0.0) == 0x8000
    assert gen.bf16_rne_scalar(float("inf")) == 0x7F80
    nan = gen.bf16_rne_scalar(float("nan"))
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0
    # widening is exact and round-trips
    h = gen.normal_bf16(9, 0, (1000,))
    assert np.array_equal(gen.f32_to_bf16(gen.bf16_to_f32(h)), h)
    assert bits(1.0) == 0x3F800000
