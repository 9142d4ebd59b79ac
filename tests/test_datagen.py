"""The seeded input generators (CPU only)."""
import math

import numpy as np

import datagen


def test_splitmix64_published_vector():
    # SplitMix64 seeded with 0: the first outputs of the reference generator
    # (Steele, Lea, Flood 2014; the same values as Vigna's splitmix64.c).
    got = datagen.splitmix64(0, 0, 3)
    assert [int(x) for x in got] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_form_is_position_independent():
    full = datagen.splitmix64(77, 0, 1000)
    np.testing.assert_array_equal(datagen.splitmix64(77, 400, 600), full[400:])
    a = datagen.normal_f32(9, 300, 700)      # crosses several internal chunks
    b = datagen.normal_f32(9, 300, 700)
    np.testing.assert_array_equal(a, b)


def test_uniform_and_normal_moments():
    u = datagen.uniform_pm1_f32(3, 512, 512)
    assert u.min() >= -1 and u.max() < 1
    assert abs(u.mean()) < 5 * (1 / math.sqrt(3)) / 512
    assert abs(u.var() - 1 / 3) < 0.01
    z = datagen.normal_f32(4, 512, 512)
    assert abs(z.mean()) < 5 / 512
    assert abs(z.std() - 1) < 0.01
    k = 4096
    zs = datagen.normal_f32(5, 256, 256, 1 / math.sqrt(k))
    assert abs(zs.std() * math.sqrt(k) - 1) < 0.01


def test_small_ints():
    x = datagen.small_int_f32(6, 100, 100)
    assert set(np.unique(x)) == set(range(-4, 5))
    assert np.array_equal(x, np.round(x))


def test_configs_and_inputs():
    c = datagen.CONFIGS
    assert [c[i].name for i in range(1, 6)] == ["f32_256", "f32_1024", "f32_4096", "f32_4097x3001x2049", "bf16_8192"]
    assert c[4].lda % 4 and c[4].ldb % 4     # rows not 16-byte aligned
    a, b = datagen.make_inputs(c[1])
    assert a.shape == (256, 256) and b.shape == (256, 256) and a.dtype == np.float32
    assert c[5].flops == 2 * 8192 ** 3
    assert c[1].seed_a == 1001 and c[5].seed_b == 2005


def test_bf16_bits_roundtrip():
    x = datagen.normal_f32(8, 64, 64)
    h = datagen.f32_to_bf16_bits(x)
    y = datagen.bf16_bits_to_f32(h)
    assert np.all(np.abs(y - x) <= np.abs(x) * 2.0 ** -8)
    np.testing.assert_array_equal(datagen.f32_to_bf16_bits(y), h)


def test_zero_distribution():
    z = datagen.draw("zeros", 7, 3, 5, 5)
    assert z.dtype == np.float32 and z.shape == (3, 5) and not z.any()
