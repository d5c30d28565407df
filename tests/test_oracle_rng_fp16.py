"""Pins for the oracle's random generator and fp16 rounding (CPU only)."""
import numpy as np
import pytest
from scipy import stats


def test_splitmix64_reference_outputs(orc):
    # First three outputs of SplitMix64 from state 0, as printed by the
    # generator's reference implementation (S. Vigna, splitmix64.c).
    assert orc.splitmix64(0, 0) == 0xE220A8397B1DCDAF
    assert orc.splitmix64(0, 1) == 0x6E789E6AA1B965F4
    assert orc.splitmix64(0, 2) == 0x06C45D188009454F


def test_stream_key_definition(orc):
    # u64(seed, stream, i) is output i of the state that output `stream` of `seed` gives
    for seed, stream, i in [(0, 0, 0), (7, 1, 5), (123456789, 14, 1000)]:
        key = orc.splitmix64(seed, stream)
        assert orc.rng_u64(seed, stream, i) == orc.splitmix64(key, i)


def test_uniform_range(orc):
    u = np.array([orc.rng_uniform(3, 2, i) for i in range(20000)])
    assert u.min() > 0.0 and u.max() <= 1.0
    assert stats.kstest(u, "uniform").pvalue > 1e-4


def test_box_muller_pairs(orc):
    n = 4000
    z = orc.rng_normals(5, 0, n)
    for j in range(0, n // 2, 97):
        u1 = orc.rng_uniform(5, 0, 2 * j)
        u2 = orc.rng_uniform(5, 0, 2 * j + 1)
        r2 = z[2 * j] ** 2 + z[2 * j + 1] ** 2
        assert r2 == pytest.approx(-2.0 * np.log(u1), rel=1e-12)
        assert np.arctan2(z[2 * j + 1], z[2 * j]) % (2 * np.pi) == pytest.approx(
            (2 * np.pi * u2) % (2 * np.pi), abs=1e-9)


def test_normals_distribution(orc):
    z = orc.rng_normals(11, 3, 200001)
    assert abs(z.mean()) < 0.01 and abs(z.var() - 1.0) < 0.01
    assert stats.kstest(z, "norm").pvalue > 1e-4
    # odd n: the last value is the cosine branch of its pair
    z5 = orc.rng_normals(11, 3, 5)
    assert np.array_equal(z5, z[:5])


def test_fp16_matches_numpy_rne(orc):
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(3000) * 10.0 ** rng.uniform(-9, 5, 3000),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -24, 2.0 ** -25,
                  2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 * (1 - 2 ** -12),
                  1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0, 0.1, 1 / 3]),
    ])
    for v in vals:
        got = orc.f16_from_double(v)
        want = int(np.array(v, dtype=np.float64).astype(np.float16).view(np.uint16))
        assert got == want, (v, hex(got), hex(want))
        if (got & 0x7C00) != 0x7C00:
            back = orc.f16_to_double(got)
            assert back == float(np.uint16(got).view(np.float16))
