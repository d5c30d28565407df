"""Pins for the coordinate density f_d and the Lloyd-Max codebook (CPU only).

f_d is the density turboquant.net prints in its "PolarQuant" section; the
Lloyd-Max quantizer is the one its pseudo-code precomputes.  Every expected
value here comes from scipy (beta distribution, quad), a closed form, or a
textbook table -- never from the oracle itself.
"""
import os

import numpy as np
import pytest
from scipy import integrate, special, stats

GOLD = os.path.join(os.path.dirname(__file__), "golden")
DIMS = [3, 4, 5, 16, 128, 200, 1536]


def eabs(d):
    # E|X| for one coordinate of a uniform point on S^{d-1}
    return float(np.exp(special.gammaln(d / 2) - special.gammaln((d + 1) / 2)) / np.sqrt(np.pi))


@pytest.mark.parametrize("d", DIMS)
def test_density_matches_scipy_beta(orc, d):
    # X = 2B - 1 with B ~ Beta((d-1)/2, (d-1)/2)
    a = (d - 1) / 2
    for x in np.linspace(-0.999, 0.999, 37) * min(1.0, 8 / np.sqrt(d)):
        want = stats.beta.pdf((1 + x) / 2, a, a) / 2
        assert orc.beta_density(d, x) == pytest.approx(want, rel=1e-9, abs=1e-300)


@pytest.mark.parametrize("d", DIMS)
def test_density_mass_and_moments(orc, d):
    assert orc.beta_integral(d, 0, -1, 1) == pytest.approx(1.0, abs=1e-10)
    assert orc.beta_integral(d, 1, -1, 1) == pytest.approx(0.0, abs=1e-12)
    # sum of squared coordinates of a unit vector is 1 -> E[X^2] = 1/d
    assert orc.beta_integral(d, 2, -1, 1) == pytest.approx(1.0 / d, rel=1e-10)
    # E|X| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))
    assert 2 * orc.beta_integral(d, 1, 0, 1) == pytest.approx(eabs(d), rel=1e-10)


def test_eabs_reference_values():
    # closed-form values quoted for the pins
    assert eabs(3) == pytest.approx(0.5, rel=1e-12)
    assert eabs(128) == pytest.approx(0.070661573, rel=1e-8)
    assert eabs(200) == pytest.approx(0.056489526, rel=1e-8)
    assert eabs(1536) == pytest.approx(0.020361752, rel=1e-8)


def test_density_d3_is_uniform(orc):
    # Archimedes: one coordinate of a uniform point on S^2 is uniform on [-1, 1]
    for x in [-0.9, -0.3, 0.0, 0.5, 0.99]:
        assert orc.beta_density(3, x) == pytest.approx(0.5, rel=1e-14)


@pytest.mark.parametrize("d", [5, 128, 1536])
def test_cdf_matches_scipy(orc, d):
    a = (d - 1) / 2
    for x in np.array([-0.5, -0.1, -0.01, 0.0, 0.003, 0.05, 0.2]) * min(1.0, 6 / np.sqrt(d)) * 3:
        want = stats.beta.cdf((1 + x) / 2, a, a)
        assert orc.beta_integral(d, 0, -1, x) == pytest.approx(want, abs=1e-11)


@pytest.mark.parametrize("d", [128, 200, 1536])
def test_lloyd_one_bit_closed_form(orc, d):
    c, D, it, ok = orc.lloyd_max(d, 1)
    assert ok
    assert c[1] == pytest.approx(eabs(d), rel=1e-12) and c[0] == -c[1]
    # D_1 = 1 - d E|X|^2
    assert D == pytest.approx(1 - d * eabs(d) ** 2, abs=1e-11)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_lloyd_d3_uniform_grid(orc, bits):
    K = 1 << bits
    c, D, it, ok = orc.lloyd_max(3, bits)
    assert ok
    np.testing.assert_allclose(c, -1 + (2 * np.arange(K) + 1) / K, atol=1e-13)
    # uniform density on [-1, 1], cell width 2/K: per-coordinate MSE (2/K)^2/12
    assert D == pytest.approx(3 * (2 / K) ** 2 / 12, rel=1e-10)


@pytest.mark.parametrize("d", [16, 128, 200, 1536])
@pytest.mark.parametrize("bits", [2, 3])
def test_lloyd_fixed_point_with_scipy_quad(orc, d, bits):
    """Each centroid is the mean of its cell, recomputed with scipy.quad."""
    c, D, it, ok = orc.lloyd_max(d, bits)
    assert ok
    K = 1 << bits
    assert np.all(np.diff(c) > 0)
    np.testing.assert_array_equal(c, -c[::-1])  # exact symmetry
    a = (d - 1) / 2
    pdf = lambda x: stats.beta.pdf((1 + x) / 2, a, a) / 2
    t = np.concatenate([[-1.0], (c[:-1] + c[1:]) / 2, [1.0]])
    s = 1 / np.sqrt(d)
    dist = 0.0
    for k in range(K):
        lo, hi = max(t[k], -12 * s), min(t[k + 1], 12 * s)
        pts = [p for p in np.arange(-12, 13) * s if lo < p < hi]
        m0 = integrate.quad(pdf, lo, hi, points=pts or None, epsabs=1e-15, epsrel=1e-13, limit=400)[0]
        m1 = integrate.quad(lambda x: x * pdf(x), lo, hi, points=pts or None, epsabs=1e-17,
                            epsrel=1e-13, limit=400)[0]
        assert m1 / m0 == pytest.approx(c[k], rel=1e-9)
        dist += integrate.quad(lambda x: (x - c[k]) ** 2 * pdf(x), lo, hi, points=pts or None,
                               epsabs=1e-17, epsrel=1e-12, limit=400)[0]
    assert D == pytest.approx(d * dist, rel=1e-8)


def test_lloyd_distortion_monotone(orc):
    for d in [128, 1536]:
        Ds = [orc.lloyd_max(d, bits)[1] for bits in [1, 2, 3, 4]]
        assert all(x > y for x, y in zip(Ds, Ds[1:]))
        c, D, it, ok, hist = orc.lloyd_max(d, 3, history=True)
        assert np.all(np.diff(hist) <= 1e-15)


def _gauss_lloyd(K, iters=20000):
    """Lloyd-Max for N(0,1) with closed-form conditional means."""
    c = np.linspace(-2, 2, K)
    for _ in range(iters):
        t = np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2, [np.inf]])
        num = stats.norm.pdf(t[:-1]) - stats.norm.pdf(t[1:])
        den = stats.norm.cdf(t[1:]) - stats.norm.cdf(t[:-1])
        c_new = num / den
        if np.max(np.abs(c_new - c)) < 1e-14:
            return c_new
        c = c_new
    return c


def test_lloyd_gaussian_limit(orc):
    table = {}
    for line in open(os.path.join(GOLD, "gaussian_lloyd_max.txt")):
        if line.strip() and not line.startswith("#"):
            v = line.split()
            table[int(v[0])] = np.array([float(x) for x in v[1:]])
    for bits in [1, 2, 3]:
        K = 1 << bits
        g = _gauss_lloyd(K)
        np.testing.assert_allclose(g[K // 2:], table[K], rtol=2e-3)  # textbook, 3-4 digits
        errs = []
        for d in [128, 200, 1536]:
            c = orc.lloyd_max(d, bits)[0]
            errs.append(np.max(np.abs(np.sqrt(d) * c - g)))
        assert errs[0] > errs[1] > errs[2]       # converges as d grows
        assert errs[2] < 4e-3


def test_distortion_within_pages_factor(orc):
    factor = float([l.split()[1] for l in open(os.path.join(GOLD, "distortion_factor.txt"))
                    if l.startswith("factor")][0])
    for d in [128, 200, 1536]:
        for bits in [1, 2, 3, 4]:
            D = orc.lloyd_max(d, bits)[1]
            assert D * 4.0 ** bits < factor


def test_lloyd_not_converged_flag(orc):
    c, D, it, ok = orc.lloyd_max(128, 3, max_iter=2)
    assert not ok and it == 2
