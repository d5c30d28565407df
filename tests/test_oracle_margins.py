"""Pins for the oracle's decision margins and for its QJL stage on given codes
(CPU only).

Every GPU quantize parity test forgives a code mismatch only where the
oracle's ``code_margin`` (the distance of the rotated coordinate y_j to the
nearest decision midpoint t_k = (c_k + c_{k+1}) / 2) is below 1e-5, and
checks the signs and gamma of such a vector against the oracle's second stage
run on the GPU's codes (``qjl_given_codes``).  Both are pinned here by
arithmetic done independently in numpy: y = Pi (x / ||x||) with numpy's
matmul, the midpoints from the centroids, the residual and sketch from their
definitions (turboquant.net pseudo-code "quant"; admirer.cn two-stage
paragraph; zingnex.cn "two-stage inner-product quantization").
"""
import numpy as np
import pytest


def tables(orc, d, b, seed=0):
    pi64, s64, pi32, s32 = orc.make_rotation(d, seed)
    c = orc.lloyd_max(d, b - 1)[0].astype(np.float32)
    return pi32, s32, c


def rotated(pi32, x):
    xh = x / np.linalg.norm(x, axis=1, keepdims=True)
    return xh @ pi32.astype(np.float64).T


def midpoint_margin(y, c):
    c = c.astype(np.float64)
    t = 0.5 * (c[:-1] + c[1:])
    return np.min(np.abs(y[..., None] - t), axis=-1), t


@pytest.mark.parametrize("d,b", [(128, 2), (128, 3), (128, 4), (200, 4), (64, 3), (5, 4)])
def test_code_margin_is_distance_to_nearest_midpoint(orc, d, b):
    pi32, s32, c = tables(orc, d, b, seed=2)
    x = np.random.default_rng(100 + d + b).standard_normal((80, d)) * 1.3
    out = orc.quantize(d, b, pi32, s32, c, x, margins=True)
    y = rotated(pi32, x)
    want, t = midpoint_margin(y, c)
    np.testing.assert_allclose(out["code_margin"], want, rtol=1e-9, atol=1e-15)
    # distances to the centroids are a different quantity: a slip from
    # midpoints to centroids cannot pass the comparison above
    to_c = np.min(np.abs(y[..., None] - c.astype(np.float64)), axis=-1)
    assert np.max(np.abs(to_c - want)) > 1e-3
    # the code is the number of midpoints strictly below y (ties: lower index)
    idx, _ = orc.unpack_records(d, b, out["planes"])
    assert np.array_equal(idx, (y[..., None] > t).sum(axis=-1))


@pytest.mark.parametrize("d,b", [(128, 1), (128, 2), (128, 3), (200, 2)])
def test_code_margin_mse_mode(orc, d, b):
    pi32 = orc.make_rotation(d, 3)[2]
    c = orc.lloyd_max(d, b)[0].astype(np.float32)
    x = np.random.default_rng(7 * d + b).standard_normal((60, d))
    out = orc.quantize_mse(d, b, pi32, c, x, margins=True)
    y = rotated(pi32, x)
    want, t = midpoint_margin(y, c)
    np.testing.assert_allclose(out["code_margin"], want, rtol=1e-9, atol=1e-15)
    assert np.array_equal(orc.unpack_codes_mse(d, b, out["planes"]),
                          (y[..., None] > t).sum(axis=-1))


def _planted(pi32, j, target, base):
    """x with (Pi x / ||x||)_j == target up to double rounding: x = Pi^-1 v,
    v = base with v_j set so that v_j / ||Pi^-1 v|| = target (fixed point)."""
    P = pi32.astype(np.float64)
    v = base.copy()
    a = target
    for _ in range(40):
        v[j] = a
        x = np.linalg.solve(P, v)
        a = target * np.linalg.norm(x)
    v[j] = a
    return np.linalg.solve(P, v)


@pytest.mark.parametrize("b", [3, 4])
def test_planted_coordinates_on_and_near_a_midpoint(orc, b):
    d = 128
    pi32, s32, c = tables(orc, d, b, seed=5)
    t = 0.5 * (c[:-1].astype(np.float64) + c[1:].astype(np.float64))
    k = len(t) - 1                               # the largest midpoint (positive side)
    rng = np.random.default_rng(11)
    base = rng.standard_normal(d) / np.sqrt(d)
    rows = [_planted(pi32, 7, t[k], base),
            _planted(pi32, 7, t[k] + 2e-5, base),
            _planted(pi32, 7, t[k] - 2e-5, base),
            _planted(pi32, 9, t[0], base)]       # the lowest midpoint (negative side)
    out = orc.quantize(d, b, pi32, s32, c, np.array(rows), margins=True)
    cm = out["code_margin"]
    idx, _ = orc.unpack_records(d, b, out["planes"])
    assert cm[0, 7] < 1e-12 and idx[0, 7] in (k, k + 1)
    assert abs(cm[1, 7] - 2e-5) < 1e-12 and idx[1, 7] == k + 1
    assert abs(cm[2, 7] - 2e-5) < 1e-12 and idx[2, 7] == k
    assert cm[3, 9] < 1e-12 and idx[3, 9] in (0, 1)


@pytest.mark.parametrize("d,b", [(128, 4), (200, 3), (64, 2)])
def test_qjl_given_own_codes_equals_quantize(orc, d, b):
    pi32, s32, c = tables(orc, d, b, seed=1)
    x = np.random.default_rng(d * b).standard_normal((50, d)) * 2.0
    x[4] = 0.0
    ref = orc.quantize(d, b, pi32, s32, c, x, margins=True)
    idx, _ = orc.unpack_records(d, b, ref["planes"])
    got = orc.qjl_given_codes(d, b, pi32, s32, c, x, idx)
    assert np.array_equal(got["planes"], ref["planes"])
    assert np.array_equal(got["norms"], ref["norms"])
    np.testing.assert_allclose(got["sign_margin"], ref["sign_margin"], rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("d,b", [(128, 4), (200, 2)])
def test_qjl_given_other_codes_from_definition(orc, d, b):
    """Codes that are not the nearest centroids: the record keeps them, and the
    signs, margins and gamma follow r = x/||x|| - Pi^T c[idx], z = S r."""
    pi32, s32, c = tables(orc, d, b, seed=4)
    rng = np.random.default_rng(d + 13 * b)
    x = rng.standard_normal((30, d))
    K = 1 << (b - 1)
    idx = rng.integers(0, K, (30, d)).astype(np.int32)
    got = orc.qjl_given_codes(d, b, pi32, s32, c, x, idx)
    gi, gs = orc.unpack_records(d, b, got["planes"])
    assert np.array_equal(gi, idx)
    xh = x / np.linalg.norm(x, axis=1, keepdims=True)
    r = xh - c.astype(np.float64)[idx] @ pi32.astype(np.float64)
    z = r @ s32.astype(np.float64).T
    assert np.array_equal(gs, np.where(z >= 0, 1, -1))
    np.testing.assert_allclose(got["sign_margin"], np.abs(z), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(got["gamma"], np.linalg.norm(r, axis=1), rtol=1e-12)
    assert np.array_equal(got["norms"][:, 1],
                          np.linalg.norm(r, axis=1).astype(np.float16).view(np.uint16))
