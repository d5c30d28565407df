"""Pins for the oracle's quantizer, estimator, dequantizer and top-k (CPU only).

The expected values come from mathematics that holds whatever the code does:
brute force over the product codebook, the Lloyd-Max distortion of the
codebook (rotated unit vectors are uniform on the sphere), the unbiasedness of
the QJL correction (zingnex.cn digest, "two-stage inner-product quantization";
admirer.cn article, QJL paragraph), the bias of the MSE-only stage (same
sections: the MSE quantizer is biased for inner products), numpy's sort and
numpy's float16 rounding.
"""
import itertools

import numpy as np
import pytest


def tables(orc, d, b, seed=0):
    pi64, s64, pi32, s32 = orc.make_rotation(d, seed)
    c = orc.lloyd_max(d, b - 1)[0].astype(np.float32)
    return pi32, s32, c


def unit_rows(rng, n, d):
    g = rng.standard_normal((n, d))
    return g / np.linalg.norm(g, axis=1, keepdims=True)


def test_pack_unpack_roundtrip(orc):
    rng = np.random.default_rng(1)
    for d, b in [(128, 2), (128, 4), (200, 3), (5, 4), (33, 2)]:
        K = 1 << (b - 1)
        idx = rng.integers(0, K, d).astype(np.int32)
        sg = np.where(rng.random(d) < 0.5, -1, 1).astype(np.int32)
        rec = orc.pack_record(d, b, idx, sg)
        assert rec.size == orc.words_per_plane(d) * b
        i2, s2 = orc.unpack_records(d, b, rec[None])
        assert np.array_equal(i2[0], idx) and np.array_equal(s2[0], sg)
        # canonical layout: word (w, p) bit j%32 is bit p of idx_j / the sign bit
        W = orc.words_per_plane(d)
        for j in range(d):
            w, bit = divmod(j, 32)
            for p in range(b - 1):
                assert (rec[w * b + p] >> bit) & 1 == (idx[j] >> p) & 1
            assert (rec[w * b + b - 1] >> bit) & 1 == (sg[j] > 0)
        # padding bits of coordinates >= d are zero
        if d % 32:
            pad = np.uint32(((1 << 32) - 1) ^ ((1 << (d % 32)) - 1))
            for p in range(b):
                assert rec[(W - 1) * b + p] & pad == 0


def test_all_codes_roundtrip_tiny(orc):
    d, b = 3, 4
    for code in itertools.product(range(8), repeat=d):
        for sg in itertools.product([-1, 1], repeat=d):
            rec = orc.pack_record(d, b, np.array(code), np.array(sg))
            i2, s2 = orc.unpack_records(d, b, rec[None])
            assert tuple(i2[0]) == code and tuple(s2[0]) == sg


@pytest.mark.parametrize("d", [3, 4, 5])
@pytest.mark.parametrize("b", [2, 3, 4])
def test_nearest_centroid_exhaustive(orc, d, b):
    """Per-coordinate argmin == argmin over all K^d product-codebook vectors."""
    pi32, s32, c = tables(orc, d, b, seed=3)
    K = 1 << (b - 1)
    rng = np.random.default_rng(d * 10 + b)
    x = rng.standard_normal((60, d))
    out = orc.quantize(d, b, pi32, s32, c, x, margins=True)
    idx, _ = orc.unpack_records(d, b, out["planes"])
    book = np.array(list(itertools.product(range(K), repeat=d)))   # K^d x d
    vecs = c.astype(np.float64)[book]                                # codewords in rotated space
    for i in range(x.shape[0]):
        dist = ((out["y"][i][None, :] - vecs) ** 2).sum(1)
        best = book[np.argmin(dist)]
        assert np.array_equal(best, idx[i])


def test_rotation_orthogonal_and_qr(orc):
    for d in [8, 128, 200]:
        pi64, s64, pi32, s32 = orc.make_rotation(d, 0)
        assert np.abs(pi64.T @ pi64 - np.eye(d)).max() < 1e-12
        assert np.abs(pi32.astype(np.float64).T @ pi32 - np.eye(d)).max() < 1e-6
        G = orc.rng_normals(0, 0, d * d).reshape(d, d)
        Q, R = np.linalg.qr(G)                      # LAPACK
        Q = Q * np.sign(np.diag(R))
        assert np.abs(Q - pi64).max() < 1e-11
        # R = Pi^T G is upper triangular with a positive diagonal
        R2 = pi64.T @ G
        assert np.abs(np.tril(R2, -1)).max() < 1e-10 and np.all(np.diag(R2) > 0)
        assert np.array_equal(s64, orc.rng_normals(0, 1, d * d).reshape(d, d))
        assert np.array_equal(pi32, pi64.astype(np.float32))
    a = orc.make_rotation(64, 5)[2]
    assert np.array_equal(a, orc.make_rotation(64, 5)[2])
    assert not np.array_equal(a, orc.make_rotation(64, 6)[2])


def test_rotated_coordinates_follow_beta(orc):
    """Coordinates of Pi x for unit x follow f_d (turboquant.net, PolarQuant)."""
    from scipy import stats
    d = 128
    pi32, s32, c = tables(orc, d, 3)
    x = unit_rows(np.random.default_rng(2), 3000, d)
    y = orc.quantize(d, 3, pi32, s32, c, x, margins=True)["y"]
    a = (d - 1) / 2
    for j in [0, 17, 127]:
        p = stats.kstest((1 + y[:, j]) / 2, stats.beta(a, a).cdf).pvalue
        assert p > 1e-4


@pytest.mark.parametrize("b", [2, 3, 4])
def test_mse_matches_lloyd_distortion(orc, b):
    """E||x - Pi^T c[idx]||^2 over unit x equals the Lloyd-Max distortion D."""
    d = 128
    pi32, s32, c = tables(orc, d, b)
    D = orc.lloyd_max(d, b - 1)[1]
    x = unit_rows(np.random.default_rng(b), 20000, d)
    out = orc.quantize(d, b, pi32, s32, c, x, margins=True)
    g2 = out["gamma"] ** 2
    se = g2.std() / np.sqrt(g2.size)
    assert abs(g2.mean() - D) < 4 * se + 1e-6
    # reconstruct the residual from the packed codes and compare its norm
    idx, _ = orc.unpack_records(d, b, out["planes"][:50])
    recon = c.astype(np.float64)[idx] @ pi32.astype(np.float64)
    np.testing.assert_allclose(np.linalg.norm(x[:50] - recon, axis=1), out["gamma"][:50],
                               rtol=1e-12)


def test_norms_fp16_and_zero_vector(orc):
    d, b = 128, 3
    pi32, s32, c = tables(orc, d, b)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((20, d)) * 3
    x[5] = 0.0
    out = orc.quantize(d, b, pi32, s32, c, x, margins=True)
    nx = np.linalg.norm(x, axis=1).astype(np.float16).view(np.uint16)
    assert np.array_equal(out["norms"][:, 0], nx)
    ng = out["gamma"].astype(np.float16).view(np.uint16)
    assert np.array_equal(out["norms"][:, 1], ng)
    # zero vector: nu = gamma = 0, codes of y = 0 (tie -> lower index K/2-1), signs +1
    idx, sg = orc.unpack_records(d, b, out["planes"][5:6])
    K = 1 << (b - 1)
    assert np.all(idx == K // 2 - 1) and np.all(sg == 1)
    assert out["norms"][5, 0] == 0 and out["norms"][5, 1] == 0
    # exactly b*d bits of codes + 2 fp16 per vector, no per-block constants
    assert out["planes"].shape[1] * 32 == b * d and out["norms"].shape[1] == 2


def test_signs_are_sign_of_sketch_of_residual(orc):
    d, b = 64, 3
    pi32, s32, c = tables(orc, d, b)
    x = np.random.default_rng(5).standard_normal((30, d))
    out = orc.quantize(d, b, pi32, s32, c, x, margins=True)
    idx, sg = orc.unpack_records(d, b, out["planes"])
    xh = x / np.linalg.norm(x, axis=1, keepdims=True)
    r = xh - c.astype(np.float64)[idx] @ pi32.astype(np.float64)
    z = r @ s32.astype(np.float64).T
    assert np.array_equal(np.where(z >= 0, 1, -1), sg)
    np.testing.assert_allclose(np.abs(z), out["sign_margin"], rtol=1e-10, atol=1e-14)


def test_estimate_equals_inner_product_with_dequant(orc):
    """est(q, x) == <q, dequant(x)> for every q (linearity of the estimator)."""
    for d, b in [(128, 4), (200, 2), (64, 3)]:
        pi32, s32, c = tables(orc, d, b)
        rng = np.random.default_rng(d + b)
        x = rng.standard_normal((40, d))
        q = rng.standard_normal((7, d))
        out = orc.quantize(d, b, pi32, s32, c, x)
        est = orc.estimate(d, b, pi32, s32, c, q, out["planes"], out["norms"], scale=0.5)
        xt = orc.dequantize(d, b, pi32, s32, c, out["planes"], out["norms"])
        np.testing.assert_allclose(est, 0.5 * q @ xt.T, rtol=1e-10, atol=1e-10)
        # unit-vector queries read the dequantized coordinates back
        e = orc.estimate(d, b, pi32, s32, c, np.eye(d), out["planes"], out["norms"])
        np.testing.assert_allclose(e.T, xt, rtol=1e-10, atol=1e-12)


def test_dequant_without_residual_is_rotation_back(orc):
    """gamma = 0 -> dequant = nu * Pi^T c[idx] (turboquant.net pseudo-code dequant)."""
    d, b = 32, 3
    pi32, s32, c = tables(orc, d, b)
    out = orc.quantize(d, b, pi32, s32, c, np.random.default_rng(7).standard_normal((5, d)))
    norms = out["norms"].copy()
    norms[:, 1] = 0
    xt = orc.dequantize(d, b, pi32, s32, c, out["planes"], norms)
    idx, _ = orc.unpack_records(d, b, out["planes"])
    nu = norms[:, 0].view(np.float16).astype(np.float64)
    np.testing.assert_allclose(xt, nu[:, None] * (c.astype(np.float64)[idx] @ pi32.astype(np.float64)),
                               rtol=1e-12, atol=1e-14)


def test_qjl_unbiased_and_mse_stage_biased(orc):
    """Over seeds of (Pi, S): the two-stage estimate is unbiased with the
    closed-form variance nu^2 [(pi/2) gamma^2 |q|^2 - <r,q>^2] / m, while the
    MSE-only stage at 1 bit is biased by the factor 1 - D_1 = d E|X|^2."""
    d, b, T = 48, 2, 3000
    rng = np.random.default_rng(8)
    x = rng.standard_normal(d)
    q = x + 0.5 * rng.standard_normal(d)
    truth = float(q @ x)
    c = orc.lloyd_max(d, b - 1)[0].astype(np.float32)
    est2, est1, var = np.empty(T), np.empty(T), np.empty(T)
    for t in range(T):
        pi64, s64, pi32, s32 = orc.make_rotation(d, 1000 + t)
        out = orc.quantize(d, b, pi32, s32, c, x[None], margins=True)
        nu, ga = out["nu"], out["gamma"]
        est2[t] = orc.estimate(d, b, pi32, s32, c, q[None], out["planes"], out["norms"],
                               nu_exact=nu, gamma_exact=ga)[0, 0]
        est1[t] = orc.estimate(d, b, pi32, s32, c, q[None], out["planes"], out["norms"],
                               nu_exact=nu, gamma_exact=np.zeros(1))[0, 0]
        idx, _ = orc.unpack_records(d, b, out["planes"])
        r = x / nu[0] - c.astype(np.float64)[idx[0]] @ pi32.astype(np.float64)
        var[t] = nu[0] ** 2 * ((np.pi / 2) * ga[0] ** 2 * (q @ q) - (r @ q) ** 2) / d
    # given Pi the estimate is unbiased, so its total variance is the mean of
    # the conditional (closed-form) variances
    se = np.sqrt(var.mean() / T)
    assert 0.7 < est2.var() / var.mean() < 1.3
    assert abs(est2.mean() - truth) < 4 * se
    D1 = orc.lloyd_max(d, 1)[1]
    se1 = est1.std() / np.sqrt(T)
    assert abs(est1.mean() - (1 - D1) * truth) < 4 * se1
    assert abs(est1.mean() - truth) > 20 * se1          # the bias is detected


def test_qjl_sign_identity_monte_carlo():
    """E[sign(<s,r>) <s,q>] = sqrt(2/pi) <r,q> / |r| for s ~ N(0, I)."""
    rng = np.random.default_rng(9)
    d = 16
    r, q = rng.standard_normal(d), rng.standard_normal(d)
    s = rng.standard_normal((400000, d))
    v = np.sign(s @ r) * (s @ q)
    want = np.sqrt(2 / np.pi) * (r @ q) / np.linalg.norm(r)
    assert abs(v.mean() - want) < 4 * v.std() / np.sqrt(v.size)


def test_topk_matches_lexsort(orc):
    rng = np.random.default_rng(10)
    sc = np.round(rng.standard_normal((6, 500)), 1)     # many ties
    idx, val = orc.topk(sc, 10)
    for a in range(6):
        order = np.lexsort((np.arange(500), -sc[a]))[:10]
        assert np.array_equal(idx[a], order) and np.array_equal(val[a], sc[a, order])
    idx, val = orc.topk(sc[:, :4], 6)
    assert np.all(idx[:, 4:] == -1)


# ---------------------------------------------------------------- MSE-only mode
# turboquant.net pseudo-code "quant" / "dequant": b-bit Lloyd-Max codes of the
# rotated coordinates, no QJL stage.
def mse_tables(orc, d, b, seed=0):
    pi64, s64, pi32, s32 = orc.make_rotation(d, seed)
    return pi32, orc.lloyd_max(d, b)[0].astype(np.float32)


@pytest.mark.parametrize("b", [1, 2, 3])
def test_mse_mode_distortion(orc, b):
    """Unit x (nu16 = 1 exactly): E||x - dequant(x)||^2 equals the Lloyd-Max
    distortion of the b-bit codebook, decreasing in b; at b = 1 it is the
    closed form 1 - d E|X|^2 with E|X| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))."""
    from scipy.special import gammaln
    d = 128
    pi32, c = mse_tables(orc, d, b)
    D = orc.lloyd_max(d, b)[1]
    x = unit_rows(np.random.default_rng(30 + b), 20000, d)
    rec = orc.quantize_mse(d, b, pi32, c, x)
    assert np.all(rec["norms"][:, 0] == np.float16(1.0).view(np.uint16))
    assert np.all(rec["norms"][:, 1] == 0)
    xt = orc.dequantize_mse(d, b, pi32, c, rec["planes"], rec["norms"])
    e2 = np.sum((x - xt) ** 2, axis=1)
    assert abs(e2.mean() - D) < 4 * e2.std() / np.sqrt(e2.size) + 1e-6
    if b == 1:
        eabs = np.exp(gammaln(d / 2) - 0.5 * np.log(np.pi) - gammaln((d + 1) / 2))
        assert abs(D - (1 - d * eabs ** 2)) < 1e-9
    if b > 1:
        assert D < orc.lloyd_max(d, b - 1)[1]


@pytest.mark.parametrize("b", [1, 2, 3])
def test_mse_codes_equal_two_stage_codes(orc, b):
    """The MSE record's codes are the code planes of the (b+1)-bit two-stage
    record (same b-bit codebook, same rotation)."""
    d = 200
    pi64, s64, pi32, s32 = orc.make_rotation(d, 4)
    c = orc.lloyd_max(d, b)[0].astype(np.float32)
    x = np.random.default_rng(40 + b).standard_normal((300, d))
    m = orc.quantize_mse(d, b, pi32, c, x)
    t = orc.quantize(d, b + 1, pi32, s32, c, x)
    idx_t, _ = orc.unpack_records(d, b + 1, t["planes"])
    assert np.array_equal(orc.unpack_codes_mse(d, b, m["planes"]), idx_t)
    assert np.array_equal(m["norms"][:, 0], t["norms"][:, 0])


@pytest.mark.parametrize("d", [3, 4])
@pytest.mark.parametrize("b", [1, 2])
def test_mse_nearest_centroid_exhaustive(orc, d, b):
    pi32, c = mse_tables(orc, d, b, seed=5)
    K = 1 << b
    x = np.random.default_rng(d + 7 * b).standard_normal((50, d))
    idx = orc.unpack_codes_mse(d, b, orc.quantize_mse(d, b, pi32, c, x)["planes"])
    y = (x / np.linalg.norm(x, axis=1, keepdims=True)) @ pi32.astype(np.float64).T
    cb = np.array(list(itertools.product(range(K), repeat=d)))
    dist = ((y[:, None, :] - c.astype(np.float64)[cb][None]) ** 2).sum(axis=2)
    assert np.array_equal(cb[np.argmin(dist, axis=1)], idx)


def test_mse_estimate_and_zero_vector(orc):
    d, b = 96, 3
    pi32, c = mse_tables(orc, d, b, seed=6)
    rng = np.random.default_rng(9)
    x = rng.standard_normal((40, d))
    x[3] = 0.0
    q = rng.standard_normal((5, d))
    rec = orc.quantize_mse(d, b, pi32, c, x)
    xt = orc.dequantize_mse(d, b, pi32, c, rec["planes"], rec["norms"])
    est = orc.estimate_mse(d, b, pi32, c, q, rec["planes"], rec["norms"], scale=0.5)
    np.testing.assert_allclose(est, 0.5 * q @ xt.T, rtol=1e-11, atol=1e-12)
    # y = 0: every coordinate ties between c[K/2 - 1] and c[K/2] -> lower index
    assert np.all(orc.unpack_codes_mse(d, b, rec["planes"][3:4]) == (1 << (b - 1)) - 1)
    assert np.all(rec["norms"][3] == 0) and np.all(xt[3] == 0)
