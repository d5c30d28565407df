"""Pins for the oracle's fractional bit widths (two instances over a channel
split; CPU only).

The pages give quality at 2.5 and 3.5 bits per channel but not the mechanism;
the reading is two independent instances over contiguous channel groups.  The
expected values come from what that reading implies whatever the code does:
the code-bit count of a record pair, unbiasedness of the summed estimate over
seeds of the four random matrices (each instance's QJL estimate is unbiased:
zingnex.cn digest, "two-stage inner-product quantization"; admirer.cn article,
QJL paragraph), the Lloyd-Max distortion of each group weighted by the
group's energy, and exact reductions when one group is zero.
"""
import numpy as np
import pytest


def inst(orc, d, b, seed, mse=False):
    pi64, s64, pi32, s32 = orc.make_rotation(d, seed)
    if mse:
        return (d, b, pi32, None, orc.lloyd_max(d, b)[0].astype(np.float32))
    return (d, b, pi32, s32, orc.lloyd_max(d, b - 1)[0].astype(np.float32))


@pytest.mark.parametrize("dh,bh,dl,bl,bits", [
    (64, 3, 64, 2, 2.5), (64, 4, 64, 3, 3.5), (32, 3, 96, 2, 2.25), (96, 4, 32, 3, 3.75),
])
def test_split_code_bits_per_channel(orc, dh, bh, dl, bl, bits):
    """A record pair holds d_hi b_hi + d_lo b_lo code bits (whole 32-channel
    words per group) and two fp16 norm pairs."""
    hi, lo = inst(orc, dh, bh, 1), inst(orc, dl, bl, 2)
    x = np.random.default_rng(3).standard_normal((5, dh + dl))
    rh, rl = orc.split_quantize(hi, lo, x)
    words = rh["planes"].shape[1] + rl["planes"].shape[1]
    assert words * 32 == (dh * bh + dl * bl) == bits * (dh + dl)
    assert rh["norms"].shape == rl["norms"].shape == (5, 2)


def test_split_estimate_unbiased(orc):
    """Over seeds of both instances' (Pi, S): mean of the split estimate is
    <q, x> within 4 standard errors (variance from the per-instance closed
    form nu^2 [(pi/2) gamma^2 |q|^2 - <r, q>^2] / m, summed); the hi term alone
    misses <q_lo, x_lo> by far more."""
    dh, bh, dl, bl, T = 24, 3, 24, 2, 1500
    rng = np.random.default_rng(11)
    x = rng.standard_normal(dh + dl)
    x[:dh] *= 2.0                                   # louder first group
    q = x + 0.5 * rng.standard_normal(dh + dl)
    truth = float(q @ x)
    est, est_hi, var = np.empty(T), np.empty(T), np.empty(T)
    for t in range(T):
        hi, lo = inst(orc, dh, bh, 5000 + 2 * t), inst(orc, dl, bl, 5001 + 2 * t)
        rh, rl = orc.split_quantize(hi, lo, x[None], margins=True)
        est[t] = orc.split_estimate(hi, lo, q[None], (rh["planes"], rh["norms"]),
                                    (rl["planes"], rl["norms"]))[0, 0]
        est_hi[t] = orc.estimate(*hi, q[None, :dh], rh["planes"], rh["norms"])[0, 0]
        v = 0.0
        for (d, b, pi32, s32, c), r_, xs, qs in ((hi, rh, x[:dh], q[:dh]),
                                                 (lo, rl, x[dh:], q[dh:])):
            idx, _ = orc.unpack_records(d, b, r_["planes"])
            nu, ga = r_["nu"][0], r_["gamma"][0]
            r = xs / nu - c.astype(np.float64)[idx[0]] @ pi32.astype(np.float64)
            v += nu ** 2 * ((np.pi / 2) * ga ** 2 * (qs @ qs) - (r @ qs) ** 2) / d
        var[t] = v
    se = np.sqrt(var.mean() / T)
    # fp16 norms shift each estimate by at most ~2^-11 relative
    assert abs(est.mean() - truth) < 4 * se + 1e-3 * abs(truth)
    assert 0.7 < est.var() / var.mean() < 1.3
    assert abs(est_hi.mean() - truth) > 20 * se


@pytest.mark.parametrize("bh,bl", [(2, 1), (3, 2)])
def test_split_mse_distortion_energy_weighted(orc, bh, bl):
    """MSE-only instances, Gaussian rows whose first group is 3x louder:
    E|x - dequant(x)|^2 = E|x_hi|^2 D_bh(d_hi) + E|x_lo|^2 D_bl(d_lo), the
    Lloyd-Max distortions of the two codebooks (each group's direction is
    uniform on its sphere).  The swapped assignment predicts a value far off."""
    dh, dl, n = 32, 96, 20000
    hi, lo = inst(orc, dh, bh, 7, mse=True), inst(orc, dl, bl, 8, mse=True)
    rng = np.random.default_rng(12)
    x = rng.standard_normal((n, dh + dl))
    x[:, :dh] *= 3.0
    rh, rl = orc.split_quantize(hi, lo, x)
    xt = orc.split_dequantize(hi, lo, (rh["planes"], rh["norms"]), (rl["planes"], rl["norms"]))
    e2 = np.sum((x - xt) ** 2, axis=1)
    Dh, Dl = orc.lloyd_max(dh, bh)[1], orc.lloyd_max(dl, bl)[1]
    want = 9.0 * dh * Dh + dl * Dl
    swapped = 9.0 * dh * orc.lloyd_max(dh, bl)[1] + dl * orc.lloyd_max(dl, bh)[1]
    se = e2.std() / np.sqrt(n)
    assert abs(e2.mean() - want) < 4 * se + 1e-3 * want
    assert abs(e2.mean() - swapped) > 20 * se


def test_split_reduces_to_one_instance_when_a_group_is_zero(orc):
    """x_lo = 0: the lo records carry nu = 0, so the split estimate equals the
    hi instance's estimate on the first channels exactly, and the dequantized
    lo channels are 0; and symmetrically for x_hi = 0 (with a logit scale)."""
    dh, dl = 40, 24
    hi, lo = inst(orc, dh, 4, 21), inst(orc, dl, 3, 22)
    rng = np.random.default_rng(13)
    x = rng.standard_normal((6, dh + dl))
    q = rng.standard_normal((3, dh + dl))
    x0 = x.copy()
    x0[:, dh:] = 0.0
    rh, rl = orc.split_quantize(hi, lo, x0)
    assert np.all(rl["norms"][:, 0] == 0)
    s = orc.split_estimate(hi, lo, q, (rh["planes"], rh["norms"]), (rl["planes"], rl["norms"]))
    e = orc.estimate(*hi, q[:, :dh], rh["planes"], rh["norms"])
    np.testing.assert_array_equal(s, e)
    xt = orc.split_dequantize(hi, lo, (rh["planes"], rh["norms"]), (rl["planes"], rl["norms"]))
    assert np.all(xt[:, dh:] == 0.0)
    np.testing.assert_array_equal(xt[:, :dh], orc.dequantize(*hi, rh["planes"], rh["norms"]))
    x1 = x.copy()
    x1[:, :dh] = 0.0
    rh, rl = orc.split_quantize(hi, lo, x1)
    s = orc.split_estimate(hi, lo, q, (rh["planes"], rh["norms"]), (rl["planes"], rl["norms"]),
                           scale=0.37)
    np.testing.assert_array_equal(
        s, orc.estimate(*lo, q[:, dh:], rl["planes"], rl["norms"], scale=0.37))
