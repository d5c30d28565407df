"""Shared test helpers: oracle tables, tolerance checks, record utilities."""
import numpy as np

TOL = 1e-3          # relative tolerance on logits, scores and dequantized vectors
CODE_MARGIN = 1e-5  # codes may differ only this close to a decision threshold
SIGN_MARGIN = 1e-5  # signs may differ only where |z| is this small


def oracle_tables(orc, d, b, seed=0):
    pi64, s64, pi32, s32 = orc.make_rotation(d, seed)
    c = orc.lloyd_max(d, b - 1)[0].astype(np.float32)
    return pi32, s32, c


def rel_err_rows(got, ref):
    """max over elements of |got - ref| / max(|ref|, rms of ref's row)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True))
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(got - ref) / den)) if got.size else 0.0


def clear_padding(planes, d, b):
    """Zero the bits of coordinates >= d in records [n, W*b] (numpy uint32 or int32)."""
    W = (d + 31) // 32
    if d % 32 == 0:
        return planes
    keep = np.uint32((1 << (d % 32)) - 1)
    v = planes.view(np.uint32).reshape(-1, W, b)
    v[:, W - 1, :] &= keep
    return planes


def f16_ulp_diff(a, b):
    """|a - b| in units of fp16 ulps for non-negative fp16 bit patterns."""
    return np.abs(np.asarray(a, np.int64) - np.asarray(b, np.int64))


def exempt_bound(band):
    """Most exempt mismatches accepted out of `band` decisions whose oracle
    margin lies below the exemption threshold.  A kernel whose rotated
    coordinates (or sketch values) err by e flips only decisions with margin
    below e, so its mismatches are about e / 1e-5 of the band; the products
    here err by about 2^-22 (a few 1e-7), a few percent of the band.  A
    systematic error of 5e-6 would flip a quarter of it: 20% plus a small
    constant for counting noise separates the two."""
    return 3 + int(0.2 * band)


def _codes_signs_norms(orc, d, b, pi, s, c, x, gp, gn, ref, stats):
    gi, gs = orc.unpack_records(d, b, gp)
    ri, rs = orc.unpack_records(d, b, ref["planes"])
    code_bad = gi != ri
    band = ref["code_margin"] < CODE_MARGIN
    out = code_bad & ~band
    assert not out.any(), f"code mismatch outside the margin: {np.argwhere(out)[:5]}"
    nb = int(code_bad.sum())
    assert nb <= exempt_bound(int(band.sum())), (nb, int(band.sum()))
    stats.update(code_mismatch=nb, code_band=int(band.sum()))
    same = ~code_bad.any(axis=1)
    # norms: nu to one fp16 ulp everywhere
    assert f16_ulp_diff(gn[:, 0], ref["norms"][:, 0]).max(initial=0) <= 1
    # vectors whose codes all match: signs and gamma against the oracle
    sign_bad = (gs != rs) & same[:, None]
    sm = ref["sign_margin"]
    # sign exemption, literal reading (|z| < 1e-5): the one asserted; the
    # count under the scaled reading (|z| < 1e-5 sqrt(d)) is reported
    out = sign_bad & (sm >= SIGN_MARGIN)
    assert not out.any(), f"sign mismatch outside the margin: {np.argwhere(out)[:5]}"
    sband = (sm < SIGN_MARGIN) & same[:, None]
    assert int(sign_bad.sum()) <= exempt_bound(int(sband.sum())), (int(sign_bad.sum()), int(sband.sum()))
    stats.update(sign_mismatch=int(sign_bad.sum()), sign_band_literal=int(sband.sum()),
                 sign_band_scaled=int(((sm < SIGN_MARGIN * np.sqrt(d)) & same[:, None]).sum()))
    assert f16_ulp_diff(gn[same, 1], ref["norms"][same, 1]).max(initial=0) <= 1
    # vectors with an exempt code mismatch: their residual follows the GPU's
    # codes, so check signs and gamma against the oracle's second stage run
    # on those codes
    rows = np.flatnonzero(~same)
    if rows.size:
        alt = orc.qjl_given_codes(d, b, pi, s, c, x[rows], gi[rows])
        _, als = orc.unpack_records(d, b, alt["planes"])
        bad = (gs[rows] != als)
        out = bad & (alt["sign_margin"] >= SIGN_MARGIN)
        assert not out.any(), f"sign mismatch (GPU codes) outside the margin: {np.argwhere(out)[:5]}"
        assert f16_ulp_diff(gn[rows, 1], alt["norms"][:, 1]).max(initial=0) <= 1
    stats["exempt_vectors"] = int(rows.size)
    return stats


def check_records(orc, d, b, pi, s, c, x, planes, norms):
    """GPU records of the rows x (float64 [n, d]) against the oracle: codes
    bit-exact except within CODE_MARGIN of a threshold, and no more such
    mismatches than exempt_bound allows; signs bit-exact except |z| <
    SIGN_MARGIN; fp16 norms within one ulp.  For a vector with an exempt code
    mismatch the signs and gamma are checked against the oracle's second stage
    on the GPU's codes.  Returns counts (mismatches, decisions in the margin
    bands under both sign readings, exempt vectors)."""
    x = np.asarray(x, np.float64).reshape(-1, d)
    planes = np.asarray(planes).view(np.uint32).reshape(x.shape[0], -1)
    norms = np.asarray(norms).view(np.uint16).reshape(x.shape[0], 2)
    ref = orc.quantize(d, b, pi, s, c, x, margins=True)
    return _codes_signs_norms(orc, d, b, pi, s, c, x, planes, norms, ref, {})


def check_records_mse(orc, d, b, pi, c, x, planes, norms):
    """MSE-only records: codes as in check_records, nu within one fp16 ulp,
    the gamma slot 0."""
    x = np.asarray(x, np.float64).reshape(-1, d)
    planes = np.asarray(planes).view(np.uint32).reshape(x.shape[0], -1)
    norms = np.asarray(norms).view(np.uint16).reshape(x.shape[0], 2)
    ref = orc.quantize_mse(d, b, pi, c, x, margins=True)
    gi = orc.unpack_codes_mse(d, b, planes)
    ri = orc.unpack_codes_mse(d, b, ref["planes"])
    bad = gi != ri
    band = ref["code_margin"] < CODE_MARGIN
    assert not np.any(bad & ~band), np.argwhere(bad & ~band)[:5]
    assert int(bad.sum()) <= exempt_bound(int(band.sum())), (int(bad.sum()), int(band.sum()))
    assert f16_ulp_diff(norms[:, 0], ref["norms"][:, 0]).max(initial=0) <= 1
    assert np.all(norms[:, 1] == 0)
    return {"code_mismatch": int(bad.sum()), "code_band": int(band.sum())}


def topk_order_ok(gi, gs):
    """Rows of a top-k result in (score desc, index asc) order: a later entry
    has a lower score, or an equal score and a higher index."""
    gi = np.asarray(gi)
    gs = np.asarray(gs)
    s0, s1 = gs[:, :-1], gs[:, 1:]
    i0, i1 = gi[:, :-1], gi[:, 1:]
    valid = i1 >= 0                      # -1 pads rows with fewer than k records
    ok = (s0 > s1) | ((s0 == s1) & (i0 < i1))
    return bool(np.all(ok | ~valid))
