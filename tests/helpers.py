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


def check_records(orc, d, b, pi, s, c, x, planes, norms):
    """GPU records of the rows x (float64 [n, d]) against the oracle: codes
    bit-exact except within CODE_MARGIN of a threshold, signs bit-exact
    except |z| < SIGN_MARGIN (in vectors whose codes all match), fp16 norms
    within one ulp.  Returns the number of exempt vectors."""
    ref = orc.quantize(d, b, pi, s, c, x, margins=True)
    gi, gs = orc.unpack_records(d, b, planes)
    ri, rs = orc.unpack_records(d, b, ref["planes"])
    code_bad = gi != ri
    assert not np.any(code_bad & (ref["code_margin"] >= CODE_MARGIN)), \
        f"code mismatch outside the margin: {np.argwhere(code_bad & (ref['code_margin'] >= CODE_MARGIN))[:5]}"
    same = ~code_bad.any(axis=1)
    sign_bad = (gs != rs) & same[:, None]
    assert not np.any(sign_bad & (ref["sign_margin"] >= SIGN_MARGIN)), \
        f"sign mismatch outside the margin: {np.argwhere(sign_bad & (ref['sign_margin'] >= SIGN_MARGIN))[:5]}"
    assert f16_ulp_diff(norms[:, 0], ref["norms"][:, 0]).max(initial=0) <= 1
    assert f16_ulp_diff(norms[same, 1], ref["norms"][same, 1]).max(initial=0) <= 1
    return int((~same).sum())
