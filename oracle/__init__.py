"""CPU oracle for the TurboQuant hot path -- TEST INFRASTRUCTURE ONLY.

Plain double-precision C (``tq_oracle.c``) behind ctypes and numpy.  Only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package; the product library never does, and the
two share no code.  Every function states what it computes; the C source cites
the passages of the pages it follows.

Parity unpinned: none of the pages prints a worked numeric example (no code
values, logits or recall figures survive on them), so absolute code values for
a given seed are pinned only through the checks in ``tests/test_oracle_*.py``
(closed forms, invariants, Monte-Carlo identities, brute force at tiny d).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        u64, i64, i32, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        P = ctypes.c_void_p
        L.orc_splitmix64.restype = u64
        L.orc_splitmix64.argtypes = [u64, u64]
        L.orc_rng_u64.restype = u64
        L.orc_rng_u64.argtypes = [u64, u64, u64]
        L.orc_rng_uniform.restype = dbl
        L.orc_rng_uniform.argtypes = [u64, u64, u64]
        L.orc_rng_normals.restype = None
        L.orc_rng_normals.argtypes = [u64, u64, i64, P]
        L.orc_f16_from_double.restype = ctypes.c_uint16
        L.orc_f16_from_double.argtypes = [dbl]
        L.orc_f16_to_double.restype = dbl
        L.orc_f16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_make_rotation.restype = ctypes.c_int
        L.orc_make_rotation.argtypes = [i32, u64, P, P, P, P]
        L.orc_beta_density.restype = dbl
        L.orc_beta_density.argtypes = [i32, dbl]
        L.orc_beta_integral.restype = dbl
        L.orc_beta_integral.argtypes = [i32, i32, dbl, dbl]
        L.orc_lloyd_max.restype = ctypes.c_int
        L.orc_lloyd_max.argtypes = [i32, i32, i32, dbl, P, P, P, P]
        L.orc_words_per_plane.restype = i32
        L.orc_words_per_plane.argtypes = [i32]
        L.orc_pack_record.restype = None
        L.orc_pack_record.argtypes = [i32, i32, P, P, P]
        L.orc_unpack_record.restype = None
        L.orc_unpack_record.argtypes = [i32, i32, P, P, P]
        L.orc_quantize.restype = None
        L.orc_quantize.argtypes = [i32, i32, P, P, P, i64, P, i64, P, P, P, P, P, P, P]
        L.orc_qjl_given_codes.restype = None
        L.orc_qjl_given_codes.argtypes = [i32, i32, P, P, P, i64, P, i64, P, P, P, P, P]
        L.orc_dequantize.restype = None
        L.orc_dequantize.argtypes = [i32, i32, P, P, P, i64, P, P, P, i64]
        L.orc_estimate.restype = None
        L.orc_estimate.argtypes = [i32, i32, P, P, P, i64, P, i64, i64, P, P, P, P, dbl, P]
        L.orc_quantize_mse.restype = None
        L.orc_quantize_mse.argtypes = [i32, i32, P, P, i64, P, i64, P, P, P]
        L.orc_dequantize_mse.restype = None
        L.orc_dequantize_mse.argtypes = [i32, i32, P, P, i64, P, P, P, i64]
        L.orc_estimate_mse.restype = None
        L.orc_estimate_mse.argtypes = [i32, i32, P, P, i64, P, i64, i64, P, P, dbl, P]
        L.orc_topk.restype = None
        L.orc_topk.argtypes = [i64, i64, P, i32, P, P]
        L.orc_num_threads.restype = i32
        L.orc_num_threads.argtypes = []
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def words_per_plane(d):
    return (d + 31) // 32


def record_words(d, b):
    return words_per_plane(d) * b


# --- random generator -----------------------------------------------------
def splitmix64(state, i):
    return lib().orc_splitmix64(state, i)


def rng_u64(seed, stream, i):
    return lib().orc_rng_u64(seed, stream, i)


def rng_uniform(seed, stream, i):
    return lib().orc_rng_uniform(seed, stream, i)


def rng_normals(seed, stream, n):
    out = np.empty(n, np.float64)
    lib().orc_rng_normals(seed, stream, n, _p(out))
    return out


# --- fp16 -----------------------------------------------------------------
def f16_from_double(v):
    return lib().orc_f16_from_double(float(v))


def f16_to_double(h):
    return lib().orc_f16_to_double(int(h))


# --- setup tables ---------------------------------------------------------
def make_rotation(d, seed):
    """Return (pi64, s64, pi32, s32): Pi (Householder QR of stream-0 Gaussians,
    diag(R) > 0) and S (stream-1 Gaussians), row-major d x d."""
    pi64 = np.empty((d, d), np.float64)
    s64 = np.empty((d, d), np.float64)
    pi32 = np.empty((d, d), np.float32)
    s32 = np.empty((d, d), np.float32)
    rc = lib().orc_make_rotation(d, seed, _p(pi64), _p(s64), _p(pi32), _p(s32))
    if rc != 0:
        raise ValueError(f"orc_make_rotation failed ({rc})")
    return pi64, s64, pi32, s32


def beta_density(d, x):
    return lib().orc_beta_density(d, float(x))


def beta_integral(d, p, a, b):
    """int_a^b x^p f_d(x) dx for p in {0, 1, 2}."""
    return lib().orc_beta_integral(d, p, float(a), float(b))


def lloyd_max(d, bits, max_iter=100000, tol=1e-13, history=False):
    """Lloyd-Max centroids (ascending, 2**bits of them) of f_d.

    Returns (centroids float64, distortion, iters, converged[, history])."""
    K = 1 << bits
    c = np.empty(K, np.float64)
    dist = ctypes.c_double(0.0)
    it = ctypes.c_int32(0)
    hist = np.full(max_iter, np.nan) if history else None
    rc = lib().orc_lloyd_max(d, bits, max_iter, tol, _p(c), ctypes.byref(dist),
                             ctypes.byref(it), _p(hist))
    if rc < 0:
        raise ValueError("orc_lloyd_max: bad arguments")
    res = (c, dist.value, it.value, rc == 0)
    if history:
        res = res + (hist[: it.value],)
    return res


# --- records --------------------------------------------------------------
def pack_record(d, b, idx, sgn):
    rec = np.empty(record_words(d, b), np.uint32)
    lib().orc_pack_record(d, b, _p(_c(idx, np.int32)), _p(_c(sgn, np.int32)), _p(rec))
    return rec


def unpack_records(d, b, planes):
    """planes: uint32 [n, W*b] -> (idx int32 [n, d], sign int32 [n, d] in {-1, +1})."""
    planes = _c(planes, np.uint32).reshape(-1, record_words(d, b))
    n = planes.shape[0]
    idx = np.empty((n, d), np.int32)
    sg = np.empty((n, d), np.int32)
    L = lib()
    for i in range(n):
        L.orc_unpack_record(d, b, _p(planes[i]), _p(idx[i]), _p(sg[i]))
    return idx, sg


# --- hot path -------------------------------------------------------------
def quantize(d, b, pi32, s32, cen32, x, margins=False):
    """Quantize rows of x (float64 [n, d]).  Returns dict with planes
    (uint32 [n, W*b]), norms (uint16 [n, 2]), and, with margins=True,
    code_margin, sign_margin ([n, d]), nu, gamma ([n]) and y ([n, d])."""
    x = _c(x, np.float64).reshape(-1, d)
    n = x.shape[0]
    planes = np.empty((n, record_words(d, b)), np.uint32)
    norms = np.empty((n, 2), np.uint16)
    out = {"planes": planes, "norms": norms}
    cm = sm = nu = ga = y = None
    if margins:
        cm = np.empty((n, d)); sm = np.empty((n, d))
        nu = np.empty(n); ga = np.empty(n); y = np.empty((n, d))
        out.update(code_margin=cm, sign_margin=sm, nu=nu, gamma=ga, y=y)
    lib().orc_quantize(d, b, _p(_c(pi32, np.float32)), _p(_c(s32, np.float32)),
                       _p(_c(cen32, np.float32)), n, _p(x), d, _p(planes), _p(norms),
                       _p(cm), _p(sm), _p(nu), _p(ga), _p(y))
    return out


def qjl_given_codes(d, b, pi32, s32, cen32, x, idx):
    """The QJL stage for given codes idx (int [n, d]) instead of the nearest
    centroids: returns dict with planes (the given codes and the signs of
    S (x/||x|| - Pi^T c[idx])), norms (uint16 [n, 2]), sign_margin ([n, d])
    and gamma ([n], unrounded)."""
    x = _c(x, np.float64).reshape(-1, d)
    idx = _c(idx, np.int32).reshape(-1, d)
    n = x.shape[0]
    assert idx.shape[0] == n
    planes = np.empty((n, record_words(d, b)), np.uint32)
    norms = np.empty((n, 2), np.uint16)
    sm = np.empty((n, d))
    ga = np.empty(n)
    lib().orc_qjl_given_codes(d, b, _p(_c(pi32, np.float32)), _p(_c(s32, np.float32)),
                              _p(_c(cen32, np.float32)), n, _p(x), d, _p(idx), _p(planes),
                              _p(norms), _p(sm), _p(ga))
    return {"planes": planes, "norms": norms, "sign_margin": sm, "gamma": ga}


def quantize_mse(d, b, pi32, cen32, x, margins=False):
    """MSE-only variant: b code planes, no QJL stage.  Returns dict with planes
    (uint32 [n, W*b]), norms (uint16 [n, 2], gamma slot 0) and, with
    margins=True, code_margin ([n, d])."""
    x = _c(x, np.float64).reshape(-1, d)
    n = x.shape[0]
    planes = np.empty((n, record_words(d, b)), np.uint32)
    norms = np.empty((n, 2), np.uint16)
    cm = np.empty((n, d)) if margins else None
    lib().orc_quantize_mse(d, b, _p(_c(pi32, np.float32)), _p(_c(cen32, np.float32)), n, _p(x), d,
                           _p(planes), _p(norms), _p(cm))
    out = {"planes": planes, "norms": norms}
    if margins:
        out["code_margin"] = cm
    return out


def dequantize_mse(d, b, pi32, cen32, planes, norms):
    planes = _c(planes, np.uint32).reshape(-1, record_words(d, b))
    norms = _c(norms, np.uint16).reshape(-1, 2)
    n = planes.shape[0]
    out = np.empty((n, d), np.float64)
    lib().orc_dequantize_mse(d, b, _p(_c(pi32, np.float32)), _p(_c(cen32, np.float32)), n,
                             _p(planes), _p(norms), _p(out), d)
    return out


def estimate_mse(d, b, pi32, cen32, q, planes, norms, scale=1.0):
    """out[a, i] = scale * nu_i * <Pi q_a, c[idx_i]> (MSE-only records)."""
    q = _c(q, np.float64).reshape(-1, d)
    planes = _c(planes, np.uint32).reshape(-1, record_words(d, b))
    norms = _c(norms, np.uint16).reshape(-1, 2)
    nq, n = q.shape[0], planes.shape[0]
    out = np.empty((nq, n), np.float64)
    lib().orc_estimate_mse(d, b, _p(_c(pi32, np.float32)), _p(_c(cen32, np.float32)), nq, _p(q),
                           d, n, _p(planes), _p(norms), float(scale), _p(out))
    return out


def unpack_codes_mse(d, b, planes):
    """uint32 [n, W*b] MSE records -> idx int32 [n, d] (numpy, for tests)."""
    planes = _c(planes, np.uint32).reshape(-1, (d + 31) // 32, b)
    j = np.arange(d)
    bits = (planes[:, j // 32, :] >> (j % 32)[None, :, None].astype(np.uint32)) & 1
    return (bits.astype(np.int32) << np.arange(b)[None, None, :]).sum(axis=2).astype(np.int32)


def dequantize(d, b, pi32, s32, cen32, planes, norms):
    planes = _c(planes, np.uint32).reshape(-1, record_words(d, b))
    norms = _c(norms, np.uint16).reshape(-1, 2)
    n = planes.shape[0]
    out = np.empty((n, d), np.float64)
    lib().orc_dequantize(d, b, _p(_c(pi32, np.float32)), _p(_c(s32, np.float32)),
                         _p(_c(cen32, np.float32)), n, _p(planes), _p(norms), _p(out), d)
    return out


def estimate(d, b, pi32, s32, cen32, q, planes, norms, scale=1.0, nu_exact=None,
             gamma_exact=None):
    """out[a, i] = scale * nu_i * (<Pi q_a, c[idx_i]> + alpha gamma_i <S q_a, s_i>)."""
    q = _c(q, np.float64).reshape(-1, d)
    planes = _c(planes, np.uint32).reshape(-1, record_words(d, b))
    norms = _c(norms, np.uint16).reshape(-1, 2)
    nq, n = q.shape[0], planes.shape[0]
    out = np.empty((nq, n), np.float64)
    ne = None if nu_exact is None else _c(nu_exact, np.float64)
    ge = None if gamma_exact is None else _c(gamma_exact, np.float64)
    lib().orc_estimate(d, b, _p(_c(pi32, np.float32)), _p(_c(s32, np.float32)),
                       _p(_c(cen32, np.float32)), nq, _p(q), d, n, _p(planes), _p(norms),
                       _p(ne), _p(ge), float(scale), _p(out))
    return out


def topk(scores, k):
    scores = _c(scores, np.float64)
    nq, n = scores.shape
    idx = np.empty((nq, k), np.int64)
    sc = np.empty((nq, k), np.float64)
    lib().orc_topk(nq, n, _p(scores), k, _p(idx), _p(sc))
    return idx, sc


def num_threads():
    return lib().orc_num_threads()


# --- fractional bit widths: two instances over a channel split ------------
# The pages quote quality at 2.5 and 3.5 bits per channel (zingnex.cn digest,
# section on theoretical guarantees and experiments; turboquant.net, the KV
# cache compression benchmark table; admirer.cn article, LongBench paragraph)
# without saying how a fractional width is formed.  Reading taken here: the
# channels are split in two contiguous groups, the first d_hi channels at
# b_hi bits and the other d_lo at b_lo, each group quantized by its own
# instance (own rotation, projection and codebook of its own dimension), so
# a record pair costs d_hi b_hi + d_lo b_lo code bits.  The estimate of
# <q, k> is the sum of the two instances' estimates over their channels (each
# unbiased, so the sum is), and a dequantized vector is the concatenation.
# An instance is a tuple (d, b, pi32, s32, cen32); s32 None marks an
# MSE-only instance (b code planes, cen32 of 2^b centroids).
def _inst_quantize(inst, x, margins):
    d, b, pi32, s32, cen32 = inst
    if s32 is None:
        return quantize_mse(d, b, pi32, cen32, x, margins=margins)
    return quantize(d, b, pi32, s32, cen32, x, margins=margins)


def split_quantize(hi, lo, x, margins=False):
    """Rows of x (float64 [n, d_hi + d_lo]) -> (records of the first d_hi
    channels under `hi`, records of the remaining d_lo channels under `lo`),
    each as returned by quantize / quantize_mse."""
    dh, dl = hi[0], lo[0]
    x = _c(x, np.float64).reshape(-1, dh + dl)
    return _inst_quantize(hi, x[:, :dh], margins), _inst_quantize(lo, x[:, dh:], margins)


def _inst_estimate(inst, q, planes, norms, scale):
    d, b, pi32, s32, cen32 = inst
    if s32 is None:
        return estimate_mse(d, b, pi32, cen32, q, planes, norms, scale=scale)
    return estimate(d, b, pi32, s32, cen32, q, planes, norms, scale=scale)


def split_estimate(hi, lo, q, rec_hi, rec_lo, scale=1.0):
    """out[a, i] = est_hi(q_a[:d_hi], record i of hi) + est_lo(q_a[d_hi:],
    record i of lo), each the instance's own estimate, times scale.
    rec_hi / rec_lo: (planes, norms)."""
    dh, dl = hi[0], lo[0]
    q = _c(q, np.float64).reshape(-1, dh + dl)
    return (_inst_estimate(hi, q[:, :dh], rec_hi[0], rec_hi[1], scale) +
            _inst_estimate(lo, q[:, dh:], rec_lo[0], rec_lo[1], scale))


def _inst_dequantize(inst, planes, norms):
    d, b, pi32, s32, cen32 = inst
    if s32 is None:
        return dequantize_mse(d, b, pi32, cen32, planes, norms)
    return dequantize(d, b, pi32, s32, cen32, planes, norms)


def split_dequantize(hi, lo, rec_hi, rec_lo):
    """[n, d_hi + d_lo]: the hi instance's reconstruction of the first d_hi
    channels followed by the lo instance's of the rest."""
    return np.hstack([_inst_dequantize(hi, *rec_hi), _inst_dequantize(lo, *rec_lo)])
