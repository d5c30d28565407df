"""C-ABI library: loads, exports every declared symbol, host set-up matches the
oracle's independent implementation, and argument validation fails before any
device work (CPU only)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def tq():
    import kv_cache_vector_pi_amd as tq
    return tq


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "tq.h")).read()
    return sorted(set(re.findall(r"TQ_API\s+[\w\s\*]+?\b(tq_\w+)\s*\(", src)))


def test_header_and_binding_agree(tq):
    assert declared_symbols() == sorted(tq.EXPORTS)


def test_library_exports_every_symbol(tq):
    out = subprocess.run(["nm", "-D", "--defined-only", tq.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in declared_symbols():
        assert name in exported, name
        assert hasattr(tq.lib(), name)


def test_ceiling_library_exports_its_header(tq):
    """libtq_ceiling.so (measurement kernels) loads and exports every function
    include/tq_ceiling.h declares; its host checks reject bad sizes before any
    launch (hipErrorInvalidValue = 1)."""
    src = open(os.path.join(ROOT, "include", "tq_ceiling.h")).read()
    names = sorted(set(re.findall(r"^int\s+(tq_ceiling_\w+)\s*\(", src, re.M)))
    assert names == ["tq_ceiling_copy", "tq_ceiling_logit_mix", "tq_ceiling_logit_mix_blocks",
                     "tq_ceiling_mfma", "tq_ceiling_overlap"]
    path = os.path.join(os.path.dirname(tq.LIB_PATH), "libtq_ceiling.so")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(names) <= exported
    lib = ctypes.CDLL(path)
    lib.tq_ceiling_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_void_p]
    lib.tq_ceiling_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p]
    lib.tq_ceiling_logit_mix.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    assert lib.tq_ceiling_copy(None, None, 17, None) == 1          # not a multiple of 16
    assert lib.tq_ceiling_copy(None, None, 0, None) == 0           # empty: no-op
    assert lib.tq_ceiling_mfma(2, 1, 1, None, None) == 1           # unknown kind
    lib.tq_ceiling_overlap.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_void_p]
    assert lib.tq_ceiling_overlap(3, 0, 1, 1, None, None) == 1     # unknown mode
    assert lib.tq_ceiling_overlap(2, 0, 0, 1, None, None) == 0     # no blocks: no-op
    lib.tq_ceiling_logit_mix_blocks.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                                ctypes.c_int, ctypes.c_void_p]
    assert lib.tq_ceiling_logit_mix_blocks(None, None, 8, None, 8, 0, None) == 1   # per_block < 1
    assert lib.tq_ceiling_logit_mix_blocks(None, None, 8, None, 4, 128, None) == 1  # out_stride < n
    assert lib.tq_ceiling_logit_mix_blocks(None, None, 8, None, 8, 128, None) == 1  # NULL with work
    assert lib.tq_ceiling_logit_mix_blocks(None, None, 0, None, 0, 128, None) == 0  # empty: no-op
    assert lib.tq_ceiling_logit_mix(None, None, 8, None, 4, None) == 1   # out_stride < n
    assert lib.tq_ceiling_logit_mix(None, None, 8, None, 8, None) == 1   # NULL with work


def test_status_strings(tq):
    assert tq.tq_status_string(0) == "TQ_OK"
    assert tq.tq_status_string(tq.TQ_ERR_NOT_CONVERGED) == "TQ_ERR_NOT_CONVERGED"
    assert tq.tq_status_string(99) == "TQ_ERR_UNKNOWN"
    assert tq.tq_words_per_plane(128) == 4 and tq.tq_words_per_plane(200) == 7
    assert tq.tq_record_words(200, 3) == 21 and tq.tq_words_per_plane(0) == 0


@pytest.mark.parametrize("d", [3, 16, 128, 200])
def test_rotation_matches_oracle(tq, orc, d):
    pi, s = tq.tq_make_rotation(d, 7)
    _, _, opi, os_ = orc.make_rotation(d, 7)
    assert np.array_equal(s, os_)              # same generator spec, bit for bit
    ulp = np.abs(pi.view(np.int32).astype(np.int64) - opi.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1                      # Gram-Schmidt vs Householder, then fp32
    assert (ulp > 0).mean() < 1e-3
    assert np.abs(pi.astype(np.float64).T @ pi - np.eye(d)).max() < 1e-6


def test_rotation_large_d_orthogonal(tq):
    pi, s = tq.tq_make_rotation(512, 3)
    assert np.abs(pi.astype(np.float64).T @ pi - np.eye(512)).max() < 2e-6


@pytest.mark.parametrize("d", [3, 128, 200, 1536])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_lloyd_matches_oracle(tq, orc, d, bits):
    c, dist, it = tq.tq_lloyd_max(d, bits)
    oc, odist, oit, ok = orc.lloyd_max(d, bits)
    assert ok
    assert np.array_equal(c, -c[::-1])
    ulp = np.abs(c.view(np.int32).astype(np.int64) - oc.astype(np.float32).view(np.int32))
    assert ulp.max() <= 1
    assert np.allclose(c.astype(np.float64), oc, rtol=1e-7, atol=0)
    assert dist == pytest.approx(odist, rel=1e-9, abs=1e-12)


def test_lloyd_errors(tq):
    with pytest.raises(tq.TqError) as e:
        tq.tq_lloyd_max(128, 3, max_iter=2)
    assert e.value.status == tq.TQ_ERR_NOT_CONVERGED
    for args in [(2, 2), (128, 0), (128, 5), (4096, 2)]:
        with pytest.raises(tq.TqError) as e:
            tq.tq_lloyd_max(*args)
        assert e.value.status == tq.TQ_ERR_INVALID_ARG
    L = tq.lib()
    c = np.empty(8, np.float32)
    assert L.tq_lloyd_max(128, 3, 100, 0.0, c.ctypes.data, None, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_lloyd_max(128, 3, 100, 1e-12, None, None, None) == tq.TQ_ERR_INVALID_ARG
    assert "tq_lloyd_max" in tq.tq_last_error()


def test_rotation_errors(tq):
    L = tq.lib()
    assert L.tq_make_rotation(2, 0, None, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_make_rotation(5000, 0, None, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_make_rotation(16, 0, None, None) == tq.TQ_OK   # nothing requested


def test_ctx_create_validation(tq, orc):
    L = tq.lib()
    h = ctypes.c_void_p()
    pi, s = tq.tq_make_rotation(128, 0)
    c, _, _ = tq.tq_lloyd_max(128, 2)
    P = lambda a: a.ctypes.data
    assert L.tq_ctx_create(128, 3, P(pi), P(s), P(c), None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_ctx_create(100, 3, P(pi), P(s), P(c), ctypes.byref(h)) == tq.TQ_ERR_UNSUPPORTED
    assert L.tq_ctx_create(128, 5, P(pi), P(s), P(c), ctypes.byref(h)) == tq.TQ_ERR_UNSUPPORTED
    assert L.tq_ctx_create(4096, 3, P(pi), P(s), P(c), ctypes.byref(h)) == tq.TQ_ERR_UNSUPPORTED
    assert L.tq_ctx_create(128, 3, None, P(s), P(c), ctypes.byref(h)) == tq.TQ_ERR_INVALID_ARG
    bad = c.copy(); bad[0] *= 1.001                       # not symmetric
    assert L.tq_ctx_create(128, 3, P(pi), P(s), P(bad), ctypes.byref(h)) == tq.TQ_ERR_INVALID_ARG
    bad = c[::-1].copy()                                  # descending
    assert L.tq_ctx_create(128, 3, P(pi), P(s), P(bad), ctypes.byref(h)) == tq.TQ_ERR_INVALID_ARG
    badpi = pi.copy(); badpi[3, 4] = np.nan
    assert L.tq_ctx_create(128, 3, P(badpi), P(s), P(c), ctypes.byref(h)) == tq.TQ_ERR_INVALID_ARG
    assert h.value is None
    assert L.tq_ctx_destroy(None) == tq.TQ_OK


def test_ctx_create_mse_validation(tq):
    """MSE-only contexts: b in 1..3 with 2^b centroids; checked before any
    device call."""
    L = tq.lib()
    h = ctypes.c_void_p()
    pi, _ = tq.tq_make_rotation(128, 0)
    c, _, _ = tq.tq_lloyd_max(128, 2)
    P = lambda a: a.ctypes.data
    assert L.tq_ctx_create_mse(128, 2, P(pi), P(c), None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_ctx_create_mse(128, 0, P(pi), P(c), ctypes.byref(h)) == tq.TQ_ERR_UNSUPPORTED
    assert L.tq_ctx_create_mse(128, 4, P(pi), P(c), ctypes.byref(h)) == tq.TQ_ERR_UNSUPPORTED
    assert L.tq_ctx_create_mse(100, 2, P(pi), P(c), ctypes.byref(h)) == tq.TQ_ERR_UNSUPPORTED
    assert L.tq_ctx_create_mse(128, 2, None, P(c), ctypes.byref(h)) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_ctx_create_mse(128, 2, P(pi), None, ctypes.byref(h)) == tq.TQ_ERR_INVALID_ARG
    bad = c.copy(); bad[0] *= 1.001                       # not symmetric
    assert L.tq_ctx_create_mse(128, 2, P(pi), P(bad), ctypes.byref(h)) == tq.TQ_ERR_INVALID_ARG
    assert h.value is None
    assert L.tq_ctx_is_mse(None) == 0


def test_hot_path_rejects_null_context(tq):
    L = tq.lib()
    assert L.tq_quantize_kv(None, None, 0, 1, 1, 128, 0, None, None, 0, 0, None) == \
        tq.TQ_ERR_INVALID_ARG
    assert L.tq_dequantize(None, None, None, 1, None, 128, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_attn_logits(None, None, 1, 32, 4096, None, None, 8, 0, None, None, 1, 1.0,
                            None, 0, None, 0, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_search_topk(None, None, 1, None, None, 1, 10, None, None, None, 0, None) == \
        tq.TQ_ERR_INVALID_ARG
    assert L.tq_attn_output(None, None, 0, 1, 32, None, None, 8, 0, None, None, 1, None, 0, None,
                            0, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_attn_output_workspace_bytes(None, 1, 32, 8, 100) == 0
    assert L.tq_attn_decode(None, None, 1, 32, 4096, None, None, None, None, 8, 0, None, None, 1,
                            1.0, None, 0, None, 0, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_attn_decode_workspace_bytes(None, 1, 32, 8, 100) == 0
    assert L.tq_decode_step_prepare(None, None, None, 1, 1, 256, 128, 128, None, None, None, None,
                                    4, 0, None, None, 32, 32, 4096, 8, None, 0, None) == \
        tq.TQ_ERR_INVALID_ARG
    assert L.tq_quantize_kv_slots(None, None, 0, 1, 1, 128, 0, None, None, None, 1, None) == \
        tq.TQ_ERR_INVALID_ARG
    assert L.tq_split_quantize_kv(None, None, None, 0, 1, 1, 128, 0, None, None, None, None, 1, 0,
                                  None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_split_dequantize(None, None, None, None, None, None, 1, None, 128, None) == \
        tq.TQ_ERR_INVALID_ARG
    assert L.tq_split_attn_logits(None, None, None, 1, 32, 4096, None, None, None, None, 8, 0,
                                  None, None, 1, 1.0, None, 0, None, 0, None) == \
        tq.TQ_ERR_INVALID_ARG
    assert L.tq_split_attn_output(None, None, None, 0, 1, 32, None, None, None, None, 8, 0, None,
                                  None, 1, None, 0, None, 0, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_split_attn_prepare(None, None, None, 1, 32, 4096, 8, None, 0, None) == \
        tq.TQ_ERR_INVALID_ARG
    assert L.tq_split_attn_logits_prepared(None, None, None, 0, 1, 32, None, None, None, None, 8,
                                           0, None, None, 1, 1.0, None, 0, None) == \
        tq.TQ_ERR_INVALID_ARG
    assert L.tq_quantize_kv_ws(None, None, 0, 1, 1, 128, 0, None, None, 1, 0, None, 0, None) == \
        tq.TQ_ERR_INVALID_ARG
    assert L.tq_quantize_workspace_bytes(None, 100) == 0
    assert L.tq_split_attn_logits_workspace_bytes(None, None, 1, 32, 8) == 0
    assert L.tq_split_attn_output_workspace_bytes(None, None, 1, 32, 8, 100) == 0
    assert L.tq_attn_logits_workspace_bytes(None, 1, 32, 8) == 0
    assert L.tq_search_workspace_bytes(None, 1, 1, 10) == 0
    assert L.tq_ctx_dim(None) == 0 and L.tq_ctx_bits(None) == 0
