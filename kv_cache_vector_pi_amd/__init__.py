"""Python binding of libtq, the MI355X TurboQuant hot path.

Thin ctypes marshalling over the C ABI in ``include/tq.h``: every function
here has the name of the C entry point it calls and does no arithmetic of its
own.  PyTorch provides device memory and the current HIP stream; all work on
the hot path runs in the HIP kernels of ``libtq.so``.  Importing this package
fails loudly when the built library is missing -- there is no fallback.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

TQ_OK = 0
TQ_ERR_INVALID_ARG = -1
TQ_ERR_UNSUPPORTED = -2
TQ_ERR_NOT_CONVERGED = -3
TQ_ERR_HIP = -4
TQ_ERR_ALLOC = -5
TQ_F32 = 0
TQ_BF16 = 1

# every symbol include/tq.h declares
EXPORTS = [
    "tq_status_string", "tq_last_error", "tq_words_per_plane", "tq_record_words",
    "tq_make_rotation", "tq_lloyd_max", "tq_ctx_create", "tq_ctx_destroy", "tq_ctx_dim",
    "tq_ctx_bits", "tq_quantize_kv", "tq_dequantize", "tq_attn_logits_workspace_bytes",
    "tq_attn_logits", "tq_attn_logits_noalloc", "tq_attn_prepare", "tq_attn_logits_prepared",
    "tq_search_workspace_bytes", "tq_search_topk", "tq_attn_output_workspace_bytes",
    "tq_attn_output", "tq_attn_decode_workspace_bytes", "tq_attn_decode",
    "tq_ctx_create_mse", "tq_ctx_is_mse", "tq_decode_step_prepare", "tq_quantize_kv_slots",
    "tq_split_quantize_kv", "tq_split_dequantize", "tq_split_attn_logits_workspace_bytes",
    "tq_split_attn_logits", "tq_split_attn_output_workspace_bytes", "tq_split_attn_output",
    "tq_split_attn_prepare", "tq_split_attn_logits_prepared", "tq_quantize_workspace_bytes",
    "tq_quantize_kv_ws",
]


class TqError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(f"libtq.so not built at {LIB_PATH}; run "
                      "`python kv_cache_vector_pi_amd/build.py` (no fallback exists)")

_lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_i32, _i64, _u64, _f32, _f64, _sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                     ctypes.c_float, ctypes.c_double, ctypes.c_size_t)


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_sig("tq_status_string", ctypes.c_char_p, [_i32])
_sig("tq_last_error", ctypes.c_char_p, [])
_sig("tq_words_per_plane", _i32, [_i32])
_sig("tq_record_words", _i32, [_i32, _i32])
_sig("tq_make_rotation", _i32, [_i32, _u64, _P, _P])
_sig("tq_lloyd_max", _i32, [_i32, _i32, _i32, _f64, _P, _P, _P])
_sig("tq_ctx_create", _i32, [_i32, _i32, _P, _P, _P, ctypes.POINTER(_P)])
_sig("tq_ctx_destroy", _i32, [_P])
_sig("tq_ctx_create_mse", _i32, [_i32, _i32, _P, _P, ctypes.POINTER(_P)])
_sig("tq_ctx_is_mse", _i32, [_P])
_sig("tq_decode_step_prepare", _i32, [_P, _P, _P, _i32, _i64, _i32, _i64, _i64, _P, _P, _P, _P,
                                      _i64, _i64, _P, _P, _i32, _i32, _i64, _i32, _P, _sz, _P])
_sig("tq_ctx_dim", _i32, [_P])
_sig("tq_ctx_bits", _i32, [_P])
_sig("tq_quantize_kv", _i32, [_P, _P, _i32, _i64, _i32, _i64, _i64, _P, _P, _i64, _i64, _P])
_sig("tq_quantize_workspace_bytes", _sz, [_P, _i64])
_sig("tq_quantize_kv_ws", _i32, [_P, _P, _i32, _i64, _i32, _i64, _i64, _P, _P, _i64, _i64, _P,
                                 _sz, _P])
_sig("tq_quantize_kv_slots", _i32, [_P, _P, _i32, _i64, _i32, _i64, _i64, _P, _P, _P, _i64, _P])
_sig("tq_dequantize", _i32, [_P, _P, _P, _i64, _P, _i64, _P])
_sig("tq_split_quantize_kv", _i32, [_P, _P, _P, _i32, _i64, _i32, _i64, _i64, _P, _P, _P, _P,
                                    _i64, _i64, _P])
_sig("tq_split_dequantize", _i32, [_P, _P, _P, _P, _P, _P, _i64, _P, _i64, _P])
_sig("tq_split_attn_logits_workspace_bytes", _sz, [_P, _P, _i32, _i32, _i32])
_sig("tq_split_attn_logits", _i32, [_P, _P, _P, _i32, _i32, _i64, _P, _P, _P, _P, _i32, _i64, _P,
                                    _P, _i32, _f32, _P, _i64, _P, _sz, _P])
_sig("tq_split_attn_prepare", _i32, [_P, _P, _P, _i32, _i32, _i64, _i32, _P, _sz, _P])
_sig("tq_split_attn_logits_prepared", _i32, [_P, _P, _P, _sz, _i32, _i32, _P, _P, _P, _P, _i32,
                                             _i64, _P, _P, _i32, _f32, _P, _i64, _P])
_sig("tq_split_attn_output_workspace_bytes", _sz, [_P, _P, _i32, _i32, _i32, _i32])
_sig("tq_split_attn_output", _i32, [_P, _P, _P, _i64, _i32, _i32, _P, _P, _P, _P, _i32, _i64,
                                    _P, _P, _i32, _P, _i64, _P, _sz, _P])
_sig("tq_attn_logits_workspace_bytes", _sz, [_P, _i32, _i32, _i32])
_sig("tq_attn_logits", _i32, [_P, _P, _i32, _i32, _i64, _P, _P, _i32, _i64, _P, _P, _i32, _f32,
                              _P, _i64, _P, _sz, _P])
_sig("tq_attn_prepare", _i32, [_P, _P, _i32, _i32, _i64, _i32, _P, _sz, _P])
_sig("tq_attn_logits_noalloc", _i32, [_P, _P, _i32, _i32, _i64, _P, _P, _i32, _i64, _P, _P,
                                     _i32, _f32, _P, _i64, _P])
_sig("tq_attn_logits_prepared", _i32, [_P, _P, _sz, _i32, _i32, _P, _P, _i32, _i64, _P, _P, _i32,
                                       _f32, _P, _i64, _P])
_sig("tq_attn_output_workspace_bytes", _sz, [_P, _i32, _i32, _i32, _i32])
_sig("tq_attn_output", _i32, [_P, _P, _i64, _i32, _i32, _P, _P, _i32, _i64, _P, _P, _i32, _P, _i64,
                              _P, _sz, _P])
_sig("tq_attn_decode_workspace_bytes", _sz, [_P, _i32, _i32, _i32, _i32])
_sig("tq_attn_decode", _i32, [_P, _P, _i32, _i32, _i64, _P, _P, _P, _P, _i32, _i64, _P, _P, _i32,
                              _f32, _P, _i64, _P, _sz, _P])
_sig("tq_search_workspace_bytes", _sz, [_P, _i64, _i64, _i32])
_sig("tq_search_topk", _i32, [_P, _P, _i64, _P, _P, _i64, _i32, _P, _P, _P, _sz, _P])


def lib():
    return _lib


def _check(status, what):
    if status != TQ_OK:
        msg = _lib.tq_last_error().decode() or what
        raise TqError(status, msg)


def _ptr(t):
    """Device or host address of a torch tensor or numpy array (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream=None):
    """Raw hipStream_t for a torch.cuda.Stream, a raw handle, or None (the
    current stream)."""
    if stream is not None:
        return getattr(stream, "cuda_stream", stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


# ---- small helpers --------------------------------------------------------
def tq_status_string(status):
    return _lib.tq_status_string(status).decode()


def tq_last_error():
    return _lib.tq_last_error().decode()


def tq_words_per_plane(d):
    return _lib.tq_words_per_plane(d)


def tq_record_words(d, b):
    return _lib.tq_record_words(d, b)


# ---- offline set-up (host) ------------------------------------------------
def tq_make_rotation(d, seed):
    """(pi, s): float32 [d, d] host arrays (see tq.h)."""
    pi = np.empty((d, d), np.float32)
    s = np.empty((d, d), np.float32)
    _check(_lib.tq_make_rotation(d, seed, pi.ctypes.data, s.ctypes.data), "tq_make_rotation")
    return pi, s


def tq_lloyd_max(d, lm_bits, max_iter=100000, tol=1e-13):
    """(centroids float32 [2**lm_bits], distortion, iterations)."""
    c = np.empty(1 << lm_bits, np.float32)
    dist = ctypes.c_double(0.0)
    it = ctypes.c_int32(0)
    st = _lib.tq_lloyd_max(d, lm_bits, max_iter, tol, c.ctypes.data, ctypes.addressof(dist),
                           ctypes.addressof(it))
    _check(st, "tq_lloyd_max")
    return c, dist.value, it.value


class TqContext:
    """Owns a tq_ctx (device tables on the current HIP device).  s=None makes
    an MSE-only context (tq_ctx_create_mse: b code bits, no QJL stage)."""

    def __init__(self, d, b, pi, s, centroids):
        pi = np.ascontiguousarray(pi, np.float32)
        c = np.ascontiguousarray(centroids, np.float32)
        h = _P()
        if s is None:
            _check(_lib.tq_ctx_create_mse(d, b, pi.ctypes.data, c.ctypes.data, ctypes.byref(h)),
                   "tq_ctx_create_mse")
        else:
            s = np.ascontiguousarray(s, np.float32)
            _check(_lib.tq_ctx_create(d, b, pi.ctypes.data, s.ctypes.data, c.ctypes.data,
                                      ctypes.byref(h)), "tq_ctx_create")
        self.handle = h.value
        self.d, self.b = d, b
        self.mse = s is None

    @property
    def W(self):
        return tq_words_per_plane(self.d)

    def close(self):
        if self.handle:
            _check(_lib.tq_ctx_destroy(self.handle), "tq_ctx_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tq_ctx_create(d, b, pi, s, centroids):
    return TqContext(d, b, pi, s, centroids)


def tq_ctx_create_mse(d, b, pi, centroids):
    return TqContext(d, b, pi, None, centroids)


def tq_ctx_is_mse(ctx):
    return int(_lib.tq_ctx_is_mse(ctx.handle if ctx is not None else None))


def tq_ctx_destroy(ctx):
    ctx.close()


# ---- device buffers -------------------------------------------------------
def alloc_records(n, d, b, device="cuda"):
    """(planes uint32-as-int32 [n, W*b], norms int16 [n, 2]) device tensors."""
    import torch
    planes = torch.zeros((n, tq_record_words(d, b)), dtype=torch.int32, device=device)
    norms = torch.zeros((n, 2), dtype=torch.int16, device=device)
    return planes, norms


# ---- hot path -------------------------------------------------------------
def _quant_input(x, n_tokens, n_heads, x_stride_token, x_stride_head):
    """(dtype code, n_tokens, n_heads, token stride, head stride) of a
    [n_heads, n_tokens, d] or [n, d] float32/bfloat16 tensor; explicit
    arguments win."""
    import torch
    if x.dtype == torch.bfloat16:
        dt = TQ_BF16
    elif x.dtype == torch.float32:
        dt = TQ_F32
    else:
        raise TypeError(f"unsupported dtype {x.dtype}")
    x3 = x.unsqueeze(0) if x.dim() == 2 else x
    return (dt, x3.shape[1] if n_tokens is None else n_tokens,
            x3.shape[0] if n_heads is None else n_heads,
            x3.stride(1) if x_stride_token is None else x_stride_token,
            x3.stride(0) if x_stride_head is None else x_stride_head)


def tq_quantize_kv(ctx, x, planes, norms, n_tokens=None, n_heads=None, x_stride_token=None,
                   x_stride_head=None, dst_stride_head=None, dst_token0=0, stream=None):
    """Quantize x ([n_heads, n_tokens, d] or [n, d] torch tensor, float32 or
    bfloat16) into planes/norms (see tq.h for the record indexing)."""
    dt, n_tokens, n_heads, x_stride_token, x_stride_head = _quant_input(
        x, n_tokens, n_heads, x_stride_token, x_stride_head)
    if dst_stride_head is None:
        dst_stride_head = n_tokens
    st = _lib.tq_quantize_kv(ctx.handle, _ptr(x), dt, n_tokens, n_heads, x_stride_token,
                             x_stride_head, _ptr(planes), _ptr(norms), dst_stride_head,
                             dst_token0, _stream(stream))
    _check(st, "tq_quantize_kv")


def tq_quantize_workspace_bytes(ctx, n_rows):
    return _lib.tq_quantize_workspace_bytes(ctx.handle, n_rows)


def tq_quantize_kv_ws(ctx, x, planes, norms, workspace, n_tokens=None, n_heads=None,
                      x_stride_token=None, x_stride_head=None, dst_stride_head=None,
                      dst_token0=0, stream=None):
    """tq_quantize_kv with a workspace (blocked products at large d; see tq.h)."""
    dt, n_tokens, n_heads, x_stride_token, x_stride_head = _quant_input(
        x, n_tokens, n_heads, x_stride_token, x_stride_head)
    if dst_stride_head is None:
        dst_stride_head = n_tokens
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.tq_quantize_kv_ws(ctx.handle, _ptr(x), dt, n_tokens, n_heads, x_stride_token,
                                x_stride_head, _ptr(planes), _ptr(norms), dst_stride_head,
                                dst_token0, _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "tq_quantize_kv_ws")


def tq_quantize_kv_slots(ctx, x, slots, planes, norms, dst_stride_head, n_tokens=None,
                         n_heads=None, x_stride_token=None, x_stride_head=None, stream=None):
    """Quantize x ([n_heads, n_tokens, d] or [n, d]) into planes/norms with
    token t's record of head h at h * dst_stride_head + slots[t] (slots: int64
    device tensor [n_tokens]; slots outside [0, dst_stride_head) are skipped)."""
    dt, n_tokens, n_heads, x_stride_token, x_stride_head = _quant_input(
        x, n_tokens, n_heads, x_stride_token, x_stride_head)
    st = _lib.tq_quantize_kv_slots(ctx.handle, _ptr(x), dt, n_tokens, n_heads, x_stride_token,
                                   x_stride_head, _ptr(slots), _ptr(planes), _ptr(norms),
                                   dst_stride_head, _stream(stream))
    _check(st, "tq_quantize_kv_slots")


def tq_dequantize(ctx, planes, norms, n, out, out_ld=None, stream=None):
    if out_ld is None:
        out_ld = out.stride(0)
    _check(_lib.tq_dequantize(ctx.handle, _ptr(planes), _ptr(norms), n, _ptr(out), out_ld,
                              _stream(stream)), "tq_dequantize")


def tq_attn_logits_workspace_bytes(ctx, batch, n_q_heads, n_kv_heads):
    return _lib.tq_attn_logits_workspace_bytes(ctx.handle, batch, n_q_heads, n_kv_heads)


def tq_attn_logits(ctx, q, batch, n_q_heads, q_stride_batch, planes, norms, n_kv_heads,
                   keys_stride_head, seq_start, seq_len, max_seq_len, scale, logits,
                   logits_stride_head, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.tq_attn_logits(ctx.handle, _ptr(q), batch, n_q_heads, q_stride_batch,
                             _ptr(planes), _ptr(norms), n_kv_heads, keys_stride_head,
                             _ptr(seq_start), _ptr(seq_len), max_seq_len, float(scale),
                             _ptr(logits), logits_stride_head, _ptr(workspace), ws_bytes,
                             _stream(stream))
    _check(st, "tq_attn_logits")


def tq_attn_logits_noalloc(ctx, q, batch, n_q_heads, q_stride_batch, planes, norms, n_kv_heads,
                           keys_stride_head, seq_start, seq_len, max_seq_len, scale, logits,
                           logits_stride_head, stream=None):
    st = _lib.tq_attn_logits_noalloc(ctx.handle, _ptr(q), batch, n_q_heads, q_stride_batch,
                                     _ptr(planes), _ptr(norms), n_kv_heads, keys_stride_head,
                                     _ptr(seq_start), _ptr(seq_len), max_seq_len, float(scale),
                                     _ptr(logits), logits_stride_head, _stream(stream))
    _check(st, "tq_attn_logits_noalloc")


def tq_attn_prepare(ctx, q, batch, n_q_heads, q_stride_batch, n_kv_heads, workspace,
                    stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.tq_attn_prepare(ctx.handle, _ptr(q), batch, n_q_heads, q_stride_batch, n_kv_heads,
                              _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "tq_attn_prepare")


def tq_decode_step_prepare(ctx, k_new, v_new, k_planes, k_norms, v_planes, v_norms, q, batch,
                           n_q_heads, q_stride_batch, n_kv_heads, workspace, dst_stride_head,
                           dst_token0=0, stream=None, dst_slots=None):
    """Quantize k_new and v_new ([n_heads, n_tokens, d], same dtype, sizes and
    strides) into the two caches and prepare q into workspace, in one launch
    at d = 128 (see tq.h).  dst_slots: None, or an int64 device tensor
    [n_tokens] of destination tokens (as tq_quantize_kv_slots)."""
    import torch
    if k_new.dtype != v_new.dtype or k_new.shape != v_new.shape or \
            k_new.stride() != v_new.stride():
        raise ValueError("k_new and v_new must share dtype, shape and strides")
    if k_new.dtype == torch.bfloat16:
        dt = TQ_BF16
    elif k_new.dtype == torch.float32:
        dt = TQ_F32
    else:
        raise TypeError(f"unsupported dtype {k_new.dtype}")
    n_heads, n_tokens = k_new.shape[0], k_new.shape[1]
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.tq_decode_step_prepare(ctx.handle, _ptr(k_new), _ptr(v_new), dt, n_tokens, n_heads,
                                     k_new.stride(1), k_new.stride(0), _ptr(k_planes),
                                     _ptr(k_norms), _ptr(v_planes), _ptr(v_norms),
                                     dst_stride_head, dst_token0, _ptr(dst_slots), _ptr(q),
                                     batch, n_q_heads,
                                     q_stride_batch, n_kv_heads, _ptr(workspace), ws_bytes,
                                     _stream(stream))
    _check(st, "tq_decode_step_prepare")


def tq_attn_logits_prepared(ctx, workspace, batch, n_q_heads, planes, norms, n_kv_heads,
                            keys_stride_head, seq_start, seq_len, max_seq_len, scale, logits,
                            logits_stride_head, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.tq_attn_logits_prepared(ctx.handle, _ptr(workspace), ws_bytes, batch, n_q_heads,
                                      _ptr(planes), _ptr(norms), n_kv_heads, keys_stride_head,
                                      _ptr(seq_start), _ptr(seq_len), max_seq_len, float(scale),
                                      _ptr(logits), logits_stride_head, _stream(stream))
    _check(st, "tq_attn_logits_prepared")


def tq_attn_output_workspace_bytes(ctx, batch, n_q_heads, n_kv_heads, max_seq_len):
    return _lib.tq_attn_output_workspace_bytes(ctx.handle, batch, n_q_heads, n_kv_heads,
                                               max_seq_len)


def tq_attn_output(ctx, p, p_stride_head, batch, n_q_heads, planes, norms, n_kv_heads,
                   values_stride_head, seq_start, seq_len, max_seq_len, out, out_stride_batch,
                   workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.tq_attn_output(ctx.handle, _ptr(p), p_stride_head, batch, n_q_heads, _ptr(planes),
                             _ptr(norms), n_kv_heads, values_stride_head, _ptr(seq_start),
                             _ptr(seq_len), max_seq_len, _ptr(out), out_stride_batch,
                             _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "tq_attn_output")


def tq_attn_decode_workspace_bytes(ctx, batch, n_q_heads, n_kv_heads, max_seq_len):
    return _lib.tq_attn_decode_workspace_bytes(ctx.handle, batch, n_q_heads, n_kv_heads,
                                               max_seq_len)


def tq_attn_decode(ctx, q, batch, n_q_heads, q_stride_batch, k_planes, k_norms, v_planes,
                   v_norms, n_kv_heads, kv_stride_head, seq_start, seq_len, max_seq_len, scale,
                   out, out_stride_batch, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.tq_attn_decode(ctx.handle, _ptr(q), batch, n_q_heads, q_stride_batch,
                             _ptr(k_planes), _ptr(k_norms), _ptr(v_planes), _ptr(v_norms),
                             n_kv_heads, kv_stride_head, _ptr(seq_start), _ptr(seq_len),
                             max_seq_len, float(scale), _ptr(out), out_stride_batch,
                             _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "tq_attn_decode")


def tq_search_workspace_bytes(ctx, n_queries, n_db, k):
    return _lib.tq_search_workspace_bytes(ctx.handle, n_queries, n_db, k)


def tq_search_topk(ctx, queries, n_queries, planes, norms, n_db, k, out_idx, out_score,
                   workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.tq_search_topk(ctx.handle, _ptr(queries), n_queries, _ptr(planes), _ptr(norms),
                             n_db, k, _ptr(out_idx), _ptr(out_score), _ptr(workspace), ws_bytes,
                             _stream(stream))
    _check(st, "tq_search_topk")


def workspace(nbytes, device="cuda"):
    """A 256-byte aligned uint8 device buffer of at least nbytes."""
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---- fractional bit widths: two instances over a channel split (see tq.h) ----
def tq_split_quantize_kv(hi, lo, x, hi_planes, hi_norms, lo_planes, lo_norms, n_tokens=None,
                         n_heads=None, x_stride_token=None, x_stride_head=None,
                         dst_stride_head=None, dst_token0=0, stream=None):
    """Quantize channels [0, d_hi) of x ([n_heads, n_tokens, d_hi + d_lo] or
    [n, d_hi + d_lo]) under `hi` and the rest under `lo`."""
    dt, n_tokens, n_heads, x_stride_token, x_stride_head = _quant_input(
        x, n_tokens, n_heads, x_stride_token, x_stride_head)
    if dst_stride_head is None:
        dst_stride_head = n_tokens
    st = _lib.tq_split_quantize_kv(hi.handle, lo.handle, _ptr(x), dt, n_tokens, n_heads,
                                   x_stride_token, x_stride_head, _ptr(hi_planes),
                                   _ptr(hi_norms), _ptr(lo_planes), _ptr(lo_norms),
                                   dst_stride_head, dst_token0, _stream(stream))
    _check(st, "tq_split_quantize_kv")


def tq_split_dequantize(hi, lo, hi_planes, hi_norms, lo_planes, lo_norms, n, out, out_ld=None,
                        stream=None):
    if out_ld is None:
        out_ld = out.stride(0)
    _check(_lib.tq_split_dequantize(hi.handle, lo.handle, _ptr(hi_planes), _ptr(hi_norms),
                                    _ptr(lo_planes), _ptr(lo_norms), n, _ptr(out), out_ld,
                                    _stream(stream)), "tq_split_dequantize")


def tq_split_attn_logits_workspace_bytes(hi, lo, batch, n_q_heads, n_kv_heads):
    return _lib.tq_split_attn_logits_workspace_bytes(hi.handle, lo.handle, batch, n_q_heads,
                                                     n_kv_heads)


def tq_split_attn_logits(hi, lo, q, batch, n_q_heads, q_stride_batch, hi_planes, hi_norms,
                         lo_planes, lo_norms, n_kv_heads, keys_stride_head, seq_start, seq_len,
                         max_seq_len, scale, logits, logits_stride_head, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.tq_split_attn_logits(hi.handle, lo.handle, _ptr(q), batch, n_q_heads,
                                   q_stride_batch, _ptr(hi_planes), _ptr(hi_norms),
                                   _ptr(lo_planes), _ptr(lo_norms), n_kv_heads, keys_stride_head,
                                   _ptr(seq_start), _ptr(seq_len), max_seq_len, float(scale),
                                   _ptr(logits), logits_stride_head, _ptr(workspace), ws_bytes,
                                   _stream(stream))
    _check(st, "tq_split_attn_logits")


def tq_split_attn_prepare(hi, lo, q, batch, n_q_heads, q_stride_batch, n_kv_heads, workspace,
                          stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.tq_split_attn_prepare(hi.handle, lo.handle, _ptr(q), batch, n_q_heads,
                                      q_stride_batch, n_kv_heads, _ptr(workspace), ws_bytes,
                                      _stream(stream)), "tq_split_attn_prepare")


def tq_split_attn_logits_prepared(hi, lo, workspace, batch, n_q_heads, hi_planes, hi_norms,
                                  lo_planes, lo_norms, n_kv_heads, keys_stride_head, seq_start,
                                  seq_len, max_seq_len, scale, logits, logits_stride_head,
                                  stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.tq_split_attn_logits_prepared(hi.handle, lo.handle, _ptr(workspace), ws_bytes,
                                            batch, n_q_heads, _ptr(hi_planes), _ptr(hi_norms),
                                            _ptr(lo_planes), _ptr(lo_norms), n_kv_heads,
                                            keys_stride_head, _ptr(seq_start), _ptr(seq_len),
                                            max_seq_len, float(scale), _ptr(logits),
                                            logits_stride_head, _stream(stream))
    _check(st, "tq_split_attn_logits_prepared")


def tq_split_attn_output_workspace_bytes(hi, lo, batch, n_q_heads, n_kv_heads, max_seq_len):
    return _lib.tq_split_attn_output_workspace_bytes(hi.handle, lo.handle, batch, n_q_heads,
                                                     n_kv_heads, max_seq_len)


def tq_split_attn_output(hi, lo, p, p_stride_head, batch, n_q_heads, hi_planes, hi_norms,
                         lo_planes, lo_norms, n_kv_heads, values_stride_head, seq_start, seq_len,
                         max_seq_len, out, out_stride_batch, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.tq_split_attn_output(hi.handle, lo.handle, _ptr(p), p_stride_head, batch,
                                   n_q_heads, _ptr(hi_planes), _ptr(hi_norms), _ptr(lo_planes),
                                   _ptr(lo_norms), n_kv_heads, values_stride_head,
                                   _ptr(seq_start), _ptr(seq_len), max_seq_len, _ptr(out),
                                   out_stride_batch, _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "tq_split_attn_output")
