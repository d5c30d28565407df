"""GPU parity: the HIP kernels against the CPU oracle, through the C ABI.

Quantize: codes bit-exact except within 1e-5 of a threshold (oracle margin);
signs bit-exact except |z| < 1e-5 (vectors whose codes all match); fp16
norms within one ulp.  Logits, dequantized vectors and search scores are fed
oracle-produced (or arbitrary) records and must agree within 1e-3 of
max(|ref|, rms of the row).  All inputs are seeded.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_vector_pi_amd as tq  # noqa: E402
import workloads  # noqa: E402
from helpers import (TOL, check_records, check_records_mse, clear_padding, oracle_tables,  # noqa: E402
                     rel_err_rows, topk_order_ok)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


_ctx_cache = {}


def ctx_for(orc, d, b, seed=0):
    key = (d, b, seed)
    if key not in _ctx_cache:
        pi, s, c = oracle_tables(orc, d, b, seed)
        _ctx_cache[key] = (tq.TqContext(d, b, pi, s, c), pi, s, c)
    return _ctx_cache[key]


def gpu_quantize(ctx, x):
    """x: torch [n, d] on the GPU -> numpy planes uint32 [n, W*b], norms uint16 [n, 2]."""
    n, d = x.shape
    planes, norms = tq.alloc_records(n, d, ctx.b)
    tq.tq_quantize_kv(ctx, x.contiguous(), planes, norms)
    torch.cuda.synchronize()
    return planes.cpu().numpy().view(np.uint32), norms.cpu().numpy().view(np.uint16)


def check_quantize(orc, d, b, x, pi, s, c, planes, norms, rows=None):
    """Compare GPU records of x (rows `rows` of the GPU output) with the
    oracle (helpers.check_records), and check that padding bits stay zero."""
    xd = x.double().cpu().numpy() if hasattr(x, "double") else np.asarray(x, np.float64)
    if rows is not None:
        xd = xd[rows]
        planes, norms = planes[rows], norms[rows]
    stats = check_records(orc, d, b, pi, s, c, xd, planes, norms)
    if d % 32:
        pc = np.array(planes, np.uint32).copy()
        clear_padding(pc, d, b)
        assert np.array_equal(pc, np.asarray(planes).view(np.uint32))
    return stats


# ---------------------------------------------------------------- quantize
@pytest.mark.parametrize("d,b,dtype,n", [
    (128, 3, torch.float32, 1024),        # tiny workload shape
    (128, 4, torch.bfloat16, 1000),       # ragged tail (1000 = 15 tiles + 40)
    (128, 2, torch.bfloat16, 257),
    (128, 4, torch.float32, 64),
    (200, 2, torch.float32, 300),
    (200, 4, torch.float32, 130),
    (64, 3, torch.float32, 77),           # odd count: the generic kernel
    (64, 4, torch.bfloat16, 1000),        # token pairs through the d = 128 kernel
    (64, 2, torch.float32, 258),
    (1536, 2, torch.float32, 40),
    (1536, 4, torch.float32, 33),
])
def test_quantize_parity(orc, d, b, dtype, n):
    say("quantize", d, b, dtype, n)
    ctx, pi, s, c = ctx_for(orc, d, b)
    x = workloads.normal((n, d), 3, 10, DEV) * 2.0
    x[5] = 0.0                          # zero vector
    x = x.to(dtype)
    planes, norms = gpu_quantize(ctx, x)
    stats = check_quantize(orc, d, b, x, pi, s, c, planes, norms)
    say("ok", stats)


def test_quantize_bf16_outliers_strided(orc):
    """[n_kv, n_tok, d] bf16 with outlier channels, quantized head by head with
    a token offset into a larger cache."""
    d, b = 128, 4
    ctx, pi, s, c = ctx_for(orc, d, b)
    K = workloads.kv_with_outliers(3, 600, d, 1, 10, DEV)
    say("quantize strided", K.shape)
    cap = 1000
    planes, norms = tq.alloc_records(3 * cap, d, b)
    tq.tq_quantize_kv(ctx, K, planes, norms, dst_stride_head=cap, dst_token0=123)
    torch.cuda.synchronize()
    P = planes.cpu().numpy().view(np.uint32).reshape(3, cap, -1)
    N = norms.cpu().numpy().view(np.uint16).reshape(3, cap, 2)
    assert not P[:, :123].any() and not P[:, 723:].any()
    for h in range(3):
        check_quantize(orc, d, b, K[h], pi, s, c, P[h, 123:723], N[h, 123:723])


@pytest.mark.parametrize("n_heads,n_tok,b,dtype", [
    (256, 1, 4, torch.bfloat16),      # one new token per (kv head, layer)
    (37, 3, 3, torch.float32),        # tiles span up to 22 heads, ragged end
    (5, 63, 2, torch.bfloat16),
    (3, 65, 4, torch.float32),        # one tile per head plus a 1-row spill
    (2, 130, 3, torch.bfloat16),
])
def test_quantize_short_heads(orc, n_heads, n_tok, b, dtype):
    """Many short heads in one call: source rows strided by head and token,
    records scattered at h * cap + 7 + t of a larger cache."""
    d = 128
    say("quantize short heads", n_heads, n_tok, b, dtype)
    ctx, pi, s, c = ctx_for(orc, d, b)
    base = workloads.normal((n_tok, n_heads, d + 8), 13, 10, DEV) * 1.5
    base[0, n_heads // 2] = 0.0                         # a zero vector
    base = base.to(dtype)
    x = base[:, :, :d].transpose(0, 1)                  # [head][token][d], strided view
    cap = n_tok + 11
    planes, norms = tq.alloc_records(n_heads * cap, d, b)
    tq.tq_quantize_kv(ctx, x, planes, norms, n_tokens=n_tok, n_heads=n_heads,
                      x_stride_token=x.stride(1), x_stride_head=x.stride(0),
                      dst_stride_head=cap, dst_token0=7)
    torch.cuda.synchronize()
    P = planes.cpu().numpy().view(np.uint32).reshape(n_heads, cap, -1)
    N = norms.cpu().numpy().view(np.uint16).reshape(n_heads, cap, 2)
    assert not P[:, :7].any() and not P[:, 7 + n_tok:].any()
    assert not N[:, :7].any() and not N[:, 7 + n_tok:].any()
    xs = x.reshape(n_heads * n_tok, d)
    check_quantize(orc, d, b, xs, pi, s, c, P[:, 7:7 + n_tok].reshape(n_heads * n_tok, -1),
                   N[:, 7:7 + n_tok].reshape(n_heads * n_tok, 2))


@pytest.mark.parametrize("n_heads,n_tok,b,dtype,cap,t0", [
    (40, 2, 4, torch.bfloat16, 2, 0),       # one pair per head: tiles across heads
    (3, 130, 3, torch.float32, 140, 6),      # pairs inside heads, offset and strided cache
    (2, 96, 2, torch.bfloat16, 100, 2),
    (2, 131, 4, torch.bfloat16, 140, 3),     # odd count: pairs + the generic last token; odd index, even b
    (3, 7, 3, torch.float32, 10, 2),         # odd count, odd b
    (2, 9, 3, torch.bfloat16, 11, 1),        # odd b at odd indices: the generic kernel
])
def test_quantize_d64_pairs(orc, n_heads, n_tok, b, dtype, cap, t0):
    """d = 64 through the d = 128 kernel on token pairs: records against the
    oracle, each token's norms its own, records at h * cap + t0 + t, and
    neighbouring records untouched."""
    say("d64 pairs", n_heads, n_tok, b, dtype, cap, t0)
    d = 64
    ctx, pi, s, c = ctx_for(orc, d, b)
    x = (workloads.normal((n_heads, n_tok, d), 61, 10, DEV) * 3.0)
    x[0, 1] = 0.0                           # second token of a pair is zero
    x[n_heads - 1, n_tok - 2] *= 1e-3      # a small token near the end
    x = x.to(dtype)
    P, N = tq.alloc_records(n_heads * cap, d, b)
    P.fill_(0x5A5A5A5A)
    N.fill_(0x3C3C)
    tq.tq_quantize_kv(ctx, x, P, N, dst_stride_head=cap, dst_token0=t0)
    torch.cuda.synchronize()
    W = tq.tq_words_per_plane(d)
    gp = P.cpu().numpy().view(np.uint32).reshape(n_heads, cap, W * b)
    gn = N.cpu().numpy().view(np.uint16).reshape(n_heads, cap, 2)
    assert np.all(gp[:, :t0] == 0x5A5A5A5A) and np.all(gp[:, t0 + n_tok:] == 0x5A5A5A5A)
    assert np.all(gn[:, :t0] == 0x3C3C) and np.all(gn[:, t0 + n_tok:] == 0x3C3C)
    rows = gp[:, t0:t0 + n_tok].reshape(n_heads * n_tok, -1)
    nrm = gn[:, t0:t0 + n_tok].reshape(n_heads * n_tok, 2)
    check_quantize(orc, d, b, x.reshape(-1, d), pi, s, c, rows, nrm)
    assert np.all(nrm[1] == 0)              # the zero token: nu = gamma = 0


def test_quantize_empty_and_deterministic(orc):
    d, b = 128, 3
    ctx, pi, s, c = ctx_for(orc, d, b)
    x = workloads.normal((500, d), 4, 10, DEV)
    planes, norms = tq.alloc_records(500, d, b)
    tq.tq_quantize_kv(ctx, x[:0], planes, norms, n_tokens=0)   # no-op
    torch.cuda.synchronize()
    assert not planes.any()
    p1, n1 = gpu_quantize(ctx, x)
    p2, n2 = gpu_quantize(ctx, x)
    assert np.array_equal(p1, p2) and np.array_equal(n1, n2)


def test_quantize_rejects_bad_arguments(orc):
    ctx, pi, s, c = ctx_for(orc, 128, 3)
    L = tq.lib()
    x = torch.zeros((4, 128), device=DEV)
    planes, norms = tq.alloc_records(4, 128, 3)
    st = L.tq_quantize_kv(ctx.handle, x.data_ptr(), 7, 4, 1, 128, 0, planes.data_ptr(),
                          norms.data_ptr(), 4, 0, None)
    assert st == tq.TQ_ERR_INVALID_ARG
    st = L.tq_quantize_kv(ctx.handle, x.data_ptr(), 0, 4, 1, 64, 0, planes.data_ptr(),
                          norms.data_ptr(), 4, 0, None)
    assert st == tq.TQ_ERR_INVALID_ARG          # stride < d
    st = L.tq_quantize_kv(ctx.handle, x.data_ptr() + 4, 0, 4, 1, 128, 0, planes.data_ptr(),
                          norms.data_ptr(), 4, 0, None)
    assert st == tq.TQ_ERR_INVALID_ARG          # misaligned
    st = L.tq_quantize_kv(ctx.handle, x.data_ptr(), 0, -1, 1, 128, 0, planes.data_ptr(),
                          norms.data_ptr(), 4, 0, None)
    assert st == tq.TQ_ERR_INVALID_ARG


# ------------------------------------------------------------------ logits
def run_logits(ctx, q, planes, norms, n_kv, keys_stride_head, starts, lens, scale, n_q,
               logits_stride_head, total_len):
    batch = len(lens)
    q_t = torch.as_tensor(q, dtype=torch.float32, device=DEV).contiguous()
    ss = torch.as_tensor(starts, dtype=torch.int64, device=DEV)
    sl = torch.as_tensor(lens, dtype=torch.int32, device=DEV)
    logits = torch.full((n_q, logits_stride_head), float("nan"), device=DEV)
    ws = tq.workspace(tq.tq_attn_logits_workspace_bytes(ctx, batch, n_q, n_kv))
    tq.tq_attn_logits(ctx, q_t, batch, n_q, n_q * ctx.d, planes, norms, n_kv,
                      keys_stride_head, ss, sl, max(lens), scale, logits, logits_stride_head, ws)
    torch.cuda.synchronize()
    return logits.cpu().numpy()


@pytest.mark.parametrize("d,b,n_q,n_kv,lens", [
    (128, 3, 16, 1, [1024]),                  # tiny workload layout
    (128, 4, 32, 8, [1000, 37, 513]),         # GQA 4, ragged batch
    (128, 2, 32, 8, [777]),
    (128, 3, 8, 8, [300, 1]),                 # G = 1
    (128, 4, 6, 2, [129]),                    # G = 3 (partial row block)
    (200, 4, 8, 2, [333, 70]),
    (1536, 2, 4, 1, [100]),
    (64, 4, 32, 8, [1000, 37, 513]),          # d <= 64: folded operands, GQA 4
    (64, 3, 8, 4, [300, 1]),                  # folded, G = 2
    (32, 2, 12, 4, [257]),                    # one word, folded, G = 3
    (64, 2, 40, 4, [200]),                    # G = 10: general kernel, unfolded
])
def test_logits_parity_oracle_records(orc, d, b, n_q, n_kv, lens):
    say("logits", d, b, n_q, n_kv, lens)
    ctx, pi, s, c = ctx_for(orc, d, b)
    total = sum(lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).tolist()
    x = workloads.normal((n_kv, total, d), 5, 10, "cpu").double().numpy()
    q = workloads.normal((len(lens), n_q, d), 5, 12, "cpu").numpy()
    recs = [orc.quantize(d, b, pi, s, c, x[h]) for h in range(n_kv)]
    planes = np.concatenate([r["planes"] for r in recs])
    norms = np.concatenate([r["norms"] for r in recs])
    P = torch.as_tensor(planes.view(np.int32), device=DEV)
    N = torch.as_tensor(norms.view(np.int16), device=DEV)
    scale = 1.0 / np.sqrt(d)
    got = run_logits(ctx, q, P, N, n_kv, total, starts, lens, scale, n_q, total, total)
    G = n_q // n_kv
    for bi, (st, ln) in enumerate(zip(starts, lens)):
        for h in range(n_kv):
            rp = planes[h * total + st: h * total + st + ln]
            rn = norms[h * total + st: h * total + st + ln]
            ref = orc.estimate(d, b, pi, s, c, q[bi, h * G:(h + 1) * G].astype(np.float64),
                               rp, rn, scale=scale)
            g = got[h * G:(h + 1) * G, st:st + ln]
            assert rel_err_rows(g, ref) < TOL, (bi, h, rel_err_rows(g, ref))


@pytest.mark.parametrize("d,b", [(128, 4), (64, 3)])
def test_prepared_queries_match_one_call(orc, d, b):
    """tq_attn_prepare + tq_attn_logits_prepared == tq_attn_logits, and one
    prepared workspace serves two caches (d = 64: folded operands)."""
    ctx, pi, s, c = ctx_for(orc, d, b)
    n = 700
    P, N = workloads.random_records(2 * n, tq.tq_record_words(d, b), 5, DEV)
    q = workloads.normal((1, 8, d), 5, 12, DEV)
    ss = torch.zeros(1, dtype=torch.int64, device=DEV)
    sl = torch.full((1,), n, dtype=torch.int32, device=DEV)
    ws = tq.workspace(tq.tq_attn_logits_workspace_bytes(ctx, 1, 8, 2))
    one = torch.empty((8, n), device=DEV)
    tq.tq_attn_logits(ctx, q, 1, 8, 8 * d, P, N, 2, n, ss, sl, n, 0.5, one, n, ws)
    ws2 = tq.workspace(tq.tq_attn_logits_workspace_bytes(ctx, 1, 8, 2))
    tq.tq_attn_prepare(ctx, q, 1, 8, 8 * d, 2, ws2)
    two = torch.empty((8, n), device=DEV)
    tq.tq_attn_logits_prepared(ctx, ws2, 1, 8, P, N, 2, n, ss, sl, n, 0.5, two, n)
    torch.cuda.synchronize()
    assert torch.equal(one, two)
    # second cache (records n..2n-1 addressed through seq_start) with the same workspace
    ss2 = torch.full((1,), 0, dtype=torch.int64, device=DEV)
    three = torch.empty((8, n), device=DEV)
    tq.tq_attn_logits_prepared(ctx, ws2, 1, 8, P[n:], N[n:], 2, 0, ss2, sl, n, 0.5, three, n)
    torch.cuda.synchronize()
    ref = orc.estimate(d, b, pi, s, c, q[0, :4].double().cpu().numpy(),
                       P[n:].cpu().numpy().view(np.uint32), N[n:].cpu().numpy().view(np.uint16),
                       scale=0.5)
    assert rel_err_rows(three[:4].cpu().numpy(), ref) < TOL
    with pytest.raises(tq.TqError):
        tq.tq_attn_logits_prepared(ctx, ws2[:64], 1, 8, P, N, 2, n, ss, sl, n, 0.5, two, n)


@pytest.mark.parametrize("b", [2, 3, 4])
def test_one_call_long_ragged_matches_prepared(orc, b):
    """At lengths where every wave of the one-call kernel streams several tile
    groups (b >= 3: the groups of a sequence taken by its waves in turn; b = 2:
    contiguous chunks) and the sequences end inside a group, the one-call
    logits equal the prepared form's bit for bit, and nothing outside the
    sequences' logit ranges is written."""
    d, n_q, n_kv = 128, 32, 8
    ctx, pi, s, c = ctx_for(orc, d, b)
    lens = [150001, 70003]
    total = sum(lens)
    starts = [0, lens[0]]
    stride_head = total + 5
    P, N = workloads.random_records(n_kv * total, tq.tq_record_words(d, b), 21 + b, DEV)
    q = workloads.normal((2, n_q, d), 21 + b, 12, DEV)
    ss = torch.as_tensor(starts, dtype=torch.int64, device=DEV)
    sl = torch.as_tensor(lens, dtype=torch.int32, device=DEV)
    one = torch.full((n_q, stride_head), float("nan"), device=DEV)
    ws = tq.workspace(tq.tq_attn_logits_workspace_bytes(ctx, 2, n_q, n_kv))
    tq.tq_attn_logits(ctx, q, 2, n_q, n_q * d, P, N, n_kv, total, ss, sl, max(lens), 0.125,
                      one, stride_head, ws)
    ws2 = tq.workspace(tq.tq_attn_logits_workspace_bytes(ctx, 2, n_q, n_kv))
    tq.tq_attn_prepare(ctx, q, 2, n_q, n_q * d, n_kv, ws2)
    two = torch.full((n_q, stride_head), float("nan"), device=DEV)
    tq.tq_attn_logits_prepared(ctx, ws2, 2, n_q, P, N, n_kv, total, ss, sl, max(lens), 0.125,
                               two, stride_head)
    torch.cuda.synchronize()
    assert torch.equal(one[:, :total], two[:, :total])
    assert bool(torch.isfinite(one[:, :total]).all())
    assert bool(torch.isnan(one[:, total:]).all()) and bool(torch.isnan(two[:, total:]).all())
    # a few tokens of each sequence against the oracle (first, last, a group edge)
    G = n_q // n_kv
    for bi, (st, ln) in enumerate(zip(starts, lens)):
        for h in (0, n_kv - 1):
            for t in (0, 63, 64, ln - 1):
                rec = h * total + st + t
                ref = orc.estimate(d, b, pi, s, c, q[bi, h * G:(h + 1) * G].double().cpu().numpy(),
                                   P[rec:rec + 1].cpu().numpy().view(np.uint32),
                                   N[rec:rec + 1].cpu().numpy().view(np.uint16), scale=0.125)
                got = one[h * G:(h + 1) * G, st + t:st + t + 1].cpu().numpy()
                assert np.abs(got - ref).max() <= 1e-3 * max(1.0, np.abs(ref).max()), (bi, h, t)


def _step_case(orc, d, b, mse, dtype, n_heads, n_tok, L, n_q, n_kv):
    if mse:
        pi = orc.make_rotation(d, 0)[2]
        c = orc.lloyd_max(d, b)[0].astype(np.float32)
        ctx, s = tq.tq_ctx_create_mse(d, b, pi, c), None
    else:
        ctx, pi, s, c = ctx_for(orc, d, b)
    kx = (workloads.normal((n_heads, n_tok, d), 14, 10, DEV) * 1.7).to(dtype)
    vx = (workloads.normal((n_heads, n_tok, d), 14, 11, DEV) * 0.6).to(dtype)
    q = workloads.normal((L, n_q, d), 14, 12, DEV)
    cap = n_tok + 5
    bufs = [tq.alloc_records(n_heads * cap, d, b) for _ in range(4)]
    ws_bytes = tq.tq_attn_logits_workspace_bytes(ctx, L, n_q, n_kv)
    ws1, ws2 = tq.workspace(ws_bytes), tq.workspace(ws_bytes)
    ws1.zero_()
    ws2.zero_()
    tq.tq_decode_step_prepare(ctx, kx, vx, *bufs[0], *bufs[1], q, L, n_q, n_q * d, n_kv, ws1,
                              dst_stride_head=cap, dst_token0=5)
    tq.tq_quantize_kv(ctx, kx, *bufs[2], dst_stride_head=cap, dst_token0=5)
    tq.tq_quantize_kv(ctx, vx, *bufs[3], dst_stride_head=cap, dst_token0=5)
    tq.tq_attn_prepare(ctx, q, L, n_q, n_q * d, n_kv, ws2)
    torch.cuda.synchronize()
    for x_, y_ in zip(bufs[0] + bufs[1], bufs[2] + bufs[3]):
        assert torch.equal(x_, y_)
    assert torch.equal(ws1, ws2)
    return ctx, pi, s, c, kx, bufs[0], cap


@pytest.mark.parametrize("d,b,mse,dtype,n_heads,n_tok,L,n_q,n_kv", [
    (128, 4, False, torch.bfloat16, 256, 1, 32, 32, 8),   # one token per (kv head, layer)
    (128, 3, False, torch.float32, 7, 70, 2, 16, 1),       # several tiles, G = 16
    (128, 2, True, torch.bfloat16, 24, 3, 3, 8, 8),        # MSE-only records
    (200, 4, False, torch.float32, 5, 9, 2, 8, 2),          # other d: separate launches
    (64, 3, False, torch.bfloat16, 16, 2, 4, 8, 2),         # d = 64: folded preparation
])
def test_decode_step_prepare_matches_separate_calls(orc, d, b, mse, dtype, n_heads, n_tok, L,
                                                    n_q, n_kv):
    """tq_decode_step_prepare == tq_quantize_kv (K), tq_quantize_kv (V) and
    tq_attn_prepare, bit for bit; the key records also against the oracle."""
    say("decode step prepare", d, b, mse, dtype, n_heads, n_tok)
    ctx, pi, s, c, kx, (kp, kn), cap = _step_case(orc, d, b, mse, dtype, n_heads, n_tok, L,
                                                  n_q, n_kv)
    if not mse:
        P = kp.cpu().numpy().view(np.uint32).reshape(n_heads, cap, -1)[:, 5:5 + n_tok]
        N = kn.cpu().numpy().view(np.uint16).reshape(n_heads, cap, 2)[:, 5:5 + n_tok]
        check_quantize(orc, d, b, kx.reshape(n_heads * n_tok, d), pi, s, c,
                       P.reshape(n_heads * n_tok, -1), N.reshape(n_heads * n_tok, 2))


def test_decode_step_prepare_rejects_bad_arguments(orc):
    d, b = 128, 4
    ctx, pi, s, c = ctx_for(orc, d, b)
    kx = torch.zeros((4, 1, d), dtype=torch.bfloat16, device=DEV)
    q = torch.zeros((1, 8, d), device=DEV)
    kp, kn = tq.alloc_records(4, d, b)
    vp, vn = tq.alloc_records(4, d, b)
    ws = tq.workspace(tq.tq_attn_logits_workspace_bytes(ctx, 1, 8, 2))
    with pytest.raises(tq.TqError):      # workspace too small
        tq.tq_decode_step_prepare(ctx, kx, kx, kp, kn, vp, vn, q, 1, 8, 8 * d, 2, ws[:16],
                                  dst_stride_head=1)
    with pytest.raises(tq.TqError):      # n_q not a multiple of n_kv
        tq.tq_decode_step_prepare(ctx, kx, kx, kp, kn, vp, vn, q, 1, 8, 8 * d, 3, ws,
                                  dst_stride_head=1)
    with pytest.raises(tq.TqError):      # NULL value cache
        tq.tq_decode_step_prepare(ctx, kx, kx, kp, kn, None, vn, q, 1, 8, 8 * d, 2, ws,
                                  dst_stride_head=1)
    torch.cuda.synchronize()
    assert not kp.any() and not kn.any()


def test_logits_random_records_and_zero_query(orc):
    d, b = 128, 4
    ctx, pi, s, c = ctx_for(orc, d, b)
    n = 2000
    P, N = workloads.random_records(n, tq.tq_record_words(d, b), 2, DEV)
    q = workloads.normal((1, 4, d), 2, 12, "cpu").numpy()
    q[0, 2] = 0.0                              # an all-zero query head
    got = run_logits(ctx, q, P, N, 1, n, [0], [n], 1.0, 4, n, n)
    ref = orc.estimate(d, b, pi, s, c, q[0].astype(np.float64), P.cpu().numpy().view(np.uint32),
                       N.cpu().numpy().view(np.uint16))
    assert rel_err_rows(np.delete(got, 2, 0), np.delete(ref, 2, 0)) < TOL
    assert np.all(got[2] == 0.0)


def test_logits_empty_sequence_writes_nothing(orc):
    d, b = 128, 3
    ctx, pi, s, c = ctx_for(orc, d, b)
    P, N = workloads.random_records(64, tq.tq_record_words(d, b), 3, DEV)
    q = np.ones((2, 4, d), np.float32)
    got = run_logits(ctx, q, P, N, 1, 64, [0, 10], [0, 20], 1.0, 4, 64, 64)
    assert np.all(np.isnan(got[:, :10])) and np.all(np.isnan(got[:, 30:]))
    assert np.all(np.isfinite(got[:, 10:30]))


# ---------------------------------------------------------- attention output
def run_vout(ctx, p, P, N, n_kv, vstride, starts, lens, n_q, p_stride):
    """tq_attn_output with weights p (numpy [n_q, p_stride]) -> numpy [batch, n_q, d]."""
    batch = len(lens)
    p_t = torch.as_tensor(np.ascontiguousarray(p, np.float32), device=DEV)
    ss = torch.as_tensor(np.asarray(starts, np.int64), device=DEV)
    sl = torch.as_tensor(np.asarray(lens, np.int32), device=DEV)
    out = torch.full((batch, n_q, ctx.d), float("nan"), device=DEV)
    mx = max(lens) if lens else 0
    ws = tq.workspace(tq.tq_attn_output_workspace_bytes(ctx, batch, n_q, n_kv, mx))
    tq.tq_attn_output(ctx, p_t, p_stride, batch, n_q, P, N, n_kv, vstride, ss, sl, mx, out,
                      n_q * ctx.d, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("d,b,n_q,n_kv,lens,signed", [
    (128, 3, 16, 1, [1024], False),           # tiny layout: G = 16 (4 row blocks)
    (128, 4, 32, 8, [1000, 37, 513], False),  # GQA 4, ragged batch
    (128, 2, 8, 8, [300, 1], True),           # G = 1, signed weights (the sum is linear)
    (128, 4, 6, 2, [700], False),             # G = 3 (partial row block)
    (200, 4, 8, 2, [333, 70], False),
    (1536, 2, 4, 1, [150], True),
    (64, 3, 16, 4, [257, 600], False),        # d = 64: two words, idle waves in a slice
])
def test_attn_output_parity(orc, d, b, n_q, n_kv, lens, signed):
    say("attn output", d, b, n_q, n_kv, lens)
    ctx, pi, s, c = ctx_for(orc, d, b)
    total = sum(lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).tolist()
    x = workloads.normal((n_kv, total, d), 8, 11, "cpu").double().numpy()
    recs = [orc.quantize(d, b, pi, s, c, x[h]) for h in range(n_kv)]
    planes = np.concatenate([r["planes"] for r in recs])
    norms = np.concatenate([r["norms"] for r in recs])
    rng = np.random.default_rng(9)
    p = rng.random((n_q, total)) if not signed else rng.standard_normal((n_q, total))
    p = p.astype(np.float32)
    P = torch.as_tensor(planes.view(np.int32), device=DEV)
    N = torch.as_tensor(norms.view(np.int16), device=DEV)
    got = run_vout(ctx, p, P, N, n_kv, total, starts, lens, n_q, total)
    G = n_q // n_kv
    deq = [orc.dequantize(d, b, pi, s, c, r["planes"], r["norms"]) for r in recs]   # [total, d]
    for bi, (st, ln) in enumerate(zip(starts, lens)):
        for hq in range(n_q):
            ref = p[hq, st:st + ln].astype(np.float64) @ deq[hq // G][st:st + ln]
            assert rel_err_rows(got[bi, hq][None], ref[None]) < TOL, (bi, hq)


def test_attn_output_empty_sequence_is_zero(orc):
    d, b = 128, 4
    ctx, pi, s, c = ctx_for(orc, d, b)
    P, N = workloads.random_records(64, tq.tq_record_words(d, b), 3, DEV)
    p = np.ones((4, 64), np.float32)
    got = run_vout(ctx, p, P, N, 1, 64, [0, 10], [0, 20], 4, 64)
    assert np.all(got[0] == 0.0)
    deq = orc.dequantize(d, b, pi, s, c, P.cpu().numpy().view(np.uint32),
                         N.cpu().numpy().view(np.uint16))
    ref = deq[10:30].sum(axis=0)
    assert rel_err_rows(got[1], np.tile(ref, (4, 1))) < TOL


def test_attn_output_rejects_bad_arguments(orc):
    d, b = 128, 3
    ctx, pi, s, c = ctx_for(orc, d, b)
    P, N = workloads.random_records(16, tq.tq_record_words(d, b), 3, DEV)
    p = torch.ones((4, 16), device=DEV)
    ss = torch.zeros(1, dtype=torch.int64, device=DEV)
    sl = torch.full((1,), 16, dtype=torch.int32, device=DEV)
    out = torch.empty((1, 4, d), device=DEV)
    ws = tq.workspace(tq.tq_attn_output_workspace_bytes(ctx, 1, 4, 1, 16))
    with pytest.raises(tq.TqError):      # n_q not a multiple of n_kv
        tq.tq_attn_output(ctx, p, 16, 1, 4, P, N, 3, 16, ss, sl, 16, out, 4 * d, ws)
    with pytest.raises(tq.TqError):      # workspace too small
        tq.tq_attn_output(ctx, p, 16, 1, 4, P, N, 1, 16, ss, sl, 16, out, 4 * d, ws[:16])


# ---------------------------------------------------- fused decode attention
def softmax_rows(x):
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=-1, keepdims=True)


@pytest.mark.parametrize("d,b,n_q,n_kv,lens", [
    (128, 3, 16, 1, [1024]),                  # tiny layout, G = 16
    (128, 4, 32, 8, [1000, 37, 513]),         # GQA 4, ragged batch
    (128, 2, 8, 8, [300, 1]),                 # G = 1, a one-token sequence
    (128, 4, 6, 2, [700]),                    # G = 3
    (200, 4, 8, 2, [333, 70]),
    (1536, 2, 4, 1, [150]),
    (64, 4, 8, 1, [513, 3]),                  # d = 64, G = 8 (two row blocks)
    (64, 3, 8, 2, [300, 700]),                # d = 64, G = 4 (unfolded preparation)
])
def test_attn_decode_parity(orc, d, b, n_q, n_kv, lens):
    say("attn decode", d, b, n_q, n_kv, lens)
    ctx, pi, s, c = ctx_for(orc, d, b)
    total = sum(lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).tolist()
    xk = workloads.normal((n_kv, total, d), 12, 10, "cpu").double().numpy()
    xv = workloads.normal((n_kv, total, d), 12, 11, "cpu").double().numpy()
    q = workloads.normal((len(lens), n_q, d), 12, 12, "cpu").numpy()
    rk = [orc.quantize(d, b, pi, s, c, xk[h]) for h in range(n_kv)]
    rv = [orc.quantize(d, b, pi, s, c, xv[h]) for h in range(n_kv)]
    cat = lambda rs, key: np.concatenate([r[key] for r in rs])
    KP = torch.as_tensor(cat(rk, "planes").view(np.int32), device=DEV)
    KN = torch.as_tensor(cat(rk, "norms").view(np.int16), device=DEV)
    VP = torch.as_tensor(cat(rv, "planes").view(np.int32), device=DEV)
    VN = torch.as_tensor(cat(rv, "norms").view(np.int16), device=DEV)
    batch, scale = len(lens), 1.0 / np.sqrt(d)
    ss = torch.as_tensor(np.asarray(starts, np.int64), device=DEV)
    sl = torch.as_tensor(np.asarray(lens, np.int32), device=DEV)
    out = torch.full((batch, n_q, d), float("nan"), device=DEV)
    ws = tq.workspace(tq.tq_attn_decode_workspace_bytes(ctx, batch, n_q, n_kv, max(lens)))
    tq.tq_attn_decode(ctx, torch.as_tensor(q, device=DEV), batch, n_q, n_q * d, KP, KN, VP, VN,
                      n_kv, total, ss, sl, max(lens), scale, out, n_q * d, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    G = n_q // n_kv
    deq = [orc.dequantize(d, b, pi, s, c, r["planes"], r["norms"]) for r in rv]
    for bi, (st, ln) in enumerate(zip(starts, lens)):
        for h in range(n_kv):
            lg = orc.estimate(d, b, pi, s, c, q[bi, h * G:(h + 1) * G].astype(np.float64),
                              rk[h]["planes"][st:st + ln], rk[h]["norms"][st:st + ln], scale=scale)
            ref = softmax_rows(lg) @ deq[h][st:st + ln]
            assert rel_err_rows(got[bi, h * G:(h + 1) * G], ref) < TOL, (bi, h)


def test_attn_decode_empty_sequence_is_zero(orc):
    d, b = 128, 4
    ctx, pi, s, c = ctx_for(orc, d, b)
    P, N = workloads.random_records(64, tq.tq_record_words(d, b), 3, DEV)
    q = workloads.normal((2, 4, d), 3, 12, DEV)
    ss = torch.tensor([0, 10], dtype=torch.int64, device=DEV)
    sl = torch.tensor([0, 20], dtype=torch.int32, device=DEV)
    out = torch.full((2, 4, d), float("nan"), device=DEV)
    ws = tq.workspace(tq.tq_attn_decode_workspace_bytes(ctx, 2, 4, 1, 20))
    tq.tq_attn_decode(ctx, q, 2, 4, 4 * d, P, N, P, N, 1, 64, ss, sl, 20, 1.0, out, 4 * d, ws)
    torch.cuda.synchronize()
    assert torch.all(out[0] == 0) and torch.isfinite(out[1]).all()


# ---------------------------------------------------------------- dequantize
@pytest.mark.parametrize("d,b,n", [(128, 3, 1024), (128, 4, 100), (200, 2, 130), (1536, 4, 20),
                                   (64, 2, 70)])
def test_dequantize_parity(orc, d, b, n):
    say("dequantize", d, b, n)
    ctx, pi, s, c = ctx_for(orc, d, b)
    x = workloads.normal((n, d), 6, 10, "cpu").double().numpy()
    ref_rec = orc.quantize(d, b, pi, s, c, x)
    ref = orc.dequantize(d, b, pi, s, c, ref_rec["planes"], ref_rec["norms"])
    P = torch.as_tensor(ref_rec["planes"].view(np.int32), device=DEV)
    N = torch.as_tensor(ref_rec["norms"].view(np.int16), device=DEV)
    out = torch.full((n, d + 3), float("nan"), device=DEV)
    tq.tq_dequantize(ctx, P, N, n, out, out_ld=d + 3)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isnan(got[:, d:]))
    assert rel_err_rows(got[:, :d], ref) < TOL


@pytest.mark.parametrize("b,mse,n,pad", [
    (4, False, 16384 + 37, 0),      # register-resident d = 128 form, ragged last tile
    (3, False, 70000, 3),           # out_ld = d + 3: staged stores, several tiles per workgroup
    (2, True, 70001, 0),            # MSE-only records, several tiles per workgroup
    (3, True, 70000, 0),
    (1, True, 65600, 2),            # MSE b = 1 with staged stores
])
def test_dequantize_d128_resident(orc, b, mse, n, pad):
    """tq_dequantize at d = 128 with enough records for the register-resident
    kernel: sampled rows (first and last tiles, random rows) against the
    oracle's dequantization of the same records; padding columns untouched."""
    say("dequantize d128 resident", b, mse, n, pad)
    d = 128
    if mse:
        pi = orc.make_rotation(d, 0)[2]
        c = orc.lloyd_max(d, b)[0].astype(np.float32)
        ctx = tq.tq_ctx_create_mse(d, b, pi, c)
        s = None
    else:
        ctx, pi, s, c = ctx_for(orc, d, b)
    x = workloads.normal((n, d), 8, 10, DEV) * 1.7
    x[3] = 0.0
    P, N = tq.alloc_records(n, d, b)
    tq.tq_quantize_kv(ctx, x, P, N)
    out = torch.full((n, d + pad), float("nan"), device=DEV)
    tq.tq_dequantize(ctx, P, N, n, out, out_ld=d + pad)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(70), np.arange(n - 70, n),
                                     np.random.default_rng(9).integers(0, n, 200)]))
    idx = torch.as_tensor(rows, device=DEV)
    rp = P[idx].cpu().numpy().view(np.uint32)
    rn = N[idx].cpu().numpy().view(np.uint16)
    if mse:
        ref = orc.dequantize_mse(d, b, pi, c, rp, rn)
    else:
        ref = orc.dequantize(d, b, pi, s, c, rp, rn)
    got = out[idx].cpu().numpy()
    assert rel_err_rows(got[:, :d], ref) < TOL
    if pad:
        assert np.all(np.isnan(out[:, d:].cpu().numpy()))
    assert torch.isfinite(out[:, :d]).all()


# -------------------------------------------------------------------- search
def topk_ok(gi, gs, ref_scores, k, tol=TOL):
    """GPU (idx, score) rows vs exact oracle scores: every returned index is
    within tolerance of the k-th best, scores match, order is valid."""
    for a in range(gi.shape[0]):
        row = ref_scores[a]
        rms = np.sqrt(np.mean(row ** 2))
        order = np.lexsort((np.arange(row.size), -row))
        kth = row[order[k - 1]]
        assert len(set(gi[a].tolist())) == k
        for j in range(k):
            idx = gi[a, j]
            assert 0 <= idx < row.size
            assert abs(gs[a, j] - row[idx]) <= tol * max(abs(row[idx]), rms)
            assert row[idx] >= kth - 2 * tol * rms          # a true top-k member up to ties
        # true top-k members clearly above the boundary must be returned
        for idx in order[:k]:
            if row[idx] > kth + 2 * tol * rms:
                assert idx in gi[a]
    assert topk_order_ok(gi, gs)


@pytest.mark.parametrize("d,b,n_db,n_q,k", [(128, 4, 5000, 70, 10), (200, 2, 40000, 5, 10),
                                            (200, 4, 3000, 3, 1), (1536, 2, 2000, 4, 10),
                                            (128, 3, 100, 2, 64),
                                            # two query tiles of 256 (the second ragged),
                                            # two record chunks with a ragged last tile
                                            (128, 3, 20000, 300, 10),
                                            # above 2048 queries the later chunks hold
                                            # 16384 records: three chunks, nine query tiles
                                            (128, 4, 23432, 2100, 10)])
def test_search_parity(orc, d, b, n_db, n_q, k):
    say("search", d, b, n_db, n_q, k)
    ctx, pi, s, c = ctx_for(orc, d, b)
    db = workloads.unit_rows(n_db, d, 7, 15, "cpu").double().numpy()
    qs = workloads.unit_rows(n_q, d, 7, 16, "cpu").numpy()
    rec = orc.quantize(d, b, pi, s, c, db)
    ref = orc.estimate(d, b, pi, s, c, qs.astype(np.float64), rec["planes"], rec["norms"])
    P = torch.as_tensor(rec["planes"].view(np.int32), device=DEV)
    N = torch.as_tensor(rec["norms"].view(np.int16), device=DEV)
    Q = torch.as_tensor(qs, device=DEV)
    oi = torch.empty((n_q, k), dtype=torch.int64, device=DEV)
    os_ = torch.empty((n_q, k), dtype=torch.float32, device=DEV)
    ws = tq.workspace(tq.tq_search_workspace_bytes(ctx, n_q, n_db, k))
    tq.tq_search_topk(ctx, Q, n_q, P, N, n_db, k, oi, os_, ws)
    torch.cuda.synchronize()
    topk_ok(oi.cpu().numpy(), os_.cpu().numpy(), ref, k)


def test_search_fewer_records_than_k(orc):
    d, b = 128, 2
    ctx, pi, s, c = ctx_for(orc, d, b)
    P, N = workloads.random_records(5, tq.tq_record_words(d, b), 4, DEV)
    Q = workloads.unit_rows(2, d, 4, 16, DEV)
    oi = torch.empty((2, 8), dtype=torch.int64, device=DEV)
    os_ = torch.empty((2, 8), dtype=torch.float32, device=DEV)
    ws = tq.workspace(tq.tq_search_workspace_bytes(ctx, 2, 5, 8))
    tq.tq_search_topk(ctx, Q, 2, P, N, 5, 8, oi, os_, ws)
    torch.cuda.synchronize()
    gi = oi.cpu().numpy()
    assert np.all(gi[:, 5:] == -1) and np.all(np.isneginf(os_.cpu().numpy()[:, 5:]))
    assert sorted(gi[0, :5].tolist()) == [0, 1, 2, 3, 4]


def test_search_ties_by_index(orc):
    """Identical records score identically; the top-k lists them by index
    ascending (the tie rule of the ranking)."""
    d, b, n_db, k = 128, 4, 3000, 10
    ctx, pi, s, c = ctx_for(orc, d, b)
    db = workloads.unit_rows(n_db, d, 17, 15, "cpu").double().numpy()
    rec = orc.quantize(d, b, pi, s, c, db)
    planes, norms = rec["planes"].copy(), rec["norms"].copy()
    dup = [10, 500, 1700, 2999]
    for i in dup[1:]:
        planes[i], norms[i] = planes[dup[0]], norms[dup[0]]
    qs = np.stack([db[10], -db[10], db[1234]]).astype(np.float32)
    P = torch.as_tensor(planes.view(np.int32), device=DEV)
    N = torch.as_tensor(norms.view(np.int16), device=DEV)
    oi = torch.empty((3, k), dtype=torch.int64, device=DEV)
    os_ = torch.empty((3, k), dtype=torch.float32, device=DEV)
    ws = tq.workspace(tq.tq_search_workspace_bytes(ctx, 3, n_db, k))
    tq.tq_search_topk(ctx, torch.as_tensor(qs, device=DEV), 3, P, N, n_db, k, oi, os_, ws)
    torch.cuda.synchronize()
    gi, gs = oi.cpu().numpy(), os_.cpu().numpy()
    assert gi[0, :4].tolist() == dup and np.all(gs[0, :4] == gs[0, 0])
    assert topk_order_ok(gi, gs)
    ref = orc.estimate(d, b, pi, s, c, qs.astype(np.float64), planes, norms)
    topk_ok(gi, gs, ref, k)


# ------------------------------------------- the library's own set-up tables
@pytest.mark.parametrize("d,b,dtype,n", [(128, 4, torch.bfloat16, 3000),
                                         (128, 3, torch.float32, 700),
                                         (200, 2, torch.float32, 300)])
def test_library_tables_end_to_end(orc, d, b, dtype, n):
    """A context built from the library's own tq_make_rotation and
    tq_lloyd_max (as bench.py builds it): records against the oracle run on
    those same fp32 tables, and logits of those records against the oracle's
    estimate.  The tables themselves are compared with the oracle's on the
    CPU (test_host_abi)."""
    say("library tables", d, b, dtype, n)
    pi, s = tq.tq_make_rotation(d, 0)
    c = tq.tq_lloyd_max(d, b - 1)[0]
    ctx = tq.TqContext(d, b, pi, s, c)
    x = (workloads.normal((n, d), 23, 10, DEV) * 1.3).to(dtype)
    planes, norms = gpu_quantize(ctx, x)
    stats = check_quantize(orc, d, b, x, pi, s, c, planes, norms)
    say("ok", stats)
    q = workloads.normal((1, 8, d), 23, 12, "cpu").numpy()
    P = torch.as_tensor(planes.view(np.int32), device=DEV)
    N = torch.as_tensor(norms.view(np.int16), device=DEV)
    got = run_logits(ctx, q, P, N, 1, n, [0], [n], 0.5, 8, n, n)
    ref = orc.estimate(d, b, pi, s, c, q[0].astype(np.float64), planes, norms, scale=0.5)
    assert rel_err_rows(got, ref) < TOL
    ctx.close()


# ------------------------------------------------------------ run-to-run
def test_repeat_calls_bit_identical(orc):
    """Logits, search, attention output and fused decode give bit-identical
    results when called twice on the same inputs (the search appends
    candidates with atomics; its merge must not depend on their order)."""
    d, b, n_q, n_kv = 128, 4, 32, 8
    ctx, pi, s, c = ctx_for(orc, d, b)
    lens = [3000, 777, 4096]
    batch, total = len(lens), sum(lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    P, N = workloads.random_records(n_kv * total, tq.tq_record_words(d, b), 19, DEV)
    q = workloads.normal((batch, n_q, d), 19, 12, DEV)
    ss = torch.as_tensor(starts, dtype=torch.int64, device=DEV)
    sl = torch.as_tensor(lens, dtype=torch.int32, device=DEV)
    mx = max(lens)

    def logits():
        out = torch.empty((n_q, total), device=DEV)
        ws = tq.workspace(tq.tq_attn_logits_workspace_bytes(ctx, batch, n_q, n_kv))
        tq.tq_attn_logits(ctx, q, batch, n_q, n_q * d, P, N, n_kv, total, ss, sl, mx, 0.1,
                          out, total, ws)
        return out

    def output(p):
        out = torch.empty((batch, n_q, d), device=DEV)
        ws = tq.workspace(tq.tq_attn_output_workspace_bytes(ctx, batch, n_q, n_kv, mx))
        tq.tq_attn_output(ctx, p, total, batch, n_q, P, N, n_kv, total, ss, sl, mx, out,
                          n_q * d, ws)
        return out

    def decode():
        out = torch.empty((batch, n_q, d), device=DEV)
        ws = tq.workspace(tq.tq_attn_decode_workspace_bytes(ctx, batch, n_q, n_kv, mx))
        tq.tq_attn_decode(ctx, q, batch, n_q, n_q * d, P, N, P, N, n_kv, total, ss, sl, mx,
                          0.1, out, n_q * d, ws)
        return out

    def search():
        n_db, nq, k = n_kv * total, 300, 10
        Q = workloads.unit_rows(nq, d, 19, 16, DEV)
        oi = torch.empty((nq, k), dtype=torch.int64, device=DEV)
        os_ = torch.empty((nq, k), dtype=torch.float32, device=DEV)
        ws = tq.workspace(tq.tq_search_workspace_bytes(ctx, nq, n_db, k))
        tq.tq_search_topk(ctx, Q, nq, P, N, n_db, k, oi, os_, ws)
        return oi, os_

    say("repeat calls")
    l1, l2 = logits(), logits()
    p = torch.softmax(l1, dim=1).contiguous()
    o1, o2 = output(p), output(p)
    d1, d2 = decode(), decode()
    s1, s2 = search(), search()
    torch.cuda.synchronize()
    assert torch.equal(l1, l2)
    assert torch.equal(o1, o2)
    assert torch.equal(d1, d2)
    assert torch.equal(s1[0], s2[0]) and torch.equal(s1[1], s2[1])


# -------------------------------- d = 128 bf16 cache fills (pipelined kernel)
def _stream_case(n_heads, n_tok, seed):
    """[n_heads][n_tok][136] bf16 source (x = first 128 columns, strided
    rows) with special vectors: zero, tiny (norm ~2^-75), huge (norm ~2^75),
    one loud channel, and a vector of bf16 subnormals."""
    base = workloads.normal((n_heads, n_tok, 136), seed, 10, DEV) * 1.4
    x = base[:, :, :128]
    if n_tok >= 8:
        x[0, 1] = 0.0
        x[0, 2] *= 2.0 ** -80
        x[n_heads - 1, n_tok - 1] *= 2.0 ** 70
        x[n_heads - 1, 3, 5] = 3.0e4
        x[n_heads // 2, 4] *= 2.0 ** -130
    return base.to(torch.bfloat16)


@pytest.mark.parametrize("b,mse,n_heads,n_tok,cap,t0", [
    (4, False, 1, 32, 32, 0),          # one block
    (3, False, 2, 96, 100, 3),         # a few blocks, records offset in a larger cache
    (2, False, 3, 4096, 4096, 0),      # several blocks per workgroup
    (4, False, 40, 2048, 2050, 1),     # 2560 blocks over 512 workgroups: ragged last round
    (1, True, 2, 160, 170, 5),         # MSE-only records
    (2, True, 5, 1024, 1024, 0),
    (3, True, 3, 2048, 2048, 0),
])
def test_quantize_stream_parity(orc, b, mse, n_heads, n_tok, cap, t0):
    """bf16 fills at d = 128 with a token count that is a multiple of 32:
    strided source rows and heads, records at h * cap + t0 + t of a larger
    cache (neighbours untouched), special vectors; records against the
    oracle (every row up to 8192 rows, else a sample plus every special row)."""
    say("quantize stream", b, mse, n_heads, n_tok, cap, t0)
    d = 128
    if mse:
        pi = orc.make_rotation(d, 0)[2]
        c = orc.lloyd_max(d, b)[0].astype(np.float32)
        ctx, s = tq.tq_ctx_create_mse(d, b, pi, c), None
    else:
        ctx, pi, s, c = ctx_for(orc, d, b)
    src = _stream_case(n_heads, n_tok, 30 + b)
    x = src[:, :, :d]
    P, N = tq.alloc_records(n_heads * cap, d, b)
    P.fill_(0x5A5A5A5A)
    N.fill_(0x3C3C)
    tq.tq_quantize_kv(ctx, x, P, N, n_tokens=n_tok, n_heads=n_heads,
                      x_stride_token=x.stride(1), x_stride_head=x.stride(0),
                      dst_stride_head=cap, dst_token0=t0)
    torch.cuda.synchronize()
    W = tq.tq_words_per_plane(d)
    gp = P.cpu().numpy().view(np.uint32).reshape(n_heads, cap, W * b)
    gn = N.cpu().numpy().view(np.uint16).reshape(n_heads, cap, 2)
    assert np.all(gp[:, :t0] == 0x5A5A5A5A) and np.all(gp[:, t0 + n_tok:] == 0x5A5A5A5A)
    assert np.all(gn[:, :t0] == 0x3C3C) and np.all(gn[:, t0 + n_tok:] == 0x3C3C)
    rows = gp[:, t0:t0 + n_tok].reshape(n_heads * n_tok, -1)
    nrm = gn[:, t0:t0 + n_tok].reshape(n_heads * n_tok, 2)
    xd = x.reshape(-1, d).double().cpu().numpy()
    n = n_heads * n_tok
    if n > 8192:
        special = [1, 2, 4, (n_heads // 2) * n_tok + 4, (n_heads - 1) * n_tok + 3, n - 1]
        pick = np.unique(np.concatenate([
            np.random.default_rng(5).choice(n, 4096, replace=False), special,
            np.arange(64), np.arange(n - 64, n)]))
    else:
        pick = np.arange(n)
    if mse:
        stats = check_records_mse(orc, d, b, pi, c, xd[pick], rows[pick], nrm[pick])
    else:
        stats = check_records(orc, d, b, pi, s, c, xd[pick], rows[pick], nrm[pick])
    say("ok", stats)
    if n_tok >= 8:
        assert np.all(nrm[1] == 0)              # the zero vector: nu = gamma = 0
    if mse:
        ctx.close()
