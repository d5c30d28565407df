"""GPU parity of the MSE-only mode (b code bits per coordinate, no QJL
stage) against the oracle's MSE functions, through the C ABI.

Same bar as the two-stage parity tests: codes bit-exact except within 1e-5
of a threshold, fp16 nu within one ulp and the gamma slot exactly 0; logits,
dequantized vectors, scores and attention outputs within 1e-3 of
max(|ref|, rms of the row).  Records fed to the consumers are the oracle's.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_vector_pi_amd as tq  # noqa: E402
import workloads  # noqa: E402
from helpers import TOL, check_records_mse, clear_padding, f16_ulp_diff, rel_err_rows  # noqa: E402
from test_gpu_parity import run_logits, run_vout, say, softmax_rows, topk_ok  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"

_ctx_cache = {}


def mse_ctx(orc, d, b, seed=0):
    key = (d, b, seed)
    if key not in _ctx_cache:
        pi = orc.make_rotation(d, seed)[2]
        c = orc.lloyd_max(d, b)[0].astype(np.float32)
        ctx = tq.tq_ctx_create_mse(d, b, pi, c)
        assert tq.tq_ctx_is_mse(ctx) == 1
        _ctx_cache[key] = (ctx, pi, c)
    return _ctx_cache[key]


def oracle_records(orc, d, b, pi, c, x):
    r = orc.quantize_mse(d, b, pi, c, x)
    return r["planes"], r["norms"]


def to_dev(planes, norms):
    return (torch.as_tensor(planes.view(np.int32), device=DEV),
            torch.as_tensor(norms.view(np.int16), device=DEV))


@pytest.mark.parametrize("d,b,dtype,n", [
    (128, 1, torch.float32, 1000),        # d = 128 kernel, ragged tail
    (128, 2, torch.bfloat16, 1000),
    (128, 3, torch.float32, 257),
    (200, 2, torch.float32, 300),         # generic kernel, padded last word
    (64, 1, torch.float32, 77),
    (64, 2, torch.bfloat16, 200),         # d = 64 token pairs (d = 128 kernel)
    (1536, 3, torch.float32, 33),
    (1536, 1, torch.bfloat16, 40),
])
def test_mse_quantize_parity(orc, d, b, dtype, n):
    say("mse quantize", d, b, dtype, n)
    ctx, pi, c = mse_ctx(orc, d, b)
    x = workloads.normal((n, d), 21, 10, DEV) * 2.0
    x[5] = 0.0                            # zero vector
    x = x.to(dtype)
    planes, norms = tq.alloc_records(n, d, b)
    tq.tq_quantize_kv(ctx, x.contiguous(), planes, norms)
    torch.cuda.synchronize()
    gp = planes.cpu().numpy().view(np.uint32)
    gn = norms.cpu().numpy().view(np.uint16)
    stats = check_records_mse(orc, d, b, pi, c, x.double().cpu().numpy(), gp, gn)
    if d % 32:
        pc = gp.copy()
        clear_padding(pc, d, b)
        assert np.array_equal(pc, gp)
    say("ok", stats)


@pytest.mark.parametrize("d,b,n", [(128, 3, 1024), (128, 1, 100), (200, 1, 130),
                                   (1536, 2, 20)])
def test_mse_dequantize_parity(orc, d, b, n):
    say("mse dequantize", d, b, n)
    ctx, pi, c = mse_ctx(orc, d, b)
    x = workloads.normal((n, d), 22, 10, "cpu").double().numpy()
    rp, rn = oracle_records(orc, d, b, pi, c, x)
    ref = orc.dequantize_mse(d, b, pi, c, rp, rn)
    P, N = to_dev(rp, rn)
    out = torch.full((n, d + 3), float("nan"), device=DEV)
    tq.tq_dequantize(ctx, P, N, n, out, out_ld=d + 3)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isnan(got[:, d:]))
    assert rel_err_rows(got[:, :d], ref) < TOL


@pytest.mark.parametrize("d,b,n_q,n_kv,lens", [
    (128, 3, 16, 1, [1024]),                  # G = 16
    (128, 1, 32, 8, [1000, 37, 513]),         # resident kernel, GQA 4, ragged batch
    (128, 2, 6, 2, [129]),                    # G = 3
    (200, 3, 8, 2, [333, 70]),                # generic kernel
    (1536, 1, 4, 1, [100]),
    (64, 3, 8, 2, [300, 77]),                 # d <= 64: folded operands
    (32, 2, 4, 4, [129]),                     # one word, folded, G = 1
])
def test_mse_logits_parity(orc, d, b, n_q, n_kv, lens):
    say("mse logits", d, b, n_q, n_kv, lens)
    ctx, pi, c = mse_ctx(orc, d, b)
    total = sum(lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).tolist()
    x = workloads.normal((n_kv, total, d), 23, 10, "cpu").double().numpy()
    q = workloads.normal((len(lens), n_q, d), 23, 12, "cpu").numpy()
    recs = [oracle_records(orc, d, b, pi, c, x[h]) for h in range(n_kv)]
    planes = np.concatenate([r[0] for r in recs])
    norms = np.concatenate([r[1] for r in recs])
    P, N = to_dev(planes, norms)
    scale = 1.0 / np.sqrt(d)
    got = run_logits(ctx, q, P, N, n_kv, total, starts, lens, scale, n_q, total, total)
    G = n_q // n_kv
    for bi, (st, ln) in enumerate(zip(starts, lens)):
        for h in range(n_kv):
            ref = orc.estimate_mse(d, b, pi, c, q[bi, h * G:(h + 1) * G].astype(np.float64),
                                   planes[h * total + st: h * total + st + ln],
                                   norms[h * total + st: h * total + st + ln], scale=scale)
            g = got[h * G:(h + 1) * G, st:st + ln]
            assert rel_err_rows(g, ref) < TOL, (bi, h, rel_err_rows(g, ref))


@pytest.mark.parametrize("d,b,n_db,n_q,k", [(128, 3, 5000, 70, 10), (200, 2, 20000, 5, 10),
                                            (1536, 1, 2000, 4, 10)])
def test_mse_search_parity(orc, d, b, n_db, n_q, k):
    say("mse search", d, b, n_db, n_q, k)
    ctx, pi, c = mse_ctx(orc, d, b)
    db = workloads.unit_rows(n_db, d, 24, 15, "cpu").double().numpy()
    qs = workloads.unit_rows(n_q, d, 24, 16, "cpu").numpy()
    rp, rn = oracle_records(orc, d, b, pi, c, db)
    ref = orc.estimate_mse(d, b, pi, c, qs.astype(np.float64), rp, rn)
    P, N = to_dev(rp, rn)
    oi = torch.empty((n_q, k), dtype=torch.int64, device=DEV)
    os_ = torch.empty((n_q, k), dtype=torch.float32, device=DEV)
    ws = tq.workspace(tq.tq_search_workspace_bytes(ctx, n_q, n_db, k))
    tq.tq_search_topk(ctx, torch.as_tensor(qs, device=DEV), n_q, P, N, n_db, k, oi, os_, ws)
    torch.cuda.synchronize()
    topk_ok(oi.cpu().numpy(), os_.cpu().numpy(), ref, k)


@pytest.mark.parametrize("d,b,n_q,n_kv,lens,signed", [
    (128, 2, 32, 8, [1000, 37, 513], False),
    (128, 1, 16, 1, [700], False),            # G = 16
    (200, 3, 8, 2, [333, 70], False),
    (1536, 1, 4, 1, [150], True),
])
def test_mse_attn_output_parity(orc, d, b, n_q, n_kv, lens, signed):
    say("mse attn output", d, b, n_q, n_kv, lens)
    ctx, pi, c = mse_ctx(orc, d, b)
    total = sum(lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).tolist()
    x = workloads.normal((n_kv, total, d), 25, 11, "cpu").double().numpy()
    recs = [oracle_records(orc, d, b, pi, c, x[h]) for h in range(n_kv)]
    P, N = to_dev(np.concatenate([r[0] for r in recs]), np.concatenate([r[1] for r in recs]))
    rng = np.random.default_rng(25)
    p = (rng.standard_normal((n_q, total)) if signed else rng.random((n_q, total)))
    p = p.astype(np.float32)
    got = run_vout(ctx, p, P, N, n_kv, total, starts, lens, n_q, total)
    G = n_q // n_kv
    deq = [orc.dequantize_mse(d, b, pi, c, r[0], r[1]) for r in recs]
    for bi, (st, ln) in enumerate(zip(starts, lens)):
        for hq in range(n_q):
            ref = p[hq, st:st + ln].astype(np.float64) @ deq[hq // G][st:st + ln]
            assert rel_err_rows(got[bi, hq][None], ref[None]) < TOL, (bi, hq)


@pytest.mark.parametrize("d,b,n_q,n_kv,lens", [
    (128, 3, 16, 1, [1024]),
    (128, 1, 8, 8, [300, 1]),                 # G = 1, a one-token sequence
    (200, 2, 8, 2, [333, 70]),
    (1536, 3, 4, 1, [140]),                   # 12 word slices
])
def test_mse_attn_decode_parity(orc, d, b, n_q, n_kv, lens):
    say("mse attn decode", d, b, n_q, n_kv, lens)
    ctx, pi, c = mse_ctx(orc, d, b)
    total = sum(lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).tolist()
    xk = workloads.normal((n_kv, total, d), 26, 10, "cpu").double().numpy()
    xv = workloads.normal((n_kv, total, d), 26, 11, "cpu").double().numpy()
    q = workloads.normal((len(lens), n_q, d), 26, 12, "cpu").numpy()
    rk = [oracle_records(orc, d, b, pi, c, xk[h]) for h in range(n_kv)]
    rv = [oracle_records(orc, d, b, pi, c, xv[h]) for h in range(n_kv)]
    KP, KN = to_dev(np.concatenate([r[0] for r in rk]), np.concatenate([r[1] for r in rk]))
    VP, VN = to_dev(np.concatenate([r[0] for r in rv]), np.concatenate([r[1] for r in rv]))
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
    deq = [orc.dequantize_mse(d, b, pi, c, r[0], r[1]) for r in rv]
    for bi, (st, ln) in enumerate(zip(starts, lens)):
        for h in range(n_kv):
            lg = orc.estimate_mse(d, b, pi, c, q[bi, h * G:(h + 1) * G].astype(np.float64),
                                  rk[h][0][st:st + ln], rk[h][1][st:st + ln], scale=scale)
            ref = softmax_rows(lg) @ deq[h][st:st + ln]
            assert rel_err_rows(got[bi, h * G:(h + 1) * G], ref) < TOL, (bi, h)


def test_mse_roundtrip_through_gpu(orc):
    """GPU quantize then GPU dequantize matches the oracle's round trip of the
    same input (records compared up to threshold ties first)."""
    d, b, n = 128, 2, 512
    ctx, pi, c = mse_ctx(orc, d, b)
    x = workloads.normal((n, d), 27, 10, DEV)
    planes, norms = tq.alloc_records(n, d, b)
    tq.tq_quantize_kv(ctx, x, planes, norms)
    out = torch.empty((n, d), device=DEV)
    tq.tq_dequantize(ctx, planes, norms, n, out)
    torch.cuda.synchronize()
    gp = planes.cpu().numpy().view(np.uint32)
    gn = norms.cpu().numpy().view(np.uint16)
    ref = orc.dequantize_mse(d, b, pi, c, gp, gn)
    assert rel_err_rows(out.cpu().numpy(), ref) < TOL
