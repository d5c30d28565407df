"""GPU parity of the fractional-bit-width path (two instances over a channel
split) against the oracle's split functions, through the C ABI.

Quantize: each group's records to the quantize bar (codes and signs
bit-exact outside the oracle margins, fp16 norms within one ulp).  Logits,
dequantized vectors and attention outputs are fed oracle-produced records and
must agree within 1e-3 of max(|ref|, rms of the row).  All inputs are seeded.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_vector_pi_amd as tq  # noqa: E402
import workloads  # noqa: E402
from helpers import TOL, check_records_mse, f16_ulp_diff, rel_err_rows  # noqa: E402
from test_gpu_parity import check_quantize  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


_cache = {}


def instance(orc, d, b, seed, mse):
    """(TqContext, oracle instance tuple)."""
    key = (d, b, seed, mse)
    if key not in _cache:
        pi64, s64, pi32, s32 = orc.make_rotation(d, seed)
        if mse:
            c = orc.lloyd_max(d, b)[0].astype(np.float32)
            _cache[key] = (tq.tq_ctx_create_mse(d, b, pi32, c), (d, b, pi32, None, c))
        else:
            c = orc.lloyd_max(d, b - 1)[0].astype(np.float32)
            _cache[key] = (tq.TqContext(d, b, pi32, s32, c), (d, b, pi32, s32, c))
    return _cache[key]


def pair(orc, dh, bh, dl, bl, mse):
    hi, ohi = instance(orc, dh, bh, 100 + dh, mse)
    lo, olo = instance(orc, dl, bl, 200 + dl, mse)
    return hi, ohi, lo, olo


def to_dev(rec):
    return (torch.as_tensor(rec["planes"].view(np.int32), device=DEV),
            torch.as_tensor(rec["norms"].view(np.int16), device=DEV))


def np_rec(P, N):
    return P.cpu().numpy().view(np.uint32), N.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("dh,bh,dl,bl,mse,dtype,n_heads,n_tok", [
    (64, 3, 64, 2, False, torch.bfloat16, 3, 70),     # 2.5 bits at d = 128
    (64, 4, 64, 3, False, torch.float32, 2, 130),     # 3.5 bits
    (32, 2, 96, 3, False, torch.float32, 2, 33),      # narrower first group, lower width
    (64, 2, 64, 1, True, torch.bfloat16, 2, 65),      # MSE-only records
])
def test_split_quantize_parity(orc, dh, bh, dl, bl, mse, dtype, n_heads, n_tok):
    say("split quantize", dh, bh, dl, bl, mse, dtype, n_heads, n_tok)
    hi, ohi, lo, olo = pair(orc, dh, bh, dl, bl, mse)
    x = (workloads.normal((n_heads, n_tok, dh + dl), 31, 10, DEV) * 1.5).to(dtype)
    n = n_heads * n_tok
    hp, hn = tq.alloc_records(n, dh, bh)
    lp, ln = tq.alloc_records(n, dl, bl)
    tq.tq_split_quantize_kv(hi, lo, x, hp, hn, lp, ln)
    torch.cuda.synchronize()
    xd = x.reshape(n, dh + dl).double().cpu()
    if mse:
        xn = xd.numpy()
        check_records_mse(orc, dh, bh, ohi[2], ohi[4], xn[:, :dh], *np_rec(hp, hn))
        check_records_mse(orc, dl, bl, olo[2], olo[4], xn[:, dh:], *np_rec(lp, ln))
    else:
        check_quantize(orc, dh, bh, xd[:, :dh], *ohi[2:], *np_rec(hp, hn))
        check_quantize(orc, dl, bl, xd[:, dh:], *olo[2:], *np_rec(lp, ln))


def test_split_dequantize_parity(orc):
    dh, bh, dl, bl = 64, 4, 64, 3
    hi, ohi, lo, olo = pair(orc, dh, bh, dl, bl, False)
    x = workloads.normal((300, dh + dl), 32, 10, "cpu").double().numpy()
    rh, rl = orc.split_quantize(ohi, olo, x)
    out = torch.full((300, dh + dl + 8), float("nan"), device=DEV)
    tq.tq_split_dequantize(hi, lo, *to_dev(rh), *to_dev(rl), 300, out)
    torch.cuda.synchronize()
    ref = orc.split_dequantize(ohi, olo, (rh["planes"], rh["norms"]), (rl["planes"], rl["norms"]))
    got = out.cpu().numpy()
    assert rel_err_rows(got[:, :dh + dl], ref) < TOL
    assert np.all(np.isnan(got[:, dh + dl:]))


def split_records(orc, ohi, olo, n_kv, total, seed):
    x = workloads.normal((n_kv, total, ohi[0] + olo[0]), seed, 10, "cpu").double().numpy()
    x[:, :, :ohi[0]] *= 2.0                 # a louder first group
    rh, rl = zip(*[orc.split_quantize(ohi, olo, x[h]) for h in range(n_kv)])
    cat = lambda rs, k: np.concatenate([r[k] for r in rs])   # noqa: E731
    return (cat(rh, "planes"), cat(rh, "norms")), (cat(rl, "planes"), cat(rl, "norms"))


@pytest.mark.parametrize("dh,bh,dl,bl,mse,n_q,n_kv,lens", [
    (64, 3, 64, 2, False, 32, 8, [1000, 37, 513]),    # 2.5 bits, GQA 4, ragged batch
    (64, 4, 64, 3, False, 8, 2, [777]),               # 3.5 bits
    (32, 2, 96, 3, False, 4, 2, [300, 1]),            # lower width first (swapped sets), G = 2
    (128, 4, 128, 3, False, 3, 1, [129]),             # d = 256, G = 3
    (64, 2, 64, 1, True, 8, 8, [400, 65]),            # MSE-only, G = 1
    (64, 3, 64, 3, False, 16, 4, [250]),              # equal widths
])
def test_split_logits_parity(orc, dh, bh, dl, bl, mse, n_q, n_kv, lens):
    say("split logits", dh, bh, dl, bl, mse, n_q, n_kv, lens)
    hi, ohi, lo, olo = pair(orc, dh, bh, dl, bl, mse)
    total = sum(lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).tolist()
    (hp, hn), (lp, ln) = split_records(orc, ohi, olo, n_kv, total, 33)
    batch, d = len(lens), dh + dl
    q = workloads.normal((batch, n_q, d), 33, 12, "cpu").numpy()
    scale = 1.0 / np.sqrt(d)
    ss = torch.as_tensor(starts, dtype=torch.int64, device=DEV)
    sl = torch.as_tensor(lens, dtype=torch.int32, device=DEV)
    logits = torch.full((n_q, total + 5), float("nan"), device=DEV)
    ws = tq.workspace(tq.tq_split_attn_logits_workspace_bytes(hi, lo, batch, n_q, n_kv))
    HP, HN = to_dev({"planes": hp, "norms": hn})
    LP, LN = to_dev({"planes": lp, "norms": ln})
    tq.tq_split_attn_logits(hi, lo, torch.as_tensor(q, device=DEV), batch, n_q, n_q * d, HP, HN,
                            LP, LN, n_kv, total, ss, sl, max(lens), scale, logits, total + 5, ws)
    torch.cuda.synchronize()
    got = logits.cpu().numpy()
    G = n_q // n_kv
    for bi, (st, ln_) in enumerate(zip(starts, lens)):
        for h in range(n_kv):
            r = slice(h * total + st, h * total + st + ln_)
            ref = orc.split_estimate(ohi, olo, q[bi, h * G:(h + 1) * G].astype(np.float64),
                                     (hp[r], hn[r]), (lp[r], ln[r]), scale=scale)
            g = got[h * G:(h + 1) * G, st:st + ln_]
            assert rel_err_rows(g, ref) < TOL, (bi, h, rel_err_rows(g, ref))
    assert np.all(np.isnan(got[:, total:]))


def test_split_prepared_queries_match_one_call(orc):
    """tq_split_attn_prepare + tq_split_attn_logits_prepared ==
    tq_split_attn_logits, bit for bit."""
    hi, ohi, lo, olo = pair(orc, 64, 4, 64, 3, False)
    total, n_q, n_kv = 1050, 8, 2
    HP, HN = workloads.random_records(n_kv * total, tq.tq_record_words(64, 4), 6, DEV)
    LP, LN = workloads.random_records(n_kv * total, tq.tq_record_words(64, 3), 7, DEV)
    q = workloads.normal((2, n_q, 128), 36, 12, DEV)
    ss = torch.tensor([0, 600], dtype=torch.int64, device=DEV)
    sl = torch.tensor([600, 450], dtype=torch.int32, device=DEV)
    ws = tq.workspace(tq.tq_split_attn_logits_workspace_bytes(hi, lo, 2, n_q, n_kv))
    one = torch.full((n_q, total + 5), float("nan"), device=DEV)
    two = one.clone()
    tq.tq_split_attn_logits(hi, lo, q, 2, n_q, n_q * 128, HP, HN, LP, LN, n_kv, total, ss, sl,
                            600, 0.3, one, total + 5, ws)
    ws2 = tq.workspace(tq.tq_split_attn_logits_workspace_bytes(hi, lo, 2, n_q, n_kv))
    tq.tq_split_attn_prepare(hi, lo, q, 2, n_q, n_q * 128, n_kv, ws2)
    tq.tq_split_attn_logits_prepared(hi, lo, ws2, 2, n_q, HP, HN, LP, LN, n_kv, total, ss, sl,
                                     600, 0.3, two, total + 5)
    torch.cuda.synchronize()
    assert torch.equal(one.nan_to_num(7.0), two.nan_to_num(7.0))
    with pytest.raises(tq.TqError):           # workspace too small
        tq.tq_split_attn_prepare(hi, lo, q, 2, n_q, n_q * 128, n_kv, ws2[:64])


def test_split_logits_unsupported_and_bad_arguments(orc):
    hi, ohi, lo, olo = pair(orc, 64, 3, 64, 2, False)
    mhi, _ = instance(orc, 64, 2, 7, True)
    big, _ = instance(orc, 200, 3, 8, False)
    P, N = workloads.random_records(16, 8, 3, DEV)
    q = torch.zeros((1, 8, 128), device=DEV)
    ss = torch.zeros(1, dtype=torch.int64, device=DEV)
    sl = torch.full((1,), 16, dtype=torch.int32, device=DEV)
    out = torch.empty((8, 16), device=DEV)
    ws = tq.workspace(1 << 20)
    with pytest.raises(tq.TqError) as e:      # 8 query heads per kv head
        tq.tq_split_attn_logits(hi, lo, q, 1, 8, 8 * 128, P, N, P, N, 1, 16, ss, sl, 16, 1.0,
                                out, 16, ws)
    assert e.value.status == tq.TQ_ERR_UNSUPPORTED
    with pytest.raises(tq.TqError) as e:      # a group wider than 128 channels
        tq.tq_split_attn_logits(big, lo, q, 1, 8, 8 * 264, P, N, P, N, 2, 16, ss, sl, 16, 1.0,
                                out, 16, ws)
    assert e.value.status == tq.TQ_ERR_UNSUPPORTED
    with pytest.raises(tq.TqError) as e:      # two-stage and MSE-only instances mixed
        tq.tq_split_attn_logits(hi, mhi, q, 1, 8, 8 * 128, P, N, P, N, 2, 16, ss, sl, 16, 1.0,
                                out, 16, ws)
    assert e.value.status == tq.TQ_ERR_INVALID_ARG
    with pytest.raises(tq.TqError):           # workspace too small
        tq.tq_split_attn_logits(hi, lo, q, 1, 8, 8 * 128, P, N, P, N, 2, 16, ss, sl, 16, 1.0,
                                out, 16, ws[:16])
    x = torch.zeros((2, 4, 128), device=DEV)
    with pytest.raises(tq.TqError):           # rows narrower than d_hi + d_lo
        tq.tq_split_quantize_kv(hi, lo, x, P, N, P, N, x_stride_token=120)


@pytest.mark.parametrize("dh,bh,dl,bl,mse,n_q,n_kv,lens", [
    (64, 3, 64, 2, False, 32, 8, [1000, 37, 513]),
    (32, 4, 96, 2, False, 16, 4, [257, 600]),
    (64, 2, 64, 1, True, 8, 2, [300, 1]),
])
def test_split_attn_output_parity(orc, dh, bh, dl, bl, mse, n_q, n_kv, lens):
    say("split attn output", dh, bh, dl, bl, mse, n_q, n_kv, lens)
    hi, ohi, lo, olo = pair(orc, dh, bh, dl, bl, mse)
    total = sum(lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).tolist()
    (hp, hn), (lp, ln) = split_records(orc, ohi, olo, n_kv, total, 34)
    batch, d = len(lens), dh + dl
    p = np.random.default_rng(35).random((n_q, total)).astype(np.float32)
    ss = torch.as_tensor(starts, dtype=torch.int64, device=DEV)
    sl = torch.as_tensor(lens, dtype=torch.int32, device=DEV)
    out = torch.full((batch, n_q, d), float("nan"), device=DEV)
    mx = max(lens)
    ws = tq.workspace(tq.tq_split_attn_output_workspace_bytes(hi, lo, batch, n_q, n_kv, mx))
    HP, HN = to_dev({"planes": hp, "norms": hn})
    LP, LN = to_dev({"planes": lp, "norms": ln})
    tq.tq_split_attn_output(hi, lo, torch.as_tensor(p, device=DEV), total, batch, n_q, HP, HN,
                            LP, LN, n_kv, total, ss, sl, mx, out, n_q * d, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    G = n_q // n_kv
    deq = [orc.split_dequantize(ohi, olo, (hp[h * total:(h + 1) * total], hn[h * total:(h + 1) * total]),
                                (lp[h * total:(h + 1) * total], ln[h * total:(h + 1) * total]))
           for h in range(n_kv)]
    for bi, (st, ln_) in enumerate(zip(starts, lens)):
        for hq in range(n_q):
            ref = p[hq, st:st + ln_].astype(np.float64) @ deq[hq // G][st:st + ln_]
            assert rel_err_rows(got[bi, hq][None], ref[None]) < TOL, (bi, hq)
