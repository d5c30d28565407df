"""GPU parity at the workloads' full sizes, through the same entry points and
launch configuration that bench.py times, checked on sampled outputs the
oracle computes one by one:

  * Llama-3.1-8B-shaped decode (8 KV / 32 q heads, d = 128, 32768 tokens,
    b = 4, outlier channels) over 32 layer caches laid out [kv][layer][token]:
    the cache fill, the new-token quantize into the caches, the prepared
    queries and one logit launch over all layers;
  * batched decode: 16 ragged sequences (4096..8192 tokens), b = 3, prefix and
    512-token chunk quantized per sequence, one logit launch; the chunks also
    as one slot-mapped call;
  * fractional widths (channels 0..63 at 3 or 4 bits, 64..127 at 2 or 3) over
    the 32 Llama-shaped layer caches;
  * long context: 8 KV heads x 131072 tokens, b in {2, 3, 4};
  * vector search: 1e6 unit vectors at d = 1536 and 200, b in {2, 4}, top-10
    of 1000 queries (the oracle ranks a subset of queries over the whole
    database from the GPU's records).

Records: sampled rows against the oracle's quantization of the same inputs.
Logits and scores: whole rows of the oracle's estimator on the GPU's records
(staged parity), 1e-3 of max(|ref|, row rms).
"""
import math
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_vector_pi_amd as tq  # noqa: E402
import workloads  # noqa: E402
from helpers import TOL, check_records, oracle_tables, rel_err_rows, topk_order_ok  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def make_ctx(orc, d, b):
    pi, s, c = oracle_tables(orc, d, b)
    return tq.TqContext(d, b, pi, s, c), pi, s, c


def np_records(planes, norms, rows):
    idx = torch.as_tensor(rows, device=planes.device)
    return (planes[idx].cpu().numpy().view(np.uint32), norms[idx].cpu().numpy().view(np.uint16))


def test_llama_decode_32_layers(orc):
    d, b, n_kv, n_q, n_tok, L = 128, 4, 8, 32, 32768, 32
    say("llama decode", L, "layers")
    ctx, pi, s, c = make_ctx(orc, d, b)
    rw = tq.tq_record_words(d, b)
    n_rec = n_kv * L * n_tok
    kp = torch.zeros((n_rec, rw), dtype=torch.int32, device=DEV)
    kn = torch.zeros((n_rec, 2), dtype=torch.int16, device=DEV)
    Kx = torch.empty((n_kv, L * n_tok, d), dtype=torch.bfloat16, device=DEV)
    for l in range(L):
        Kx[:, l * n_tok:(l + 1) * n_tok] = workloads.llama(DEV, seed=l, n_tok=n_tok)["K"]
    q_all = torch.stack([workloads.normal((n_q, d), l, workloads.STREAM_Q, DEV) for l in range(L)])
    # cache fill (one call over all layers), sampled records
    tq.tq_quantize_kv(ctx, Kx, kp, kn)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = rng.choice(n_rec, 1536, replace=False)
    x = Kx.view(-1, d)[torch.as_tensor(rows, device=DEV)].double().cpu().numpy()
    P, N = np_records(kp, kn, rows)
    check_records(orc, d, b, pi, s, c, x, P, N)
    # new token of every (kv head, layer) at position n_tok - 1, written over
    # the cache records by the strided call bench.py makes
    newK = workloads.normal((n_kv * L, 1, d), 99, workloads.STREAM_K, DEV).to(torch.bfloat16)
    tq.tq_quantize_kv(ctx, newK, kp, kn, dst_stride_head=n_tok, dst_token0=n_tok - 1)
    torch.cuda.synchronize()
    rows_new = np.arange(n_kv * L) * n_tok + n_tok - 1
    P, N = np_records(kp, kn, rows_new)
    check_records(orc, d, b, pi, s, c, newK.view(-1, d).double().cpu().numpy(), P, N)
    # neighbours of the new token are untouched
    before = np_records(kp, kn, rows_new - 1)
    assert before[0].any()
    # prepared queries + one logit launch over all 32 layers
    ws = tq.workspace(tq.tq_attn_logits_workspace_bytes(ctx, L, n_q, n_kv), DEV)
    seq_start = torch.arange(L, dtype=torch.int64, device=DEV) * n_tok
    seq_len = torch.full((L,), n_tok, dtype=torch.int32, device=DEV)
    logits = torch.empty((n_q, L * n_tok), dtype=torch.float32, device=DEV)
    scale = 1.0 / math.sqrt(d)
    tq.tq_attn_prepare(ctx, q_all, L, n_q, n_q * d, n_kv, ws)
    tq.tq_attn_logits_prepared(ctx, ws, L, n_q, kp, kn, n_kv, L * n_tok, seq_start, seq_len,
                               n_tok, scale, logits, L * n_tok)
    torch.cuda.synchronize()
    for (l, hq) in [(0, 0), (5, 13), (17, 31), (31, 6)]:
        h = hq // (n_q // n_kv)
        base = (h * L + l) * n_tok
        P, N = np_records(kp, kn, np.arange(base, base + n_tok))
        ref = orc.estimate(d, b, pi, s, c, q_all[l, hq:hq + 1].double().cpu().numpy(), P, N,
                           scale=scale)
        got = logits[hq, l * n_tok:(l + 1) * n_tok].cpu().numpy()[None]
        assert rel_err_rows(got, ref) < TOL, (l, hq, rel_err_rows(got, ref))
    ctx.close()


def test_batched_ragged_decode(orc):
    d, b = 128, 3
    say("batched decode")
    ctx, pi, s, c = make_ctx(orc, d, b)
    wl = workloads.batched(DEV)
    lens, chunk, n_kv, n_q = wl["lens"], wl["chunk"], wl["n_kv"], wl["n_q"]
    batch, total = len(lens), sum(lens)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    rw = tq.tq_record_words(d, b)
    kp = torch.zeros((n_kv * total, rw), dtype=torch.int32, device=DEV)
    kn = torch.zeros((n_kv * total, 2), dtype=torch.int16, device=DEV)
    K = wl["K"]
    for i in range(batch):
        a, n = int(offs[i]), lens[i] - chunk
        tq.tq_quantize_kv(ctx, K[:, a:a + n], kp, kn, dst_stride_head=total, dst_token0=a)
        tq.tq_quantize_kv(ctx, K[:, a + n:a + n + chunk], kp, kn, dst_stride_head=total,
                          dst_token0=a + n)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    rows = rng.choice(n_kv * total, 1024, replace=False)
    x = K.reshape(-1, d)[torch.as_tensor(rows, device=DEV)].double().cpu().numpy()
    P, N = np_records(kp, kn, rows)
    check_records(orc, d, b, pi, s, c, x, P, N)
    ss = torch.as_tensor(offs, device=DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    logits = torch.full((n_q, total), float("nan"), device=DEV)
    ws = tq.workspace(tq.tq_attn_logits_workspace_bytes(ctx, batch, n_q, n_kv), DEV)
    tq.tq_attn_logits(ctx, wl["q"], batch, n_q, n_q * d, kp, kn, n_kv, total, ss, sl, max(lens),
                      1.0 / math.sqrt(d), logits, total, ws)
    torch.cuda.synchronize()
    assert not torch.isnan(logits).any()
    for (bi, hq) in [(0, 0), (7, 21), (15, 31)]:
        h = hq // (n_q // n_kv)
        a = int(offs[bi])
        P, N = np_records(kp, kn, np.arange(h * total + a, h * total + a + lens[bi]))
        ref = orc.estimate(d, b, pi, s, c, wl["q"][bi, hq:hq + 1].double().cpu().numpy(), P, N,
                           scale=1.0 / math.sqrt(d))
        got = logits[hq, a:a + lens[bi]].cpu().numpy()[None]
        assert rel_err_rows(got, ref) < TOL, (bi, hq, rel_err_rows(got, ref))
    ctx.close()


def test_batched_chunks_slot_mapped(orc):
    """The batched workload's chunk appends as bench.py times them: the 16
    sequences' 512-token chunks gathered into one input and written by one
    tq_quantize_kv_slots call, and per sequence with tq_quantize_kv (512
    tokens: the pipelined bf16 kernel, while slot maps run the tiled one).
    Both write exactly the chunk records; sampled records of each match the
    oracle, and the two caches differ only in the few records with a
    decision inside the oracle's margins or a norm one ulp apart."""
    d, b = 128, 3
    say("batched chunks, slot-mapped")
    ctx, pi, s, c = make_ctx(orc, d, b)
    wl = workloads.batched(DEV)
    lens, chunk, n_kv = wl["lens"], wl["chunk"], wl["n_kv"]
    total = sum(lens)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    rw = tq.tq_record_words(d, b)
    kp = torch.zeros((n_kv * total, rw), dtype=torch.int32, device=DEV)
    kn = torch.zeros((n_kv * total, 2), dtype=torch.int16, device=DEV)
    ref_p, ref_n = torch.zeros_like(kp), torch.zeros_like(kn)
    K = wl["K"]
    for i in range(len(lens)):
        a = int(offs[i]) + lens[i] - chunk
        tq.tq_quantize_kv(ctx, K[:, a:a + chunk], ref_p, ref_n, dst_stride_head=total,
                          dst_token0=a)
    idx = torch.cat([torch.arange(int(o) + n - chunk, int(o) + n) for o, n in zip(offs, lens)])
    idx = idx.to(DEV)
    Kn = K[:, idx].contiguous()
    tq.tq_quantize_kv_slots(ctx, Kn, idx, kp, kn, total)
    torch.cuda.synchronize()
    written = kn.view(torch.int32).ne(0)
    assert torch.equal(written, ref_n.view(torch.int32).ne(0))
    assert int(written.sum()) == n_kv * idx.numel()
    differ = (kp != ref_p).any(dim=1) | (kn != ref_n).any(dim=1)
    assert float(differ.float().mean()) < 0.05 * idx.numel() * n_kv / kp.shape[0]
    rng = np.random.default_rng(4)
    pick = rng.choice(n_kv * idx.numel(), 1024, replace=False)
    h, t = pick // idx.numel(), pick % idx.numel()
    rows = h * total + idx.cpu().numpy()[t]
    x = Kn[torch.as_tensor(h, device=DEV), torch.as_tensor(t, device=DEV)].double().cpu().numpy()
    check_records(orc, d, b, pi, s, c, x, *np_records(kp, kn, rows))
    check_records(orc, d, b, pi, s, c, x, *np_records(ref_p, ref_n, rows))
    ctx.close()


@pytest.mark.parametrize("bh,bl", [(3, 2), (4, 3)])
def test_llama_split_32_layers(orc, bh, bl):
    """Fractional widths as bench.py --workload split runs them: channels
    0..63 at bh bits and 64..127 at bl over the 32 Llama-shaped layer caches;
    sampled record pairs against the oracle's split quantization, and whole
    logit rows of one prepared launch over all layers against its split
    estimate."""
    d, dh, n_kv, n_q, n_tok, L = 128, 64, 8, 32, 32768, 32
    say("llama split", bh, bl)
    insts = []
    for bb, seed in ((bh, 1), (bl, 2)):
        pi64, s64, pi32, s32 = orc.make_rotation(dh, seed)
        cen = orc.lloyd_max(dh, bb - 1)[0].astype(np.float32)
        insts.append((tq.TqContext(dh, bb, pi32, s32, cen), (dh, bb, pi32, s32, cen)))
    (hi, ohi), (lo, olo) = insts
    n_rec = n_kv * L * n_tok
    hp = torch.zeros((n_rec, tq.tq_record_words(dh, bh)), dtype=torch.int32, device=DEV)
    lp = torch.zeros((n_rec, tq.tq_record_words(dh, bl)), dtype=torch.int32, device=DEV)
    hn = torch.zeros((n_rec, 2), dtype=torch.int16, device=DEV)
    ln = torch.zeros_like(hn)
    Kx = torch.empty((n_kv, L * n_tok, d), dtype=torch.bfloat16, device=DEV)
    for l in range(L):
        Kx[:, l * n_tok:(l + 1) * n_tok] = workloads.llama(DEV, seed=l, n_tok=n_tok)["K"]
    q_all = torch.stack([workloads.normal((n_q, d), l, workloads.STREAM_Q, DEV) for l in range(L)])
    tq.tq_split_quantize_kv(hi, lo, Kx, hp, hn, lp, ln)
    torch.cuda.synchronize()
    rows = np.random.default_rng(5).choice(n_rec, 1024, replace=False)
    x = Kx.view(-1, d)[torch.as_tensor(rows, device=DEV)].double().cpu().numpy()
    check_records(orc, dh, bh, *ohi[2:], x[:, :dh], *np_records(hp, hn, rows))
    check_records(orc, dh, bl, *olo[2:], x[:, dh:], *np_records(lp, ln, rows))
    ws = tq.workspace(tq.tq_split_attn_logits_workspace_bytes(hi, lo, L, n_q, n_kv), DEV)
    seq_start = torch.arange(L, dtype=torch.int64, device=DEV) * n_tok
    seq_len = torch.full((L,), n_tok, dtype=torch.int32, device=DEV)
    logits = torch.empty((n_q, L * n_tok), dtype=torch.float32, device=DEV)
    scale = 1.0 / math.sqrt(d)
    tq.tq_split_attn_prepare(hi, lo, q_all, L, n_q, n_q * d, n_kv, ws)
    tq.tq_split_attn_logits_prepared(hi, lo, ws, L, n_q, hp, hn, lp, ln, n_kv, L * n_tok,
                                     seq_start, seq_len, n_tok, scale, logits, L * n_tok)
    torch.cuda.synchronize()
    for (l, hq) in [(0, 0), (9, 14), (31, 31)]:
        h = hq // (n_q // n_kv)
        r = np.arange((h * L + l) * n_tok, (h * L + l + 1) * n_tok)
        ref = orc.split_estimate(ohi, olo, q_all[l, hq:hq + 1].double().cpu().numpy(),
                                 np_records(hp, hn, r), np_records(lp, ln, r), scale=scale)
        got = logits[hq, l * n_tok:(l + 1) * n_tok].cpu().numpy()[None]
        assert rel_err_rows(got, ref) < TOL, (l, hq, rel_err_rows(got, ref))
    hi.close()
    lo.close()


@pytest.mark.parametrize("b", [2, 3, 4])
def test_long_context(orc, b):
    d, n_kv, n_q, n_tok = 128, 8, 32, 131072
    say("long context", b)
    ctx, pi, s, c = make_ctx(orc, d, b)
    wl = workloads.long_context(DEV)
    rw = tq.tq_record_words(d, b)
    kp = torch.zeros((n_kv * n_tok, rw), dtype=torch.int32, device=DEV)
    kn = torch.zeros((n_kv * n_tok, 2), dtype=torch.int16, device=DEV)
    tq.tq_quantize_kv(ctx, wl["K"], kp, kn)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3 + b)
    rows = rng.choice(n_kv * n_tok, 1024, replace=False)
    x = wl["K"].reshape(-1, d)[torch.as_tensor(rows, device=DEV)].double().cpu().numpy()
    P, N = np_records(kp, kn, rows)
    check_records(orc, d, b, pi, s, c, x, P, N)
    ss = torch.zeros(1, dtype=torch.int64, device=DEV)
    sl = torch.full((1,), n_tok, dtype=torch.int32, device=DEV)
    logits = torch.empty((n_q, n_tok), device=DEV)
    ws = tq.workspace(tq.tq_attn_logits_workspace_bytes(ctx, 1, n_q, n_kv), DEV)
    tq.tq_attn_logits(ctx, wl["q"], 1, n_q, n_q * d, kp, kn, n_kv, n_tok, ss, sl, n_tok,
                      1.0 / math.sqrt(d), logits, n_tok, ws)
    torch.cuda.synchronize()
    for hq in [3, 30]:
        h = hq // (n_q // n_kv)
        P, N = np_records(kp, kn, np.arange(h * n_tok, (h + 1) * n_tok))
        ref = orc.estimate(d, b, pi, s, c, wl["q"][hq:hq + 1].double().cpu().numpy(), P, N,
                           scale=1.0 / math.sqrt(d))
        got = logits[hq].cpu().numpy()[None]
        assert rel_err_rows(got, ref) < TOL, (hq, rel_err_rows(got, ref))
    ctx.close()


def test_llama_attn_output(orc):
    """Values of the Llama-shaped layer (8 KV heads x 32768 tokens, b = 4,
    outlier channels), weights = softmax of the packed-key logits of a
    seeded query: sampled query heads against the oracle's weighted sum of
    dequantized values."""
    d, b, n_kv, n_q, n_tok = 128, 4, 8, 32, 32768
    say("llama attn output")
    ctx, pi, s, c = make_ctx(orc, d, b)
    wl = workloads.llama(DEV, n_tok=n_tok)
    rw = tq.tq_record_words(d, b)
    kp = torch.zeros((n_kv * n_tok, rw), dtype=torch.int32, device=DEV)
    kn = torch.zeros((n_kv * n_tok, 2), dtype=torch.int16, device=DEV)
    vp, vn = torch.zeros_like(kp), torch.zeros_like(kn)
    tq.tq_quantize_kv(ctx, wl["K"], kp, kn)
    tq.tq_quantize_kv(ctx, wl["V"], vp, vn)
    ss = torch.zeros(1, dtype=torch.int64, device=DEV)
    sl = torch.full((1,), n_tok, dtype=torch.int32, device=DEV)
    logits = torch.empty((n_q, n_tok), device=DEV)
    ws = tq.workspace(tq.tq_attn_logits_workspace_bytes(ctx, 1, n_q, n_kv), DEV)
    tq.tq_attn_logits(ctx, wl["q"], 1, n_q, n_q * d, kp, kn, n_kv, n_tok, ss, sl, n_tok,
                      1.0 / math.sqrt(d), logits, n_tok, ws)
    p = torch.softmax(logits, dim=1).contiguous()
    out = torch.empty((1, n_q, d), device=DEV)
    wo = tq.workspace(tq.tq_attn_output_workspace_bytes(ctx, 1, n_q, n_kv, n_tok), DEV)
    tq.tq_attn_output(ctx, p, n_tok, 1, n_q, vp, vn, n_kv, n_tok, ss, sl, n_tok, out, n_q * d, wo)
    torch.cuda.synchronize()
    pn = p.cpu().numpy().astype(np.float64)
    for hq in [0, 9, 22, 31]:
        h = hq // (n_q // n_kv)
        P, N = np_records(vp, vn, np.arange(h * n_tok, (h + 1) * n_tok))
        deq = orc.dequantize(d, b, pi, s, c, P, N)
        ref = pn[hq] @ deq
        got = out[0, hq].cpu().numpy()
        assert rel_err_rows(got[None], ref[None]) < TOL, (hq, rel_err_rows(got[None], ref[None]))
    ctx.close()


def test_llama_decode_fused(orc):
    """Fused decode attention over the Llama-shaped layer (8 KV heads x 32768
    tokens, b = 4): sampled query heads against softmax(oracle logits) @
    oracle-dequantized values on the GPU's records."""
    d, b, n_kv, n_q, n_tok = 128, 4, 8, 32, 32768
    say("llama fused decode")
    ctx, pi, s, c = make_ctx(orc, d, b)
    wl = workloads.llama(DEV, n_tok=n_tok)
    rw = tq.tq_record_words(d, b)
    kp = torch.zeros((n_kv * n_tok, rw), dtype=torch.int32, device=DEV)
    kn = torch.zeros((n_kv * n_tok, 2), dtype=torch.int16, device=DEV)
    vp, vn = torch.zeros_like(kp), torch.zeros_like(kn)
    tq.tq_quantize_kv(ctx, wl["K"], kp, kn)
    tq.tq_quantize_kv(ctx, wl["V"], vp, vn)
    ss = torch.zeros(1, dtype=torch.int64, device=DEV)
    sl = torch.full((1,), n_tok, dtype=torch.int32, device=DEV)
    out = torch.empty((1, n_q, d), device=DEV)
    ws = tq.workspace(tq.tq_attn_decode_workspace_bytes(ctx, 1, n_q, n_kv, n_tok), DEV)
    scale = 1.0 / math.sqrt(d)
    tq.tq_attn_decode(ctx, wl["q"], 1, n_q, n_q * d, kp, kn, vp, vn, n_kv, n_tok, ss, sl, n_tok,
                      scale, out, n_q * d, ws)
    torch.cuda.synchronize()
    for hq in [0, 13, 31]:
        h = hq // (n_q // n_kv)
        rows = np.arange(h * n_tok, (h + 1) * n_tok)
        KP, KN = np_records(kp, kn, rows)
        VP, VN = np_records(vp, vn, rows)
        lg = orc.estimate(d, b, pi, s, c, wl["q"][hq:hq + 1].double().cpu().numpy(), KP, KN,
                          scale=scale)[0]
        p = np.exp(lg - lg.max())
        p /= p.sum()
        ref = p @ orc.dequantize(d, b, pi, s, c, VP, VN)
        got = out[0, hq].cpu().numpy()
        assert rel_err_rows(got[None], ref[None]) < TOL, (hq, rel_err_rows(got[None], ref[None]))
    ctx.close()


@pytest.mark.parametrize("d,b", [(1536, 2), (1536, 4), (200, 2), (200, 4)])
def test_vector_search_1m(orc, d, b):
    """Top-10 of 1000 queries over 1e6 records as bench.py times it.  Every
    query: each returned (index, score) pair against the oracle's estimate of
    that one record, and the (score desc, index asc) order.  A deterministic
    subset of 20 queries: the whole ranking against the oracle's scores of the
    full database (staged parity on the GPU's records)."""
    k = 10
    say("search 1e6", d, b)
    ctx, pi, s, c = make_ctx(orc, d, b)
    wl = workloads.search(DEV, d)
    db, qs = wl["db"], wl["queries"]
    n_db, n_q = db.shape[0], qs.shape[0]
    planes, norms = tq.alloc_records(n_db, d, b, DEV)
    # as bench.py: the workspace form (blocked products at d = 1536)
    nb = tq.tq_quantize_workspace_bytes(ctx, n_db)
    tq.tq_quantize_kv_ws(ctx, db, planes, norms, tq.workspace(nb, DEV) if nb else None)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    rows = rng.choice(n_db, 256, replace=False)
    P, N = np_records(planes, norms, rows)
    check_records(orc, d, b, pi, s, c, db[torch.as_tensor(rows, device=DEV)].double().cpu().numpy(),
                  P, N)
    oi = torch.empty((n_q, k), dtype=torch.int64, device=DEV)
    osc = torch.empty((n_q, k), dtype=torch.float32, device=DEV)
    ws = tq.workspace(tq.tq_search_workspace_bytes(ctx, n_q, n_db, k), DEV)
    tq.tq_search_topk(ctx, qs, n_q, planes, norms, n_db, k, oi, osc, ws)
    torch.cuda.synchronize()
    gi, gs = oi.cpu().numpy(), osc.cpu().numpy()
    assert np.all((gi >= 0) & (gi < n_db))
    assert all(len(set(r.tolist())) == k for r in gi)
    assert topk_order_ok(gi, gs)
    qd = qs.double().cpu().numpy()
    # every query: the returned pairs against the oracle's scores of those records
    # (a row's rms over the database from a random sample of 4096 records)
    uniq, inv = np.unique(gi, return_inverse=True)
    inv = inv.reshape(gi.shape)
    samp = rng.choice(n_db, 4096, replace=False)
    UP, UN = np_records(planes, norms, np.concatenate([uniq, samp]))
    nu_ = uniq.size
    for a0 in range(0, n_q, 250):
        sc = orc.estimate(d, b, pi, s, c, qd[a0:a0 + 250], UP, UN)
        for a in range(a0, min(a0 + 250, n_q)):
            ref = sc[a - a0, inv[a]]
            rms = np.sqrt(np.mean(sc[a - a0, nu_:] ** 2))
            assert np.all(np.abs(gs[a] - ref) <= TOL * np.maximum(np.abs(ref), rms)), a
    # 20 queries: the ranking over the whole database
    allP = planes.cpu().numpy().view(np.uint32)
    allN = norms.cpu().numpy().view(np.uint16)
    picks = np.linspace(0, n_q - 1, 20).round().astype(int)
    ref = orc.estimate(d, b, pi, s, c, qd[picks], allP, allN)
    del allP, allN
    for j, a in enumerate(picks):
        row = ref[j]
        rms = np.sqrt(np.mean(row ** 2))
        order = np.lexsort((np.arange(row.size), -row))
        kth = row[order[k - 1]]
        for t in range(k):
            idx = gi[a, t]
            assert abs(gs[a, t] - row[idx]) <= TOL * max(abs(row[idx]), rms)
            assert row[idx] >= kth - 2 * TOL * rms
        for idx in order[:k]:
            if row[idx] > kth + 2 * TOL * rms:
                assert idx in gi[a]
    ctx.close()


def test_dequantize_llama_layer(orc):
    """tq_dequantize as bench.py --workload dequant runs it: one Llama-shaped
    layer's keys (262,144 records, d = 128, b = 4) in one call, sampled rows
    against the oracle's dequantization of the same records."""
    d, b = 128, 4
    say("dequantize llama layer")
    ctx, pi, s, c = make_ctx(orc, d, b)
    x = workloads.llama(DEV, seed=0)["K"].reshape(-1, d).contiguous()
    n = x.shape[0]
    planes, norms = tq.alloc_records(n, d, b)
    tq.tq_quantize_kv(ctx, x, planes, norms)
    out = torch.full((n, d), float("nan"), device=DEV)
    tq.tq_dequantize(ctx, planes, norms, n, out)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(64), np.arange(n - 64, n),
                                     np.random.default_rng(7).integers(0, n, 300)]))
    P, N = np_records(planes, norms, rows)
    ref = orc.dequantize(d, b, pi, s, c, P, N)
    got = out[torch.as_tensor(rows, device=DEV)].cpu().numpy()
    assert rel_err_rows(got, ref) < TOL
    assert torch.isfinite(out).all()
