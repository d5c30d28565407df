"""GPU parity of the slot-mapped appends (tq_quantize_kv_slots and
tq_decode_step_prepare with dst_slots): a token's record must be bit-identical
to what tq_quantize_kv writes for it, land at its slot, and the valid records
must match the oracle; records of skipped slots and untouched records keep
their previous contents.  All inputs are seeded.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_vector_pi_amd as tq  # noqa: E402
import workloads  # noqa: E402
from helpers import oracle_tables  # noqa: E402
from test_gpu_parity import check_quantize  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"
FILL_P, FILL_N = 0x5A5A5A5A, 0x3C3C


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def make_ctx(orc, d, b, mse):
    if mse:
        pi = orc.make_rotation(d, 0)[2]
        c = orc.lloyd_max(d, b)[0].astype(np.float32)
        return tq.tq_ctx_create_mse(d, b, pi, c), pi, None, c
    pi, s, c = oracle_tables(orc, d, b, 0)
    return tq.TqContext(d, b, pi, s, c), pi, s, c


def make_slots(n_tok, cap, seed):
    """Distinct destinations in [0, cap) for most tokens; a few are skipped
    (negative, or cap and beyond)."""
    rng = np.random.default_rng(seed)
    slots = rng.permutation(cap)[:n_tok].astype(np.int64)
    if n_tok >= 4:
        slots[1] = -1
        slots[n_tok // 2] = cap
        slots[-1] = cap + 1000
    return slots


def filled(n, d, b):
    p, nn = tq.alloc_records(n, d, b)
    p.fill_(FILL_P)
    nn.fill_(FILL_N)
    return p, nn


def expected_scatter(dense_p, dense_n, slots, n_heads, n_tok, cap, d, b):
    """Records of tq_quantize_kv (dense [n_heads * n_tok]) moved to their slots
    in a [n_heads * cap] buffer filled with the fill patterns."""
    ep, en = filled(n_heads * cap, d, b)
    ep, en = ep.cpu(), en.cpu()
    dp, dn = dense_p.cpu(), dense_n.cpu()
    for t, s in enumerate(slots):
        if 0 <= s < cap:
            for h in range(n_heads):
                ep[h * cap + s] = dp[h * n_tok + t]
                en[h * cap + s] = dn[h * n_tok + t]
    return ep, en


@pytest.mark.parametrize("d,b,mse,dtype,n_heads,n_tok", [
    (128, 4, False, torch.bfloat16, 3, 300),   # tiles across heads, ragged tail
    (128, 3, True, torch.float32, 40, 1),      # one token per head (decoding)
    (128, 2, False, torch.float32, 2, 64),     # whole tiles inside one head
    (200, 2, False, torch.float32, 2, 70),     # other d (padded groups)
    (64, 2, True, torch.bfloat16, 5, 33),
])
def test_quantize_slots(orc, d, b, mse, dtype, n_heads, n_tok):
    say("quantize slots", d, b, mse, dtype, n_heads, n_tok)
    ctx, pi, s, c = make_ctx(orc, d, b, mse)
    x = (workloads.normal((n_heads, n_tok, d), 21, 10, DEV) * 1.3).to(dtype)
    cap = 2 * n_tok + 7
    slots = make_slots(n_tok, cap, 5 + n_tok)
    sl = torch.from_numpy(slots).to(DEV)
    P, N = filled(n_heads * cap, d, b)
    tq.tq_quantize_kv_slots(ctx, x, sl, P, N, cap)
    dp, dn = tq.alloc_records(n_heads * n_tok, d, b)
    tq.tq_quantize_kv(ctx, x, dp, dn)
    torch.cuda.synchronize()
    ep, en = expected_scatter(dp, dn, slots, n_heads, n_tok, cap, d, b)
    assert torch.equal(P.cpu(), ep) and torch.equal(N.cpu(), en)
    if not mse:
        # the records at the slots against the oracle
        ok = [(h, t) for h in range(n_heads) for t in range(n_tok) if 0 <= slots[t] < cap]
        rows = [h * cap + slots[t] for h, t in ok]
        xs = torch.stack([x[h, t] for h, t in ok]).float()
        check_quantize(orc, d, b, xs, pi, s, c, P.cpu().numpy().view(np.uint32)[rows],
                       N.cpu().numpy().view(np.uint16)[rows])


def test_quantize_slots_rerun_and_empty(orc):
    """A second call into the same cache overwrites only its own slots;
    n_tokens == 0 writes nothing."""
    d, b = 128, 3
    ctx, pi, s, c = make_ctx(orc, d, b, False)
    n_heads, cap = 4, 96
    x1 = workloads.normal((n_heads, 64, d), 22, 10, DEV)
    x2 = workloads.normal((n_heads, 16, d), 22, 11, DEV)
    s1 = torch.arange(0, 64, dtype=torch.int64, device=DEV)
    s2 = torch.arange(64, 80, dtype=torch.int64, device=DEV)
    P, N = filled(n_heads * cap, d, b)
    tq.tq_quantize_kv_slots(ctx, x1, s1, P, N, cap)
    tq.tq_quantize_kv_slots(ctx, x2, s2, P, N, cap)
    tq.tq_quantize_kv_slots(ctx, x2[:, :0], s2[:0], P, N, cap)
    rp, rn = filled(n_heads * cap, d, b)
    tq.tq_quantize_kv(ctx, x1, rp, rn, dst_stride_head=cap, dst_token0=0)
    tq.tq_quantize_kv(ctx, x2, rp, rn, dst_stride_head=cap, dst_token0=64)
    torch.cuda.synchronize()
    assert torch.equal(P, rp) and torch.equal(N, rn)


def test_quantize_slots_rejects_bad_arguments(orc):
    d, b = 128, 4
    ctx, pi, s, c = make_ctx(orc, d, b, False)
    x = torch.zeros((2, 4, d), dtype=torch.bfloat16, device=DEV)
    P, N = filled(2 * 8, d, b)
    sl = torch.arange(4, dtype=torch.int64, device=DEV)
    with pytest.raises(tq.TqError):          # NULL slots
        tq.tq_quantize_kv_slots(ctx, x, None, P, N, 8)
    with pytest.raises(tq.TqError):          # empty slot range
        tq.tq_quantize_kv_slots(ctx, x, sl, P, N, 0)
    L = tq.lib()
    raw = torch.zeros(5, dtype=torch.int64, device=DEV)
    st = L.tq_quantize_kv_slots(ctx.handle, x.data_ptr(), tq.TQ_BF16, 4, 2, d, 4 * d,
                                raw.data_ptr() + 4, P.data_ptr(), N.data_ptr(), 8, None)
    assert st == tq.TQ_ERR_INVALID_ARG       # slots not 8-byte aligned
    q = torch.zeros((1, 8, d), device=DEV)
    ws = tq.workspace(tq.tq_attn_logits_workspace_bytes(ctx, 1, 8, 2))
    with pytest.raises(tq.TqError):          # slots with a nonzero dst_token0
        tq.tq_decode_step_prepare(ctx, x, x, P, N, P, N, q, 1, 8, 8 * d, 2, ws,
                                  dst_stride_head=8, dst_token0=1, dst_slots=sl)
    torch.cuda.synchronize()
    assert bool((P == FILL_P).all()) and bool((N == FILL_N).all())


@pytest.mark.parametrize("d,b,mse,dtype,n_heads,n_tok,L,n_q,n_kv", [
    (128, 4, False, torch.bfloat16, 256, 16, 32, 32, 8),   # 16 sequences x one token
    (128, 2, True, torch.bfloat16, 24, 3, 3, 8, 8),
    (200, 4, False, torch.float32, 5, 9, 2, 8, 2),          # other d: separate launches
])
def test_decode_step_prepare_slots(orc, d, b, mse, dtype, n_heads, n_tok, L, n_q, n_kv):
    """tq_decode_step_prepare with dst_slots == tq_quantize_kv_slots (K, V)
    and tq_attn_prepare, bit for bit."""
    say("decode step prepare slots", d, b, mse, dtype, n_heads, n_tok)
    ctx, pi, s, c = make_ctx(orc, d, b, mse)
    kx = (workloads.normal((n_heads, n_tok, d), 23, 10, DEV) * 1.7).to(dtype)
    vx = (workloads.normal((n_heads, n_tok, d), 23, 11, DEV) * 0.6).to(dtype)
    q = workloads.normal((L, n_q, d), 23, 12, DEV)
    cap = 3 * n_tok + 2
    slots = torch.from_numpy(make_slots(n_tok, cap, 40 + n_tok)).to(DEV)
    bufs = [filled(n_heads * cap, d, b) for _ in range(4)]
    ws_bytes = tq.tq_attn_logits_workspace_bytes(ctx, L, n_q, n_kv)
    ws1, ws2 = tq.workspace(ws_bytes), tq.workspace(ws_bytes)
    ws1.zero_()
    ws2.zero_()
    tq.tq_decode_step_prepare(ctx, kx, vx, *bufs[0], *bufs[1], q, L, n_q, n_q * d, n_kv, ws1,
                              dst_stride_head=cap, dst_slots=slots)
    tq.tq_quantize_kv_slots(ctx, kx, slots, *bufs[2], cap)
    tq.tq_quantize_kv_slots(ctx, vx, slots, *bufs[3], cap)
    tq.tq_attn_prepare(ctx, q, L, n_q, n_q * d, n_kv, ws2)
    torch.cuda.synchronize()
    for x_, y_ in zip(bufs[0] + bufs[1], bufs[2] + bufs[3]):
        assert torch.equal(x_, y_)
    assert torch.equal(ws1, ws2)
