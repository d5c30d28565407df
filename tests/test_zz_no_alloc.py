"""tq_attn_logits_noalloc (the entry point for callers that cannot allocate):
bit-identical to tq_attn_logits with a workspace, on two calls in a row (the
second smaller, so stale scratch contents from the first must not leak), and
a clear error when the prepared queries exceed the static scratch."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_vector_pi_amd as tq  # noqa: E402
import workloads  # noqa: E402
from helpers import TOL, oracle_tables, rel_err_rows  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(ctx, lens, n_q, n_kv, seed):
    d, b = ctx.d, ctx.b
    total = sum(lens)
    P, N = workloads.random_records(n_kv * total, tq.tq_record_words(d, b), seed, DEV)
    q = workloads.normal((len(lens), n_q, d), seed, 12, DEV)
    ss = torch.as_tensor(np.concatenate([[0], np.cumsum(lens)[:-1]]), dtype=torch.int64,
                         device=DEV)
    sl = torch.as_tensor(lens, dtype=torch.int32, device=DEV)
    return P, N, q, ss, sl, total


def _both(ctx, lens, n_q, n_kv, seed, scale):
    P, N, q, ss, sl, total = _case(ctx, lens, n_q, n_kv, seed)
    batch, mx = len(lens), max(lens)
    ref = torch.full((n_q, total), float("nan"), device=DEV)
    ws = tq.workspace(tq.tq_attn_logits_workspace_bytes(ctx, batch, n_q, n_kv))
    tq.tq_attn_logits(ctx, q, batch, n_q, n_q * ctx.d, P, N, n_kv, total, ss, sl, mx, scale,
                      ref, total, ws)
    got = torch.full((n_q, total), float("nan"), device=DEV)
    tq.tq_attn_logits_noalloc(ctx, q, batch, n_q, n_q * ctx.d, P, N, n_kv, total, ss, sl, mx,
                              scale, got, total)
    torch.cuda.synchronize()
    return got, ref, (P, N, q)


# (d, b, q heads per kv head): d = 128 with G = 8 and d = 200 take the two
# launches through the static scratch; d = 64, G = 4 is the one-launch path
@pytest.mark.parametrize("d,b,G", [(128, 4, 8), (200, 3, 4), (64, 3, 4)])
def test_noalloc_matches_workspace_form(orc, d, b, G):
    pi, s, c = oracle_tables(orc, d, b)
    ctx = tq.TqContext(d, b, pi, s, c)
    # first call: 16 sequences x 8 KV heads x G q heads each (2.6 MB of
    # prepared queries at d = 128, G = 8), second call smaller: 3 ragged
    # sequences, 4 KV heads
    g1, r1, _ = _both(ctx, [512] * 16, 8 * G, 8, 41, 0.125)
    assert torch.equal(g1, r1)
    g2, r2, (P, N, q) = _both(ctx, [300, 77, 1000], 4 * G, 4, 42, 0.5)
    assert torch.equal(g2, r2)
    # and against the oracle, one head
    est = orc.estimate(d, b, pi, s, c, q[0, :4].double().cpu().numpy(),
                       P[:300].cpu().numpy().view(np.uint32),
                       N[:300].cpu().numpy().view(np.uint16), scale=0.5)
    assert rel_err_rows(g2[:4, :300].cpu().numpy(), est) < TOL
    ctx.close()


def test_noalloc_rejects_oversized_preparation(orc):
    d, b = 1536, 4
    pi, s, c = oracle_tables(orc, d, b)
    ctx = tq.TqContext(d, b, pi, s, c)
    batch, n_q, n_kv = 64, 8, 8          # about 63 MB of prepared queries
    assert tq.tq_attn_logits_workspace_bytes(ctx, batch, n_q, n_kv) > (4 << 20)
    P, N = workloads.random_records(16, tq.tq_record_words(d, b), 3, DEV)
    q = torch.zeros((batch, n_q, d), device=DEV)
    ss = torch.zeros(batch, dtype=torch.int64, device=DEV)
    sl = torch.full((batch,), 1, dtype=torch.int32, device=DEV)
    out = torch.empty((n_q, 16), device=DEV)
    with pytest.raises(tq.TqError) as ei:
        tq.tq_attn_logits_noalloc(ctx, q, batch, n_q, n_q * d, P, N, n_kv, 0, ss, sl, 1, 1.0,
                                  out, 16)
    assert "static scratch" in str(ei.value)
    ctx.close()
