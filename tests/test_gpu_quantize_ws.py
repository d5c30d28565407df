"""GPU parity of the blocked large-d quantizer (tq_quantize_kv_ws): records
against the oracle (codes and signs bit-exact outside the oracle margins,
fp16 norms within one ulp), the same records as tq_quantize_kv outside those
margins, independence of the workspace size (chunking), destination
indexing, and its argument checks.  All inputs are seeded.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_vector_pi_amd as tq  # noqa: E402
import workloads  # noqa: E402
from helpers import check_records_mse, f16_ulp_diff, oracle_tables  # noqa: E402
from test_gpu_parity import check_quantize  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


_ctx = {}


def make_ctx(orc, d, b, mse):
    key = (d, b, mse)
    if key not in _ctx:
        if mse:
            pi = orc.make_rotation(d, 0)[2]
            c = orc.lloyd_max(d, b)[0].astype(np.float32)
            _ctx[key] = (tq.tq_ctx_create_mse(d, b, pi, c), pi, None, c)
        else:
            pi, s, c = oracle_tables(orc, d, b, 0)
            _ctx[key] = (tq.TqContext(d, b, pi, s, c), pi, s, c)
    return _ctx[key]


def ws_quantize(ctx, x, rows_ws=None, **kw):
    n = x.shape[0] * (x.shape[1] if x.dim() == 3 else 1)
    nb = tq.tq_quantize_workspace_bytes(ctx, n if rows_ws is None else rows_ws)
    ws = tq.workspace(nb) if nb else None
    P, N = tq.alloc_records(n, ctx.d, ctx.b)
    tq.tq_quantize_kv_ws(ctx, x, P, N, ws, **kw)
    return P, N


def np_rec(P, N):
    return P.cpu().numpy().view(np.uint32), N.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("d,b,mse,dtype,n", [
    (1536, 4, False, torch.float32, 300),     # 3 tiles, ragged
    (1536, 2, False, torch.bfloat16, 129),
    (1000, 3, False, torch.float32, 200),     # padded words (d < Dp)
    (512, 4, False, torch.bfloat16, 257),
    (768, 2, True, torch.float32, 130),       # MSE-only records
    (1536, 3, True, torch.bfloat16, 64),
])
def test_quantize_ws_parity(orc, d, b, mse, dtype, n):
    say("quantize ws", d, b, mse, dtype, n)
    ctx, pi, s, c = make_ctx(orc, d, b, mse)
    x = (workloads.normal((n, d), 41, 10, DEV) * 2.5).to(dtype)
    x[7] = 0                                       # a zero vector
    P, N = ws_quantize(ctx, x)
    torch.cuda.synchronize()
    xd = x.double().cpu().numpy()
    gp, gn = np_rec(P, N)
    if mse:
        check_records_mse(orc, d, b, pi, c, xd, gp, gn)
    else:
        check_quantize(orc, d, b, x.float(), pi, s, c, gp, gn)
    assert np.all(gn[7] == 0)
    # against the one-kernel quantizer: identical outside the decision margins
    P1, N1 = tq.alloc_records(n, d, b)
    tq.tq_quantize_kv(ctx, x, P1, N1)
    torch.cuda.synchronize()
    g1, n1 = np_rec(P1, N1)
    assert f16_ulp_diff(gn[:, 0], n1[:, 0]).max() <= 1
    diff_rows = np.any(gp != g1, axis=1)
    assert diff_rows.mean() < 0.05, diff_rows.mean()


def test_quantize_ws_chunking_and_indexing(orc):
    """A one-tile workspace (several chunks) gives the same records as a
    whole-input one; heads and tokens land at h*dst_stride_head + dst_token0
    + t, and neighbouring records are left alone."""
    d, b = 1536, 4
    ctx, pi, s, c = make_ctx(orc, d, b, False)
    n_heads, n_tok, cap, t0 = 3, 150, 170, 9
    x = workloads.normal((n_heads, n_tok, d), 42, 10, DEV)
    big = tq.workspace(tq.tq_quantize_workspace_bytes(ctx, n_heads * n_tok))
    small = tq.workspace(tq.tq_quantize_workspace_bytes(ctx, 1))
    outs = []
    for ws in (big, small):
        P, N = tq.alloc_records(n_heads * cap, d, b)
        P.fill_(0x5A5A5A5A)
        N.fill_(0x3C3C)
        tq.tq_quantize_kv_ws(ctx, x, P, N, ws, dst_stride_head=cap, dst_token0=t0)
        outs.append((P, N))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    P, N = outs[0]
    gp = P.cpu().numpy().view(np.uint32).reshape(n_heads, cap, -1)
    gn = N.cpu().numpy().view(np.uint16).reshape(n_heads, cap, 2)
    assert np.all(gp[:, :t0] == 0x5A5A5A5A) and np.all(gp[:, t0 + n_tok:] == 0x5A5A5A5A)
    assert np.all(gn[:, :t0] == 0x3C3C)
    rows = gp[:, t0:t0 + n_tok].reshape(n_heads * n_tok, -1)
    nrm = gn[:, t0:t0 + n_tok].reshape(n_heads * n_tok, 2)
    check_quantize(orc, d, b, x.reshape(-1, d), pi, s, c, rows, nrm)


def test_quantize_ws_arguments(orc):
    d, b = 1536, 2
    ctx, pi, s, c = make_ctx(orc, d, b, False)
    x = torch.zeros((4, d), device=DEV)
    P, N = tq.alloc_records(4, d, b)
    with pytest.raises(tq.TqError):            # d needs a workspace
        tq.tq_quantize_kv_ws(ctx, x, P, N, None)
    with pytest.raises(tq.TqError):            # smaller than one tile
        tq.tq_quantize_kv_ws(ctx, x, P, N, tq.workspace(1024))
    big = tq.workspace(tq.tq_quantize_workspace_bytes(ctx, 4) + 512)
    with pytest.raises(tq.TqError):            # not 256-byte aligned
        tq.tq_quantize_kv_ws(ctx, x, P, N, big[16:])
    # small d: the one-kernel path, no workspace needed
    ctx2, _, _, _ = make_ctx(orc, 128, 3, False)
    assert tq.tq_quantize_workspace_bytes(ctx2, 1000) == 0
    x2 = workloads.normal((10, 128), 43, 10, DEV)
    P2, N2 = tq.alloc_records(10, 128, 3)
    tq.tq_quantize_kv_ws(ctx2, x2, P2, N2, None)
    P3, N3 = tq.alloc_records(10, 128, 3)
    tq.tq_quantize_kv(ctx2, x2, P3, N3)
    torch.cuda.synchronize()
    assert torch.equal(P2, P3) and torch.equal(N2, N3)
