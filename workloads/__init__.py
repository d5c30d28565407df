"""Seeded synthetic inputs for the five TurboQuant workloads.

Holds only input generation (no quantization arithmetic); both the tests and
``bench.py`` draw from here, so the HIP path and the oracle see the same data.
Every tensor is drawn with its own ``torch.Generator`` seeded by
``seed * 1000 + stream`` on the requested device (streams: K = 10, V = 11,
Q = 12, outlier channels = 13, ragged lengths = 14, database = 15,
search queries = 16, random records = 17).

Workloads (shapes from the benchmark configurations; the pages' own data --
Llama-3.1-8B KV caches, GloVe-200, OpenAI embeddings -- are not available, so
these stand in for them):
  tiny:     K [1024, 128] and Q [16, 128] fp32 N(0, 1); b = 3
  llama:    K, V [8, 32768, 128] bf16 N(0, 1) with 4 channels per KV head
            scaled by 10 (outliers); q [32, 128] fp32 N(0, 1); b = 4
  batched:  16 sequences, lengths uniform in [4096, 8192]; K, V as llama
            (bf16, outliers), a 512-token chunk per sequence; one query of
            32 heads per sequence; b = 3
  long:     K, V [8, 131072, 128] bf16 N(0, 1); q [32, 128]; b in {2, 3, 4}
  search:   database [1e6, d] and queries [1000, d] fp32 unit vectors
            (normalised N(0, I)), d in {1536, 200}; b in {2, 4}; k = 10
"""
import torch

STREAM_K, STREAM_V, STREAM_Q, STREAM_OUTLIER, STREAM_LEN = 10, 11, 12, 13, 14
STREAM_DB, STREAM_SQ, STREAM_REC = 15, 16, 17


def gen(seed, stream, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000 + int(stream))
    return g


def normal(shape, seed, stream, device, dtype=torch.float32):
    return torch.randn(shape, generator=gen(seed, stream, device), device=device,
                       dtype=torch.float32).to(dtype)


def kv_with_outliers(n_kv, n_tok, d, seed, stream, device, outliers=4, factor=10.0):
    """[n_kv, n_tok, d] bf16: N(0, 1), with `outliers` distinct channels per
    KV head multiplied by `factor` before rounding to bf16."""
    x = torch.randn((n_kv, n_tok, d), generator=gen(seed, stream, device), device=device)
    if outliers:
        go = gen(seed, STREAM_OUTLIER * 100 + stream, "cpu")
        for h in range(n_kv):
            ch = torch.randperm(d, generator=go)[:outliers].to(device)
            x[h, :, ch] *= factor
    return x.to(torch.bfloat16)


def unit_rows(n, d, seed, stream, device):
    x = torch.randn((n, d), generator=gen(seed, stream, device), device=device)
    return x / x.norm(dim=1, keepdim=True)


def tiny(device, seed=0):
    return {"d": 128, "b": 3,
            "K": normal((1024, 128), seed, STREAM_K, device),
            "Q": normal((16, 128), seed, STREAM_Q, device)}


def llama(device, seed=0, n_tok=32768, n_kv=8, n_q=32, d=128):
    return {"d": d, "b": 4, "n_kv": n_kv, "n_q": n_q,
            "K": kv_with_outliers(n_kv, n_tok, d, seed, STREAM_K, device),
            "V": kv_with_outliers(n_kv, n_tok, d, seed, STREAM_V, device),
            "q": normal((n_q, d), seed, STREAM_Q, device)}


def batched_lengths(seed=0, batch=16, lo=4096, hi=8192):
    g = gen(seed, STREAM_LEN, "cpu")
    return torch.randint(lo, hi + 1, (batch,), generator=g).tolist()


def batched(device, seed=0, batch=16, chunk=512, n_kv=8, n_q=32, d=128, lo=4096, hi=8192):
    lens = batched_lengths(seed, batch, lo, hi)
    total = sum(lens)
    return {"d": d, "b": 3, "n_kv": n_kv, "n_q": n_q, "lens": lens, "chunk": chunk,
            "K": kv_with_outliers(n_kv, total, d, seed, STREAM_K, device),
            "V": kv_with_outliers(n_kv, total, d, seed, STREAM_V, device),
            "q": normal((batch, n_q, d), seed, STREAM_Q, device)}


def long_context(device, seed=0, n_tok=131072, n_kv=8, n_q=32, d=128):
    return {"d": d, "n_kv": n_kv, "n_q": n_q,
            "K": kv_with_outliers(n_kv, n_tok, d, seed, STREAM_K, device, outliers=0),
            "V": kv_with_outliers(n_kv, n_tok, d, seed, STREAM_V, device, outliers=0),
            "q": normal((n_q, d), seed, STREAM_Q, device)}


def search(device, d, seed=0, n_db=1_000_000, n_q=1000):
    return {"d": d, "db": unit_rows(n_db, d, seed, STREAM_DB, device),
            "queries": unit_rows(n_q, d, seed, STREAM_SQ, device)}


def random_records(n, words, seed, device):
    """Arbitrary packed records (every bit pattern is a valid code) with fp16
    norms in [0.5, 2) (nu) and [0, 0.5) (gamma).  The caller clears the
    padding bits when d is not a multiple of 32.  Returns (planes int32
    [n, words], norms int16 [n, 2])."""
    g = gen(seed, STREAM_REC, device)
    planes = torch.randint(-2 ** 31, 2 ** 31, (n, words), generator=g, device=device,
                           dtype=torch.int64).to(torch.int32)
    nu = torch.rand((n,), generator=g, device=device) * 1.5 + 0.5
    ga = torch.rand((n,), generator=g, device=device) * 0.5
    norms = torch.stack([nu.half().view(torch.int16), ga.half().view(torch.int16)], dim=1)
    return planes, norms.contiguous()
