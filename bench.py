"""Benchmark of the TurboQuant hot path on one MI355X.

Workload: the Llama-3.1-8B-shaped decode layer (32 query heads, 8 KV heads,
head_dim 128, batch 1, 32768 cached tokens, bf16 K/V N(0, 1) with 4 outlier
channels per KV head scaled by 10, b = 4, logits for one new token).  One
step runs that layer's hot path for L = 32 independent layer caches (as in a
32-layer model, so the 704 MB of packed keys and logits per step are well
beyond the 256 MB Infinity Cache): quantize each layer's new-token K and V
into its packed cache, rotate/project each layer's 32 query heads, and stream
all cached keys of every layer into attention logits.  Each stage is one
launch covering all layers.

Outside the timed steps: a cache-fill leg times tq_quantize_kv on all K and V
of the 32 layers (quantize vectors/s), and the CPU oracle is timed on a
bounded sample of the same decode work (cpu_baseline).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
Prints one JSON line.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
N_KV, N_Q, D, B, N_TOK, LAYERS = 8, 32, 128, 4, 32768, 32


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--fill-reps", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run a plain device copy of this size (for scaling HBM "
                         "byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); the hot path has no multi-GPU leg in this build.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kv_cache_vector_pi_amd as tq
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    L = args.layers
    stream = torch.cuda.current_stream()

    # ---- set-up through the library's own host calls --------------------
    pi, s = tq.tq_make_rotation(D, 0)
    cent, _, _ = tq.tq_lloyd_max(D, B - 1)
    ctx = tq.TqContext(D, B, pi, s, cent)
    W = tq.tq_words_per_plane(D)
    rw = tq.tq_record_words(D, B)

    # caches laid out [kv head][layer][token]: record (h, l, t) at
    # h * (L * N_TOK) + l * N_TOK + t, so layer l is "sequence" l of one launch
    n_rec = N_KV * L * N_TOK
    k_planes = torch.zeros((n_rec, rw), dtype=torch.int32, device=dev)
    k_norms = torch.zeros((n_rec, 2), dtype=torch.int16, device=dev)
    v_planes = torch.zeros_like(k_planes)
    v_norms = torch.zeros_like(k_norms)
    # bf16 K/V of every layer, [kv head][layer * token][d]
    Kx = torch.empty((N_KV, L * N_TOK, D), dtype=torch.bfloat16, device=dev)
    Vx = torch.empty_like(Kx)
    for l in range(L):
        wl = workloads.llama(dev, seed=l, n_tok=N_TOK)
        Kx[:, l * N_TOK:(l + 1) * N_TOK] = wl["K"]
        Vx[:, l * N_TOK:(l + 1) * N_TOK] = wl["V"]
        del wl
    q_all = torch.stack([workloads.normal((N_Q, D), l, workloads.STREAM_Q, dev)
                         for l in range(L)])                     # [L][32][128]
    seq_start = torch.arange(L, dtype=torch.int64, device=dev) * N_TOK
    seq_len = torch.full((L,), N_TOK, dtype=torch.int32, device=dev)
    logits = torch.empty((N_Q, L * N_TOK), dtype=torch.float32, device=dev)
    ws = tq.workspace(tq.tq_attn_logits_workspace_bytes(ctx, L, N_Q, N_KV), dev)
    scale = 1.0 / math.sqrt(D)

    if args.copy_calibration_mb:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings give
        # the scale between those counters and bytes actually moved
        nb = args.copy_calibration_mb * (1 << 20)
        src = torch.empty(nb // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- cache-fill leg: quantize every K and V vector ---------------------
    def fill():
        tq.tq_quantize_kv(ctx, Kx, k_planes, k_norms)
        tq.tq_quantize_kv(ctx, Vx, v_planes, v_norms)

    fill()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.fill_reps)]
    for r in range(args.fill_reps):
        ev[2 * r].record(stream)
        fill()
        ev[2 * r + 1].record(stream)
    torch.cuda.synchronize()
    fill_ms = sum(ev[2 * r].elapsed_time(ev[2 * r + 1]) for r in range(args.fill_reps)) \
        / args.fill_reps
    n_fill = 2 * N_KV * L * N_TOK
    q_bytes_per_vec = 2 * D + (B * D // 8 + 4)        # bf16 in, packed record out
    quant_vps = n_fill / (fill_ms * 1e-3)
    quant_gbs = quant_vps * q_bytes_per_vec / 1e9

    # ---- decode step ---------------------------------------------------------
    # new-token K/V at cache position N_TOK - 1 of every layer
    newK = Kx.view(N_KV, L, N_TOK, D)[:, :, N_TOK - 1].contiguous()    # [8][L][128]
    newV = Vx.view(N_KV, L, N_TOK, D)[:, :, N_TOK - 1].contiguous()
    ev_a = torch.cuda.Event(enable_timing=True)
    ev_b = torch.cuda.Event(enable_timing=True)

    def step(times=None):
        # quantize the new token of each (kv head, layer): "head" = (h, l) pair
        tq.tq_quantize_kv(ctx, newK.view(N_KV * L, 1, D), k_planes, k_norms,
                          dst_stride_head=N_TOK, dst_token0=N_TOK - 1)
        tq.tq_quantize_kv(ctx, newV.view(N_KV * L, 1, D), v_planes, v_norms,
                          dst_stride_head=N_TOK, dst_token0=N_TOK - 1)
        tq.tq_attn_prepare(ctx, q_all, L, N_Q, N_Q * D, N_KV, ws)
        if times is not None:
            ev_a.record(stream)
        tq.tq_attn_logits_prepared(ctx, ws, L, N_Q, k_planes, k_norms, N_KV, L * N_TOK,
                                   seq_start, seq_len, N_TOK, scale, logits, L * N_TOK)
        if times is not None:
            ev_b.record(stream)
            ev_b.synchronize()
            times.append(ev_a.elapsed_time(ev_b))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # logit kernel alone, events on its stream (separate pass: the per-step
    # event synchronisation would otherwise sit inside the timed steps)
    ktimes = []
    for _ in range(max(10, min(args.steps, 50))):
        step(ktimes)
    torch.cuda.synchronize()
    k_ms = sorted(ktimes)[len(ktimes) // 2]
    k_mean_ms = sum(ktimes) / len(ktimes)

    logits_per_step = N_Q * L * N_TOK
    keys_per_step = N_KV * L * N_TOK
    rec_bytes = B * D // 8 + 4
    alg_bytes = keys_per_step * rec_bytes + logits_per_step * 4     # per launch
    achieved = alg_bytes / (k_mean_ms * 1e-3) / 1e9

    # ---- CPU oracle on a bounded sample of the same decode work -------------
    cpu = None
    if not args.no_cpu:
        import oracle
        _, _, opi, os_ = oracle.make_rotation(D, 0)
        oc = oracle.lloyd_max(D, B - 1)[0].astype(np.float32)
        n_tok_cpu = N_TOK
        P, Nn = workloads.random_records(N_KV * n_tok_cpu, rw, 99, "cpu")
        P = P.numpy().view(np.uint32)
        Nn = Nn.numpy().view(np.uint16)
        q0 = q_all[0].double().cpu().numpy()
        newk = newK[:, 0].double().cpu().numpy()
        done_logits, t_cpu = 0, 0.0
        while t_cpu < args.cpu_seconds or done_logits == 0:
            c0 = time.perf_counter()
            oracle.quantize(D, B, opi, os_, oc, newk)          # new token K (and V below)
            oracle.quantize(D, B, opi, os_, oc, newk)
            for h in range(N_KV):
                oracle.estimate(D, B, opi, os_, oc, q0[4 * h:4 * h + 4],
                                P[h * n_tok_cpu:(h + 1) * n_tok_cpu],
                                Nn[h * n_tok_cpu:(h + 1) * n_tok_cpu], scale=scale)
            t_cpu += time.perf_counter() - c0
            done_logits += N_Q * n_tok_cpu
        cpu = {"value": done_logits / t_cpu, "unit": "logits/s", "cores": oracle.num_threads(),
               "kind": "oracle",
               "sample": f"{done_logits // (N_Q * n_tok_cpu)} decode layer(s) of the same "
                         f"shape (32 q heads x 32768 keys, b=4, new-token K/V quantized), "
                         f"{t_cpu:.1f} s of fp64 oracle work"}

    out = {
        "metric": "packed-key attention logits/sec + HBM GB/s (% roofline); quantize vec/s",
        "value": logits_per_step / (ms_per_step * 1e-3),
        "unit": "logits/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8-mfma/fp32",
        "data": "synthetic (seeded; bf16 N(0,1) K/V with outlier channels)",
        "config": {"workload": "llama-3.1-8b decode layer: 32 q / 8 kv heads, d=128, batch 1, "
                               "32768 cached tokens, b=4, logits for 1 new token; 32 independent "
                               "layer caches per step",
                   "layers_per_step": L, "cached_tokens": N_TOK, "head_dim": D, "bits": B,
                   "q_heads": N_Q, "kv_heads": N_KV, "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "kernel": "attn_logits_kernel<4>",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "alg_bytes_per_launch": alg_bytes,
                     "kernel_ms_mean": k_mean_ms, "kernel_ms_median": k_ms},
        "logit_keys_per_s": keys_per_step / (k_mean_ms * 1e-3),
        "quantize": {"vec_per_s": quant_vps, "GB_per_s": quant_gbs,
                     "hbm_frac": quant_gbs / HBM_PEAK_GBS, "vectors_per_call": n_fill // 2,
                     "bytes_per_vector": q_bytes_per_vec, "ms_per_fill": fill_ms},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    ctx.close()


if __name__ == "__main__":
    main()
